// Grouped expert GEMMs on the gfx950 scaled MFMA (MXFP8 activations x MXFP4
// weights, fp32 accumulate): gate_up with a fused SwiGLU + MXFP8 re-quantise
// epilogue, and down.  "Kimi K3 Tech Intro", section 4.3 names the routed +
// shared experts and the A8W4 fused operators on MI355X; SwiGLU stands in for
// the SiTU activation the pages name without defining.
//
// Operand layout of V_MFMA_SCALE_F32_16X16X128_F8F6F4 (established by probes
// in the exact-arithmetic regime):
//   * an FP4 operand lane (row r = lane%16, group g = lane/16) holds 32
//     consecutive logical k = 32g .. 32g+31 (16 bytes, element 2i in the low
//     nibble of byte i);
//   * an FP8 operand lane holds bytes j = 0..31 at logical k = 64(j/16) + 16g
//     + j%16, i.e. two 16-byte halves from logical blocks g/2 and 2 + g/2;
//   * the scale byte of lane (r, g) applies to logical block g (k = 32g..32g+31)
//     of row r; the result of lane l, register i is D[4(l/16)+i][l%16].
// MFMA step s covers K = 128s .. 128s+127 in natural order.  Weights arrive
// packed (moe_pack_mx4): the FP4 operand of one 16-row block and step is 1 KB
// contiguous in lane order, and the block scales of four steps one dword per
// lane (byte j for step 4q + j).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mx_device.h"

namespace mxmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, v4f c, uint32_t sa, uint32_t sb) {
  // A: FP8 E4M3 (format 0), B: FP4 E2M1 (format 4); scale in byte 0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Raw buffer access (offsets in bytes): an offset past num_records reads as
// zero without touching memory, which gives padding rows for free.
constexpr uint32_t kBufOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ uint32_t buf4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ v8i make_a(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}
__device__ __forceinline__ v8i make_b(uint4 v) {
  v8i r;
  r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// ---------------------------------------------------------------------------
// Decode variant: 16-row tiles (a few tokens per expert), weight-streaming.
// Each wave owns 16*NI output columns (gate and up subtiles for gate_up) over
// a contiguous share of K; the KS waves of a workgroup split K and reduce
// through LDS in a fixed order.  K is walked in groups of GS MFMA steps; the
// loads of the next group are issued before the MFMAs of the current one, so
// a whole group of weight bytes per wave stays in flight.  Padding rows of the
// tile read as zero through out-of-range buffer loads (no memory traffic).
// ---------------------------------------------------------------------------

template <int NB, int GS>
struct DecFrag {
  uint4 b[NB][GS];
  uint4 a[GS][2];
  uint32_t sa[GS];
  uint32_t sb[NB];
  uint32_t bsh;  // byte offset of this group's first step inside the scale dword
};

template <int NI, int KS, int GS, bool GU>
__global__ void __launch_bounds__(64 * KS) k_gemm_dec(FwdArgs a) {
  constexpr int NB = GU ? 2 * NI : NI;
  const int tile_idx = blockIdx.x;
  if (tile_idx >= *a.tile_count) return;
  const Tile tile = a.tiles[tile_idx];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = GU ? a.d : a.dff;
  const int N = GU ? a.dff : a.d;
  const int nsteps = K / 128, nq4 = (K + 511) / 512;
  const int col0 = blockIdx.y * (16 * NI);

  const bool shared = tile.ex >= a.E;
  const int sidx = tile.ex - a.E;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + tile.ex * wc_stride)
                         : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + tile.ex * wc_stride);
  const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + tile.ex * ws_stride)
                         : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + tile.ex * ws_stride);

  const int arow = tile.row_begin + r16;
  const bool avalid = arow < tile.row_end;
  uint32_t src = 0;
  if (avalid) src = GU ? (arow < a.Rr ? a.row_token[arow] : arow - a.Rr - sidx * a.T) : arow;
  const uint32_t a_rows = GU ? a.T : a.R;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(GU ? a.x_codes : a.h_codes, a_rows * uint32_t(K));
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(GU ? a.x_scales : a.h_scales, a_rows * uint32_t(K / 32));
  const uint32_t a_base = avalid ? src * uint32_t(K) + 16 * g : kBufOOB;
  const uint32_t as_base = avalid ? src * uint32_t(K / 32) : kBufOOB;
  const uint8_t* bp[NB];
  const uint8_t* bsp[NB];
#pragma unroll
  for (int nj = 0; nj < NB; ++nj) {
    const int n = col0 + 16 * (nj % NI);
    const int64_t blk = ((GU && nj >= NI) ? a.dff + n : n) / 16;
    bp[nj] = wc + blk * nsteps * 1024 + 16 * lane;
    bsp[nj] = ws + blk * nq4 * 256 + 4 * lane;
  }

  // K groups of this wave: a contiguous range
  const int nq = nsteps / GS;
  const int q0 = (nq * wave) / KS, q1 = (nq * (wave + 1)) / KS;
  const int n = q1 - q0;

  auto load = [&](DecFrag<NB, GS>& f, int q) {
    const int st0 = q * GS;
    f.bsh = 8 * (st0 & 3);
#pragma unroll
    for (int nj = 0; nj < NB; ++nj) {
      f.sb[nj] = *reinterpret_cast<const uint32_t*>(bsp[nj] + (st0 >> 2) * 256);
#pragma unroll
      for (int s = 0; s < GS; ++s) f.b[nj][s] = ld16(bp[nj] + (st0 + s) * 1024);
    }
#pragma unroll
    for (int s = 0; s < GS; ++s) {
      // scale bytes 4*step .. 4*step+3 of the row; lane group g uses byte g
      f.sa[s] = buf4(ras, as_base + 4 * (st0 + s));
      f.a[s][0] = buf16(ra, a_base + 128 * (st0 + s));
      f.a[s][1] = buf16(ra, a_base + 128 * (st0 + s) + 64);
    }
  };
  v4f acc[NB];
#pragma unroll
  for (int nj = 0; nj < NB; ++nj) acc[nj] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const DecFrag<NB, GS>& f) {
#pragma unroll
    for (int s = 0; s < GS; ++s) {
      const v8i av = make_a(f.a[s][0], f.a[s][1]);
      const uint32_t sa = f.sa[s] >> (8 * g);
#pragma unroll
      for (int nj = 0; nj < NB; ++nj)
        acc[nj] = mfma_mx(av, make_b(f.b[nj][s]), acc[nj], sa, f.sb[nj] >> (f.bsh + 8 * s));
    }
  };

  DecFrag<NB, GS> f0, f1;
  if (n > 0) {
    load(f0, q0);
    int i = 0;
    for (; i + 2 < n; i += 2) {  // f0 holds group q0 + i
      load(f1, q0 + i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(f0);
      __builtin_amdgcn_sched_barrier(0);
      load(f0, q0 + i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (n - i == 2) {
      load(f1, q0 + i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(f0);
      __builtin_amdgcn_sched_barrier(0);
      compute(f1);
    } else {
      compute(f0);
    }
  }

  // split-K reduction in wave order (deterministic)
  if (KS > 1) {
    __shared__ v4f red[KS > 1 ? (KS - 1) * NB * 64 : 1];
    if (wave > 0) {
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) red[((wave - 1) * NB + nj) * 64 + lane] = acc[nj];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < KS; ++w)
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) acc[nj] += red[((w - 1) * NB + nj) * 64 + lane];
  }

  // epilogue (wave 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tile.row_begin + 4 * g + i;
    const bool valid = row < tile.row_end;
    if (GU) {
#pragma unroll
      for (int p = 0; p < NI / 2; ++p) {
        float h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int j = 2 * p + hh;
          const float gt = acc[j][i], up = acc[NI + j][i];
          h[hh] = gt / (1.0f + expf(-gt)) * up;
          if (valid && a.gu_acc) {
            const int col = col0 + 16 * j + r16;
            a.gu_acc[int64_t(row) * 2 * a.dff + col] = gt;
            a.gu_acc[int64_t(row) * 2 * a.dff + a.dff + col] = up;
          }
        }
        const float amax = group_max<16>(fmaxf(fabsf(h[0]), fabsf(h[1])));
        const int e = mx8_block_exp(amax);
        if (valid) {
          const int col = col0 + 32 * p + r16;
          uint8_t* hc = a.h_codes + int64_t(row) * a.dff;
          hc[col] = static_cast<uint8_t>(mx8_encode(h[0], e));
          hc[col + 16] = static_cast<uint8_t>(mx8_encode(h[1], e));
          if (r16 == 0) a.h_scales[int64_t(row) * (a.dff / 32) + (col0 + 32 * p) / 32] = static_cast<uint8_t>(e + 127);
        }
      }
    } else if (valid) {
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) a.o[int64_t(row) * N + col0 + 16 * nj + r16] = acc[nj][i];
    }
  }
}

template <int NI, int KS, bool GU>
static hipError_t launch_dec(const FwdArgs& a, hipStream_t st) {
  const int K = GU ? a.d : a.dff;
  const int N = GU ? a.dff : a.d;
  dim3 grid(a.max_tiles, N / (16 * NI));
  if (K % 256 == 0)
    hipLaunchKernelGGL((k_gemm_dec<NI, KS, 2, GU>), grid, dim3(64 * KS), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_dec<NI, KS, 1, GU>), grid, dim3(64 * KS), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill variant: 128-row x 256-weight-row workgroup tiles, MFMA-bound.
// Operands move global -> LDS with direct-to-LDS loads placed in MFMA lane
// order (each 1 KB copy is one A half-operand of a 16-row subtile or one
// packed 16-row weight step), so every LDS read is one conflict-free read per
// lane and no registers stage the copies.  The block scales travel the same
// way (4 bytes per A row, the packed scale dword per weight block and lane).
// Four LDS stages of one 128-wide K step each keep three steps in flight;
// each wave issues 13 copies per stage and waits on its own copies before the
// barrier that publishes the stage.  Wave w computes rows 32w .. 32w+31
// against all 256 weight rows; a wave whose rows are all past the tile's end
// skips its MFMAs.
// ---------------------------------------------------------------------------

// stage slot: A codes 16 KB | B codes 16 KB | A scales 4 x 256 B | B scales 16 x 256 B
constexpr int kPfA = 0, kPfB = 16384, kPfAS = 32768, kPfBS = 33792, kPfStageBytes = 37888;
constexpr int kPfCopies = 13;  // per wave per stage: 4 A + 4 B + 1 A-scale + 4 B-scale
__shared__ __attribute__((aligned(1024))) uint8_t pf_s0[kPfStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t pf_s1[kPfStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t pf_s2[kPfStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t pf_s3[kPfStageBytes];

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct-to-LDS copy of 16 (or 4) bytes per lane to LDS byte address
// lds + lane*16 (lane*4).  Issued as inline assembly so that the compiler's
// wait insertion does not guard later LDS reads against it: the kernel waits
// for its own copies with explicit counts.  M0 holds the LDS base; one wait
// state separates its write from the copy.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)p));
}

// s_waitcnt with vmcnt = n, lgkmcnt and expcnt left unconstrained
#define PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))

// Work order of the prefill GEMMs: items (tile, column block) expert-major,
// column block next, tile fastest, cut into 8 contiguous ranges, one per XCD
// (workgroups go to the XCDs round-robin by linear id).  An expert's tiles
// and column blocks then run on one XCD close together in time, so its
// activation rows and each weight block come from that XCD's L2 after the
// first touch.  Returns false for a workgroup with no item.
__device__ __forceinline__ bool pf_work_item(const FwdArgs& a, int nblocks, int* tile_out, int* blk_out) {
  const int total = *a.tile_count * nblocks;
  const int per_xcd = (total + 7) / 8;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int w = xcd * per_xcd + i;
  if (i >= per_xcd || w >= total) return false;
  // expert e: the last with ex_tiles[e] <= w / nblocks
  const int q = w / nblocks;
  int lo = 0, hi = a.E + a.S;  // ex_tiles[lo] <= q < ex_tiles[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.ex_tiles[mid] <= q) lo = mid; else hi = mid;
  }
  const int t0 = a.ex_tiles[lo], nt = a.ex_tiles[lo + 1] - t0;
  const int local = w - t0 * nblocks;
  *blk_out = local / nt;
  *tile_out = t0 + local % nt;
  return true;
}

template <bool GU>
__global__ void __launch_bounds__(256, 1) k_gemm_pf(FwdArgs a) {
  int tile_idx, nblk;
  if (!pf_work_item(a, GU ? a.dff / 128 : a.d / 256, &tile_idx, &nblk)) return;
  const Tile tile = a.tiles[tile_idx];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = GU ? a.d : a.dff;
  const int nsteps = K / 128, nq4 = (K + 511) / 512;

  const bool shared = tile.ex >= a.E;
  const int sidx = tile.ex - a.E;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + tile.ex * wc_stride)
                         : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + tile.ex * wc_stride);
  const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + tile.ex * ws_stride)
                         : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + tile.ex * ws_stride);

  // 16 weight-row blocks of this tile: gate then up (gate_up) or 256 outputs (down)
  const int c0 = GU ? nblk * 128 : nblk * 256;
  auto wblk = [&](int j) -> int64_t {
    if (GU) return j < 8 ? (c0 + 16 * j) / 16 : (a.dff + c0 + 16 * (j - 8)) / 16;
    return (c0 + 16 * j) / 16;
  };
  // activation row of this wave's row slot q (0..31); padding rows read row_begin
  auto src_row = [&](int q) -> int64_t {
    int row = tile.row_begin + 32 * wave + q;
    if (row >= tile.row_end) row = tile.row_begin;
    return GU ? (row < a.Rr ? a.row_token[row] : row - a.Rr - sidx * a.T) : row;
  };

  // copy sources of this wave: its A subtiles 2w, 2w+1, weight blocks 4w..4w+3
  const uint8_t* a_src[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) a_src[ms] = (GU ? a.x_codes : a.h_codes) + src_row(16 * ms + r16) * K + 16 * g;
  const uint8_t* as_src = (GU ? a.x_scales : a.h_scales) + src_row(lane & 31) * (K / 32);
  const uint8_t* b_src[4];
  const uint8_t* bs_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b_src[j] = wc + wblk(4 * wave + j) * nsteps * 1024 + 16 * lane;
    bs_src[j] = ws + wblk(4 * wave + j) * nq4 * 256 + 4 * lane;
  }

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform for M0
  auto issue = [&](int st, uint8_t* buf) {
    const uint32_t base = lds_addr(buf);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        lds_copy16(a_src[ms] + 128 * st + 64 * h, base + kPfA + ((2 * wave_u + ms) * 2 + h) * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy16(b_src[j] + st * 1024, base + kPfB + (4 * wave_u + j) * 1024);
    // scale bytes 4st .. 4st+3 of this wave's 32 rows (lanes 32..63 repeat 0..31)
    lds_copy4(as_src + 4 * st, base + kPfAS + wave_u * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_copy4(bs_src[j] + (st >> 2) * 256, base + kPfBS + (4 * wave_u + j) * 256);
  };

  const bool active = tile.row_begin + 32 * wave < tile.row_end;
  v4f acc[2][16];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[ms][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const uint8_t* buf) {
    if (!active) return;
    v8i av[2];
    uint32_t sa[2];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const uint8_t* p = buf + kPfA + (2 * wave + ms) * 2048 + 16 * lane;
      av[ms] = make_a(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 1024));
      sa[ms] = *reinterpret_cast<const uint32_t*>(buf + kPfAS + wave * 256 + (16 * ms + r16) * 4) >> (8 * g);
    }
    const int bsh = 8 * (st & 3);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const v8i bv = make_b(*reinterpret_cast<const uint4*>(buf + kPfB + j * 1024 + 16 * lane));
      const uint32_t sb = *reinterpret_cast<const uint32_t*>(buf + kPfBS + j * 256 + 4 * lane) >> bsh;
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) acc[ms][j] = mfma_mx(av[ms], bv, acc[ms][j], sa[ms], sb);
    }
  };

  // stage st: wait for this wave's copies of st (later stages may stay in
  // flight), publish with a barrier, refill the slot stage st-1 used with
  // stage st+3, then compute.
  auto stage = [&](int st, const uint8_t* cur, uint8_t* nxt) {
    const int later = nsteps - 1 - st;  // stages issued after st: min(later, 2)
    if (later >= 2) PF_WAIT_VM(2 * kPfCopies);
    else if (later == 1) PF_WAIT_VM(kPfCopies);
    else PF_WAIT_VM(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (st + 3 < nsteps) issue(st + 3, nxt);
    __builtin_amdgcn_sched_barrier(0);
    compute(st, cur);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, pf_s0);
  if (1 < nsteps) issue(1, pf_s1);
  if (2 < nsteps) issue(2, pf_s2);
  for (int st0 = 0; st0 < nsteps; st0 += 4) {
    stage(st0, pf_s0, pf_s3);
    if (st0 + 1 < nsteps) stage(st0 + 1, pf_s1, pf_s0);
    if (st0 + 2 < nsteps) stage(st0 + 2, pf_s2, pf_s1);
    if (st0 + 3 < nsteps) stage(st0 + 3, pf_s3, pf_s2);
  }
  if (!active) return;

  // epilogue: rows 32w + 16ms + 4g + i
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile.row_begin + 32 * wave + 16 * ms + 4 * g + i;
      const bool valid = row < tile.row_end;
      if (GU) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int j = 2 * p + hh;
            const float gt = acc[ms][j][i], up = acc[ms][8 + j][i];
            h[hh] = gt / (1.0f + expf(-gt)) * up;
            if (valid && a.gu_acc) {
              const int col = c0 + 16 * j + r16;
              a.gu_acc[int64_t(row) * 2 * a.dff + col] = gt;
              a.gu_acc[int64_t(row) * 2 * a.dff + a.dff + col] = up;
            }
          }
          const float amax = group_max<16>(fmaxf(fabsf(h[0]), fabsf(h[1])));
          const int e = mx8_block_exp(amax);
          if (valid) {
            const int col = c0 + 32 * p + r16;
            uint8_t* hc = a.h_codes + int64_t(row) * a.dff;
            hc[col] = static_cast<uint8_t>(mx8_encode(h[0], e));
            hc[col + 16] = static_cast<uint8_t>(mx8_encode(h[1], e));
            if (r16 == 0) a.h_scales[int64_t(row) * (a.dff / 32) + (c0 + 32 * p) / 32] = static_cast<uint8_t>(e + 127);
          }
        }
      } else if (valid) {
        uint16_t* orow = a.o16 + int64_t(row) * a.d + c0 + r16;
#pragma unroll
        for (int j = 0; j < 16; ++j) orow[16 * j] = f32_to_bf16_rne(acc[ms][j][i]);
      }
    }
  }
}

template <bool GU>
static hipError_t launch_pf(const FwdArgs& a, hipStream_t st) {
  const int64_t N = GU ? a.dff / 128 : a.d / 256;
  const int64_t items = int64_t(a.max_tiles) * N;
  hipLaunchKernelGGL((k_gemm_pf<GU>), dim3(8 * ((items + 7) / 8)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const FwdArgs& a, hipStream_t st) {
  if (a.bm == 16) return launch_dec<2, 2, true>(a, st);
  return launch_pf<true>(a, st);
}

hipError_t launch_gemm_down(const FwdArgs& a, hipStream_t st) {
  if (a.bm == 16) return launch_dec<2, 1, false>(a, st);
  return launch_pf<false>(a, st);
}

}  // namespace mxmoe
