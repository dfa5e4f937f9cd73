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
// Prefill variant: 256-row x 256-weight-row workgroup tiles, eight waves (two
// per SIMD) on the 32x32x64 scaled MFMA.
//
// Operands move global -> LDS with direct-to-LDS copies (no registers stage
// them) through a ring of three K-step slots, so two steps are in flight
// while one is computed.  A slot holds
//   * A codes, 32 KB: row-major, 128 bytes per row, with the 16-byte chunks
//     of row r XOR-swizzled by (r/2)%8.  One copy moves 8 whole rows (8
//     lanes per row, each 128-byte line read once) and the MFMA fragment
//     reads (32 rows x one chunk) hit every bank once per 16 lanes;
//   * B codes, 16 KB: the 16 packed 1 KB weight chunks (16 rows x 128 K);
//     the FP4 operand of 32 rows x 64 K is a per-lane gather over two chunks
//     that touches 16 consecutive bytes per lane group (conflict free);
//   * A scales, 2 KB: one dword (the step's four block scales) per row, in
//     eight 256-byte copies of 32 rows -- only when K is not a multiple of
//     512.  Otherwise the activation scales of four steps (16 bytes per row)
//     come once per group: waves 0-3 each copy 64 rows into 1 KB of the
//     (then unused) A-scale areas of slots 0 and 1, and every wave keeps its
//     rows' 16 bytes in registers for the group.
// The packed weight scales (one dword per lane covering four steps) go to
// two 4 KB slots, one per group of four steps.  Every wave issues its own
// share of the copies (4 A, 2 B, 1 A-scale per step, 2 B-scale per group)
// and waits on its own copies before the barrier that publishes a step.
//
// Wave w computes rows 64(w%4) .. +63 (two 32-row blocks) against 128 of
// the 256 weight rows: gate and up rows of the same 64 h columns for
// gate_up, 128 output columns for down.  Row blocks past the tile's end
// skip their MFMAs.
// ---------------------------------------------------------------------------

typedef float v16f __attribute__((ext_vector_type(16)));

// A: FP8 E4M3 with its scale in byte 0; B: FP4 E2M1 with its scale in byte SB
template <int SB>
__device__ __forceinline__ v16f mfma32_mx(const v8i& a, const v8i& b, v16f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, static_cast<int>(sa), SB,
                                                         static_cast<int>(sb));
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

constexpr int kPfSlot = 51200;                 // A 32 KB | B 16 KB | A scales 2 KB
constexpr int kPfA = 0, kPfB = 32768, kPfAS = 49152;
constexpr int kPfBS = 3 * kPfSlot;             // two 4 KB weight-scale slots
constexpr int kPfLds = kPfBS + 2 * 4096;       // 161792 bytes
// copies per wave per step: 4 A + 2 B (+1 A-scale dword when scales are not
// grouped); per group: 2 weight-scale dwords (+1 A-scale group copy, waves 0-3)
__shared__ __attribute__((aligned(1024))) uint8_t pf_lds[kPfLds];

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
// cut into 8 contiguous ranges, one per XCD (workgroups go to the XCDs
// round-robin by linear id).  Inside an expert the items run in groups of
// kPfGroupTiles tiles, column block next and tile fastest, so the workgroups
// an XCD runs at once cover a few tiles x several column blocks: every
// activation window and every weight window they read in the same K step is
// shared by several of them and comes from that XCD's L2.  Returns false for
// a workgroup with no item.
constexpr int kPfGroupTiles = 4;
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
  const int tg = local / (kPfGroupTiles * nblocks);           // tile group
  const int gsize = min(kPfGroupTiles, nt - tg * kPfGroupTiles);
  const int rem = local - tg * kPfGroupTiles * nblocks;
  *blk_out = rem / gsize;
  *tile_out = t0 + tg * kPfGroupTiles + rem % gsize;
  return true;
}

// LDS address of the A-scale group area written by wave w (0..3)
__device__ __forceinline__ int pf_asg_off(int w) { return (w >> 1) * kPfSlot + kPfAS + (w & 1) * 1024; }

template <bool GU, bool AG>
__global__ void __launch_bounds__(512, 1) k_gemm_pf(FwdArgs a) {
  constexpr int kCopies = AG ? 6 : 7;
  int tile_idx, nblk;
  if (!pf_work_item(a, GU ? a.dff / 128 : a.d / 256, &tile_idx, &nblk)) return;
  const Tile tile = a.tiles[tile_idx];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g32 = lane >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform copy of the wave index
  const int wm = wu & 3, wn = wu >> 2;
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

  // the tile's 16 weight-row blocks (16 rows each): gate then up (gate_up), or
  // 256 consecutive output rows (down)
  const int c0 = GU ? nblk * 128 : nblk * 256;
  auto wblk = [&](int j) -> int64_t {
    if (GU) return j < 8 ? (c0 + 16 * j) / 16 : (a.dff + c0 + 16 * (j - 8)) / 16;
    return (c0 + 16 * j) / 16;
  };
  // activation row r of the tile; padding rows read the tile's first row
  auto src_row = [&](int r) -> int64_t {
    int row = tile.row_begin + r;
    if (row >= tile.row_end) row = tile.row_begin;
    return GU ? (row < a.Rr ? a.row_token[row] : row - a.Rr - sidx * a.T) : row;
  };

  // ---- copy sources of this wave: rows 32wu .. 32wu+31, weight blocks 2wu, 2wu+1.
  // A copy q covers rows 32wu + 8q .. +7: lane l reads chunk (l%8) ^ swz(row)
  // of row 32wu + 8q + l/8 and lands at LDS row*128 + 16(l%8).
  const uint8_t* a_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rl = 32 * wu + 8 * q + (lane >> 3);
    a_src[q] = (GU ? a.x_codes : a.h_codes) + src_row(rl) * K + 16 * ((lane & 7) ^ ((rl >> 1) & 7));
  }
  const uint8_t* as_src = (GU ? a.x_scales : a.h_scales) + src_row(AG ? (64 * wu + lane) & 255 : 32 * wu + l32) * (K / 32);
  const uint8_t* b_src[2];
  const uint8_t* bs_src[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    b_src[jj] = wc + wblk(2 * wu + jj) * nsteps * 1024 + 16 * lane;
    bs_src[jj] = ws + wblk(2 * wu + jj) * nq4 * 256 + 4 * lane;
  }
  const uint32_t lds0 = lds_addr(pf_lds);

  // copies of step st into slot st % 3 (and of the weight scales of group
  // st / 4 when st starts a group)
  auto issue = [&](int st, bool group_start) {
    const uint32_t slot = lds0 + (st % 3) * kPfSlot;
#pragma unroll
    for (int q = 0; q < 4; ++q) lds_copy16(a_src[q] + 128 * st, slot + kPfA + (32 * wu + 8 * q) * 128);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) lds_copy16(b_src[jj] + st * 1024, slot + kPfB + (2 * wu + jj) * 1024);
    if (!AG) lds_copy4(as_src + 4 * st, slot + kPfAS + wu * 256);
    if (group_start) {
      if (AG && wu < 4) lds_copy16(as_src + 16 * (st >> 2), lds0 + pf_asg_off(wu));
      const int q = st >> 2;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        lds_copy4(bs_src[jj] + q * 256, lds0 + kPfBS + (q & 1) * 4096 + (2 * wu + jj) * 256);
    }
  };

  // ---- per-lane LDS read offsets
  // weight fragment p (32 rows) starts at chunk j0(p) of the tile's 16
  auto j0 = [&](int p) -> int { return GU ? (p < 2 ? 4 * wn + 2 * p : 8 + 4 * wn + 2 * (p - 2)) : 8 * wn + 2 * p; };
  const int b_lane = ((l32 >> 4) << 10) + 16 * (16 * g32 + (lane & 15));  // + j0*1024 + 512h
  // A fragment (row l32 of a 32-row block, K half h, piece c): chunk 4h+2c+g32
  int a_lane[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) a_lane[h][c] = l32 * 128 + 16 * ((4 * h + 2 * c + g32) ^ ((l32 >> 1) & 7));
  const int bs_lane = ((l32 >> 4) << 8) + 4 * (16 * g32 + (lane & 15));   // + j0*256 + 128h
  const int rows_left = tile.row_end - tile.row_begin - 64 * wm;
  const int nact = rows_left <= 0 ? 0 : (rows_left <= 32 ? 1 : 2);   // active row blocks

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[i][p] = v16f{};

  auto main_loop = [&](auto nact_c) {
    constexpr int NACT = decltype(nact_c)::value;
    uint32_t bsr[4][2];  // weight scale dwords of the current group
    uint4 asg[2];        // grouped activation scales of this lane's rows

    auto compute = [&](int st, auto ic) {
      constexpr int I = decltype(ic)::value;  // st % 4
      if (NACT == 0) return;
      const uint8_t* sb = pf_lds + (st % 3) * kPfSlot;
      if (I == 0) {
        const uint8_t* bsb = pf_lds + kPfBS + ((st >> 2) & 1) * 4096 + bs_lane;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            bsr[pp][h] = *reinterpret_cast<const uint32_t*>(bsb + j0(pp) * 256 + 128 * h);
        if (AG) {
#pragma unroll
          for (int i = 0; i < NACT; ++i)
            asg[i] = *reinterpret_cast<const uint4*>(pf_lds + pf_asg_off(wm) + (32 * i + l32) * 16);
        }
      }
      uint32_t asr[2];
      v8i av[2][2];
      v8i bv[2][4];
#pragma unroll
      for (int i = 0; i < NACT; ++i) {
        if (AG) asr[i] = I == 0 ? asg[i].x : I == 1 ? asg[i].y : I == 2 ? asg[i].z : asg[i].w;
        else asr[i] = *reinterpret_cast<const uint32_t*>(sb + kPfAS + (2 * wm + i) * 256 + 4 * l32);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < NACT; ++i) {
          const uint8_t* pa = sb + kPfA + (2 * wm + i) * 4096;
          av[h][i] = make_a(ld16(pa + a_lane[h][0]), ld16(pa + a_lane[h][1]));
        }
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) bv[h][pp] = make_b(ld16(sb + kPfB + j0(pp) * 1024 + 512 * h + b_lane));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < NACT; ++i) {
          const uint32_t sa = asr[i] >> (8 * (2 * h + g32));
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) acc[i][pp] = mfma32_mx<I>(av[h][i], bv[h][pp], acc[i][pp], sa, bsr[pp][h]);
        }
    };

    // step st: wait for this wave's copies of st (the next step's may stay
    // in flight), publish with a barrier, refill the slot of step st-1 with
    // step st+2, then compute
    auto stage = [&](int st, auto ic) {
      constexpr int I = decltype(ic)::value;
      if (st + 1 < nsteps) {
        if (((I + 1) & 3) == 0) {
          if (AG && wu < 4) PF_WAIT_VM(kCopies + 3);
          else PF_WAIT_VM(kCopies + 2);
        } else {
          PF_WAIT_VM(kCopies);
        }
      } else {
        PF_WAIT_VM(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (st + 2 < nsteps) issue(st + 2, ((I + 2) & 3) == 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(st, ic);
      __builtin_amdgcn_sched_barrier(0);
    };

    issue(0, true);
    if (1 < nsteps) issue(1, false);
    for (int st0 = 0; st0 < nsteps; st0 += 4) {
      stage(st0, IntC<0>{});
      if (st0 + 1 < nsteps) stage(st0 + 1, IntC<1>{});
      if (st0 + 2 < nsteps) stage(st0 + 2, IntC<2>{});
      if (st0 + 3 < nsteps) stage(st0 + 3, IntC<3>{});
    }
  };
  if (nact == 2) main_loop(IntC<2>{});
  else if (nact == 1) main_loop(IntC<1>{});
  else main_loop(IntC<0>{});

  // ---- epilogue through LDS: every wave is past its last operand read
  // after this barrier, and each wave then owns a private stage region.
  // acc[i][p] register r holds tile row 64wm + 32i + 8(r/4) + 4 g32 + r%4
  // and column l32 of weight fragment p.
  __syncthreads();
  if (nact == 0) return;
  if (GU) {
    // h = silu(gate) * up as fp32 [64 rows][64 h columns] (row stride 68)
    float* hs = reinterpret_cast<float*>(pf_lds) + wu * (64 * 68);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nact) break;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * i + 8 * (r / 4) + 4 * g32 + (r % 4);
          const float gt = acc[i][pp][r], up = acc[i][pp + 2][r];
          hs[rl * 68 + 32 * pp + l32] = gt / (1.0f + __expf(-gt)) * up;
          if (a.gu_acc) {
            const int row = tile.row_begin + 64 * wm + rl;
            if (row < tile.row_end) {
              const int col = c0 + 64 * wn + 32 * pp + l32;
              a.gu_acc[int64_t(row) * 2 * a.dff + col] = gt;
              a.gu_acc[int64_t(row) * 2 * a.dff + a.dff + col] = up;
            }
          }
        }
    }
    // lane l quantises row l: two MXFP8 blocks of 32 h values
    const int row = tile.row_begin + 64 * wm + lane;
    if (row < tile.row_end) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float4* src = reinterpret_cast<const float4*>(hs + lane * 68 + 32 * blk);
        float v[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 t = src[q];
          v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; ++q) amax = fmaxf(amax, fabsf(v[q]));
        const int e = mx8_block_exp(amax);
        const float sc = exp2_int(-e);
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = e4m3_cvt4(v[4 * q] * sc, v[4 * q + 1] * sc, v[4 * q + 2] * sc, v[4 * q + 3] * sc);
        const int col = c0 + 64 * wn + 32 * blk;
        uint4* dst = reinterpret_cast<uint4*>(a.h_codes + int64_t(row) * a.dff + col);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        a.h_scales[int64_t(row) * (a.dff / 32) + (col >> 5)] = static_cast<uint8_t>(e + 127);
      }
    }
  } else {
    // bf16 outputs [64 rows][128 columns] (row stride 136 halves), then
    // 16-byte row chunks: 16 per row, 1024 per wave, 16 per lane
    uint16_t* os = reinterpret_cast<uint16_t*>(pf_lds) + wu * (64 * 136);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (i >= nact) break;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = 32 * i + 8 * (r / 4) + 4 * g32 + (r % 4);
          os[rl * 136 + 32 * pp + l32] = f32_to_bf16_rne(acc[i][pp][r]);
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ch = q * 64 + lane;          // chunk: row ch / 16, 8 columns at 8 (ch % 16)
      const int rl = ch >> 4, cc = 8 * (ch & 15);
      const int row = tile.row_begin + 64 * wm + rl;
      if (row < tile.row_end) {
        const uint4 t = *reinterpret_cast<const uint4*>(os + rl * 136 + cc);
        *reinterpret_cast<uint4*>(a.o16 + int64_t(row) * a.d + c0 + 128 * wn + cc) = t;
      }
    }
  }
}

template <bool GU>
static hipError_t launch_pf(const FwdArgs& a, hipStream_t st) {
  const int64_t N = GU ? a.dff / 128 : a.d / 256;
  const int64_t items = int64_t(a.max_tiles) * N;
  const int K = GU ? a.d : a.dff;
  const dim3 grid(8 * ((items + 7) / 8));
  if (K % 512 == 0)
    hipLaunchKernelGGL((k_gemm_pf<GU, true>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm_pf<GU, false>), grid, dim3(512), 0, st, a);
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
