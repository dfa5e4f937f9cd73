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

// MI: 16-row M subtiles per wave; NI: 16-column N subtiles per wave (h columns
// for gate_up, each needing a gate and an up subtile); NW: waves per workgroup
// along N; G4: K handled in groups of 512 (4 MFMA steps sharing a scale dword),
// else one 128-wide step at a time.
template <int MI, int NI, int NW, bool GU>
__global__ void __launch_bounds__(64 * NW) k_gemm(FwdArgs a) {
  constexpr int NB = GU ? 2 * NI : NI;
  const int tile_idx = blockIdx.x;
  if (tile_idx >= *a.tile_count) return;
  const Tile tile = a.tiles[tile_idx];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = GU ? a.d : a.dff;
  const int N = GU ? a.dff : a.d;
  const int nsteps = K / 128, nq4 = (K + 511) / 512;
  const int col0 = blockIdx.y * (16 * NI * NW) + wave * (16 * NI);

  // packed weights of this expert
  const bool shared = tile.ex >= a.E;
  const int sidx = tile.ex - a.E;
  const int64_t wrows = GU ? 2 * a.dff : a.d;
  const int64_t wc_stride = wrows * (K / 2), ws_stride = packed_scale_bytes(wrows, K);
  const uint8_t* wc = GU ? (shared ? a.sgu_c + sidx * wc_stride : a.gu_c + tile.ex * wc_stride)
                         : (shared ? a.sdn_c + sidx * wc_stride : a.dn_c + tile.ex * wc_stride);
  const uint8_t* ws = GU ? (shared ? a.sgu_s + sidx * ws_stride : a.gu_s + tile.ex * ws_stride)
                         : (shared ? a.sdn_s + sidx * ws_stride : a.dn_s + tile.ex * ws_stride);

  // activation rows (clamped to a valid row for padding lanes)
  const uint8_t* ap[MI];
  const uint8_t* asp[MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    int row = tile.row_begin + 16 * mi + r16;
    if (row >= tile.row_end) row = tile.row_begin;
    int64_t src;
    if (GU)
      src = row < a.Rr ? a.row_token[row] : row - a.Rr - sidx * a.T;
    else
      src = row;
    ap[mi] = (GU ? a.x_codes : a.h_codes) + src * K + 16 * g;
    asp[mi] = (GU ? a.x_scales : a.h_scales) + src * (K / 32) + g;
  }
  const uint8_t* bp[NB];
  const uint8_t* bsp[NB];
#pragma unroll
  for (int nj = 0; nj < NB; ++nj) {
    const int n = col0 + 16 * (nj % NI);
    const int64_t blk = ((GU && nj >= NI) ? a.dff + n : n) / 16;
    bp[nj] = wc + blk * nsteps * 1024 + 16 * lane;
    bsp[nj] = ws + blk * nq4 * 256 + 4 * lane;
  }

  v4f acc[MI][NB];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB; ++nj) acc[mi][nj] = v4f{0.f, 0.f, 0.f, 0.f};

  uint32_t sb[NB];
  for (int st = 0; st < nsteps; ++st) {
    if ((st & 3) == 0) {
#pragma unroll
      for (int nj = 0; nj < NB; ++nj) sb[nj] = *reinterpret_cast<const uint32_t*>(bsp[nj] + (st >> 2) * 256);
    }
    v8i av[MI], bv[NB];
    uint32_t sa[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      av[mi] = make_a(ld16(ap[mi] + 128 * st), ld16(ap[mi] + 128 * st + 64));
      sa[mi] = asp[mi][4 * st];
    }
#pragma unroll
    for (int nj = 0; nj < NB; ++nj) bv[nj] = make_b(ld16(bp[nj] + st * 1024));
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < NB; ++nj)
        acc[mi][nj] = mfma_mx(av[mi], bv[nj], acc[mi][nj], sa[mi], sb[nj] >> (8 * (st & 3)));
  }

  // epilogue
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = tile.row_begin + 16 * mi + 4 * g + i;
      const bool valid = row < tile.row_end;
      if (GU) {
#pragma unroll
        for (int p = 0; p < NI / 2; ++p) {
          float h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int j = 2 * p + hh;
            const float gt = acc[mi][j][i], up = acc[mi][NI + j][i];
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
        for (int nj = 0; nj < NB; ++nj) a.o[int64_t(row) * N + col0 + 16 * nj + r16] = acc[mi][nj][i];
      }
    }
  }
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

template <int MI, int NI, int NW, bool GU>
static hipError_t launch_cfg(const FwdArgs& a, hipStream_t st) {
  const int N = GU ? a.dff : a.d;
  dim3 grid(a.max_tiles, N / (16 * NI * NW));
  hipLaunchKernelGGL((k_gemm<MI, NI, NW, GU>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const FwdArgs& a, hipStream_t st) {
  if (a.bm == 16) return launch_dec<2, 2, true>(a, st);
  return launch_cfg<4, 2, 4, true>(a, st);
}

hipError_t launch_gemm_down(const FwdArgs& a, hipStream_t st) {
  if (a.bm == 16) return launch_dec<2, 1, false>(a, st);
  return launch_cfg<4, 2, 4, false>(a, st);
}

}  // namespace mxmoe
