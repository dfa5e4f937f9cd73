// Router, top-k, activation quantiser, token permutation and combine kernels.
//
// Router and top-k follow "Kimi K3 Tech Intro", section 4.3 ("Router (Top-16,
// ...)") and the 16-of-896 routing of the section 1 architecture table; the
// sigmoid score with renormalisation over the selected experts is the reading
// taken for the unspecified score function.  The MXFP8 activation format is
// the "MXFP8 activations" of "Kimi K3 ... MoE推理系统工程分析".
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "internal.h"
#include "mx_device.h"
#include "topk_device.h"

namespace mxmoe {

// ---------------------------------------------------------------------------
// MXFP8 quantisation of 32-element blocks
// ---------------------------------------------------------------------------

// Quantise 32 floats -> 32 codes (two 16-byte stores) + returns the scale byte.
__device__ __forceinline__ uint32_t quant_block32(const float* v, uint8_t* codes) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx8_block_exp(amax);
  // v / 2^e is exact (a power-of-two scale; a product below the fp32 normal
  // range encodes to a signed zero either way), then the hardware E4M3
  // conversion with the +-448 clamp
  const float sc = exp2_int(-e);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3_cvt4(v[4 * i] * sc, v[4 * i + 1] * sc, v[4 * i + 2] * sc, v[4 * i + 3] * sc);
  uint4* dst = reinterpret_cast<uint4*>(codes);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  return static_cast<uint32_t>(e + 127);
}

__device__ __forceinline__ void load_block32_bf16(const uint16_t* src, float* v) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 u = s[q];
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
      v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ void load_block32_f32(const float* src, float* v) {
  const float4* s = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float4 f = s[q];
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
}

template <bool F32>
__global__ void __launch_bounds__(256) k_quantize(const void* __restrict__ src, int64_t rows,
                                                  int64_t cols, int64_t ld,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int64_t nb = cols / 32;
  const int64_t total = rows * nb;
  for (int64_t b = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; b < total;
       b += int64_t(gridDim.x) * blockDim.x) {
    int64_t r = b / nb, c = b - r * nb;
    float v[32];
    if (F32)
      load_block32_f32(static_cast<const float*>(src) + r * ld + c * 32, v);
    else
      load_block32_bf16(static_cast<const uint16_t*>(src) + r * ld + c * 32, v);
    scales[r * nb + c] = static_cast<uint8_t>(quant_block32(v, codes + r * cols + c * 32));
  }
}

hipError_t launch_quantize(const void* src, int src_fp32, int64_t rows, int64_t cols, int64_t ld,
                           uint8_t* codes, uint8_t* scales, hipStream_t st) {
  int64_t total = rows * (cols / 32);
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  if (src_fp32)
    hipLaunchKernelGGL(k_quantize<true>, dim3(grid), dim3(256), 0, st, src, rows, cols, ld, codes, scales);
  else
    hipLaunchKernelGGL(k_quantize<false>, dim3(grid), dim3(256), 0, st, src, rows, cols, ld, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router logits  l[t][e] = sum_i x[t][i] W_r[e][i] + b[e]   (fp32 accumulate)
// ---------------------------------------------------------------------------

// Few tokens: one 256-thread workgroup per expert streams its W_r row (up to 8
// float4 loads in flight per thread, non-temporal: read once per forward) once
// per 8 tokens.  The same launch quantises x to MXFP8: workgroup e takes the
// 32 consecutive activation blocks 32e .. 32e+31 of all T*d/32.

typedef float v4f_nt __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_router_small(FwdArgs a) {
  __shared__ float part[4][8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int d = a.d, T = a.T;
  const int nb = d / 32;
  // Loads are never made conditional: indices past the end are clamped to a
  // valid element and the value is masked afterwards.  A load under a
  // per-lane condition would be placed in its own branch with a full wait,
  // one memory round trip after another.
  // MXFP8 quantisation of x, 8 threads per 32-element block, 32 blocks per
  // workgroup (workgroup e takes blocks 32e .. 32e+31 of all T*d/32): its
  // operand is loaded with the first router weights and used after the dot
  // products (loaded before the loop it would be waited for at the loop head).
  const int qb = 32 * e + (tid >> 3), qj = tid & 7;
  const bool qok = qb < T * nb && !a.a16;  // bf16 activations (A16W4): nothing to quantise
  const int qt = qok ? qb / nb : 0, qc = qok ? qb - qt * nb : 0;
  uint2 qraw = make_uint2(0u, 0u);

  const float4* w4 = reinterpret_cast<const float4*>(a.wr + int64_t(e) * d);
  const int n4 = d / 4;
  const float bias = a.br ? a.br[e] : 0.f;
  for (int t0 = 0; t0 < T; t0 += 8) {
    const int nt = T - t0 < 8 ? T - t0 : 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int base = 0; base < n4; base += 256 * 8) {
      float4 w[8];
      uint32_t ok[8];  // all ones for columns inside the row
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = base + tid + 256 * i;
        ok[i] = c < n4 ? ~0u : 0u;
        // router weights are read once per forward: non-temporal
        const v4f_nt wv = __builtin_nontemporal_load(reinterpret_cast<const v4f_nt*>(w4 + (c < n4 ? c : 0)));
        w[i] = make_float4(wv.x, wv.y, wv.z, wv.w);
      }
      if (t0 == 0 && base == 0)
        qraw = *reinterpret_cast<const uint2*>(a.x + int64_t(qt) * d + qc * 32 + 4 * qj);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        if (tt < nt) {  // the same in every lane
          const uint2* xr = reinterpret_cast<const uint2*>(a.x + int64_t(t0 + tt) * d);
          uint2 xb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = base + tid + 256 * i;
            xb[i] = xr[c < n4 ? c : 0];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            // masked bf16 pairs: columns past the row contribute 0 * w
            const uint32_t x0 = xb[i].x & ok[i], x1 = xb[i].y & ok[i];
            acc[tt] = fmaf(__uint_as_float(x0 << 16), w[i].x, acc[tt]);
            acc[tt] = fmaf(__uint_as_float(x0 & 0xFFFF0000u), w[i].y, acc[tt]);
            acc[tt] = fmaf(__uint_as_float(x1 << 16), w[i].z, acc[tt]);
            acc[tt] = fmaf(__uint_as_float(x1 & 0xFFFF0000u), w[i].w, acc[tt]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      if (tt < nt) {
        float s = group_sum<64>(acc[tt]);
        if (lane == 0) part[wv][tt] = s;
      }
    }
    __syncthreads();
    if (tid < nt) a.logits[int64_t(t0 + tid) * a.E + e] =
        ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) + bias;
    __syncthreads();
  }

  {
    float v[4] = {__uint_as_float(qraw.x << 16), __uint_as_float(qraw.x & 0xFFFF0000u),
                  __uint_as_float(qraw.y << 16), __uint_as_float(qraw.y & 0xFFFF0000u)};
    const float amax = group_max<8>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const int ex = mx8_block_exp(amax);
    const float sc = exp2_int(-ex);
    const uint32_t wq = e4m3_cvt4(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
    if (qok) {
      *reinterpret_cast<uint32_t*>(a.x_codes + int64_t(qt) * d + qc * 32 + 4 * qj) = wq;
      if (qj == 0) a.x_scales[int64_t(qt) * nb + qc] = static_cast<uint8_t>(ex + 127);
    }
  }
}

// Many tokens: router logits on the bf16 MFMA.  x is bf16 already; every
// fp32 router weight w is cut exactly into three bf16 terms by truncation
// (hi = w with the low 16 mantissa bits cleared, mid the same of w - hi, lo =
// w - hi - mid, which has at most 8 significant bits), so x.w = x.hi + x.mid
// + x.lo with every product exact and fp32 accumulation, i.e. fp32 GEMM
// accuracy at bf16 MFMA rate.
//
// Workgroup: 128 tokens x 128 experts, four waves of 64 x 64 (2 x 2 blocks of
// V_MFMA_F32_32X32X16_BF16), K in steps of 32.  Each step's x tile and the
// three weight planes sit in LDS rows of 80 bytes (conflict-free fragment
// reads); the next step's global loads are in registers while the current
// one computes.  With router_ks > 1, blockIdx.z takes one K slice and writes
// partial logits that k_router_reduce sums in slice order.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f_r __attribute__((ext_vector_type(16)));

constexpr int kRtRow = 80;                   // bytes per LDS row (32 bf16 + pad)
constexpr int kRtPlane = 128 * kRtRow;       // one 128-row operand plane
constexpr int kRtStage = 4 * kRtPlane;       // x, w_hi, w_mid, w_lo
constexpr int kRtDepth = 4;                  // K steps in flight (register sets)
template <int N>
struct RtSlot {
  static constexpr int value = N;
};
// f(RtSlot<B>{}), ..., f(RtSlot<E-1>{})
template <int B, int E, typename F>
__device__ __forceinline__ void rt_for(F&& f) {
  if constexpr (B < E) {
    f(RtSlot<B>{});
    rt_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ uint32_t pack_bf16_hi(float a, float b) {
  // upper halves of two floats whose low 16 bits are zero: (b, a) bf16 pair
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

__global__ void __launch_bounds__(256, 1) k_router_mfma(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kRtStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * 128, e0 = blockIdx.y * 128;
  const int kslice = ((a.d / a.router_ks + 31) / 32) * 32;
  const int kb = blockIdx.z * kslice, ke = min(a.d, kb + kslice);
  const int nsteps = ke > kb ? (ke - kb) / 32 : 0;

  // global -> register loads: thread -> row tid/2, 16 K values at 16(tid%2)
  const int lr = tid >> 1, lk = 16 * (tid & 1);
  const uint16_t* xp = a.x + int64_t(min(t0 + lr, a.T - 1)) * a.d + kb + lk;
  const float* wp = a.wr + int64_t(min(e0 + lr, a.E - 1)) * a.d + kb + lk;
  // kRtDepth register sets: step st's global loads go out kRtDepth - 1 steps
  // before its data is split and stored to LDS (one step ahead left the load
  // latency exposed at every step)
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  typedef float v4f_r __attribute__((ext_vector_type(4)));
  v4u xr[kRtDepth][2];
  v4f_r wr4[kRtDepth][4];
  auto load = [&](int st, auto S) __attribute__((always_inline)) {
    constexpr int slot = decltype(S)::value;
    const v4u* xs = reinterpret_cast<const v4u*>(xp + 32 * st);
    xr[slot][0] = xs[0];
    xr[slot][1] = xs[1];
    const v4f_r* ws = reinterpret_cast<const v4f_r*>(wp + 32 * st);
#pragma unroll
    for (int q = 0; q < 4; ++q) wr4[slot][q] = ws[q];
  };
  // split the weights of register set `slot` into three bf16 planes and store
  // the step to LDS buffer b
  auto store = [&](int b, auto S) __attribute__((always_inline)) {
    constexpr int slot = decltype(S)::value;
    uint8_t* base = lds + b * kRtStage + lr * kRtRow + 2 * lk;
    *reinterpret_cast<v4u*>(base) = xr[slot][0];
    *reinterpret_cast<v4u*>(base + 16) = xr[slot][1];
    float w[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[4 * q] = wr4[slot][q].x; w[4 * q + 1] = wr4[slot][q].y;
      w[4 * q + 2] = wr4[slot][q].z; w[4 * q + 3] = wr4[slot][q].w;
    }
    uint32_t hi[8], mid[8], lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float h2[2], m2[2], l2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float v = w[2 * j + u];
        const float h = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
        const float r = v - h;
        const float m = __uint_as_float(__float_as_uint(r) & 0xFFFF0000u);
        h2[u] = h;
        m2[u] = m;
        l2[u] = r - m;
      }
      hi[j] = pack_bf16_hi(h2[0], h2[1]);
      mid[j] = pack_bf16_hi(m2[0], m2[1]);
      lo[j] = pack_bf16_hi(l2[0], l2[1]);
    }
    uint8_t* wb = lds + b * kRtStage + kRtPlane + lr * kRtRow + 2 * lk;
    *reinterpret_cast<uint4*>(wb) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(wb + 16) = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    *reinterpret_cast<uint4*>(wb + kRtPlane) = make_uint4(mid[0], mid[1], mid[2], mid[3]);
    *reinterpret_cast<uint4*>(wb + kRtPlane + 16) = make_uint4(mid[4], mid[5], mid[6], mid[7]);
    *reinterpret_cast<uint4*>(wb + 2 * kRtPlane) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(wb + 2 * kRtPlane + 16) = make_uint4(lo[4], lo[5], lo[6], lo[7]);
  };

  v16f_r acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f_r{};
  // fragment lane: row l%32 of a 32-row block, K elements 8(l/32) .. +7 of a 16-chunk
  const int frag = (lane & 31) * kRtRow + 16 * (lane >> 5);
  auto compute = [&](int b) __attribute__((always_inline)) {
    const uint8_t* base = lds + b * kRtStage;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      v8bf av[2], bv[3][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const v8bf*>(base + (64 * wm + 32 * i) * kRtRow + frag + 32 * kc);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bv[pl][j] = *reinterpret_cast<const v8bf*>(base + (pl + 1) * kRtPlane + (64 * wn + 32 * j) * kRtRow +
                                                     frag + 32 * kc);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[pl][j], acc[i][j], 0, 0, 0);
    }
  };

  if (nsteps > 0) {
    // steps 0 .. kRtDepth-2 in flight; step s lives in register set s % kRtDepth
    rt_for<0, kRtDepth - 1>([&](auto U) { load(min(decltype(U)::value, nsteps - 1), U); });
    store(0, RtSlot<0>{});
    __syncthreads();
    // one step; U (a compile-time constant) picks the register sets
    auto step = [&](int st, auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      // past the last step the last one is loaded again (never stored)
      load(min(st + kRtDepth - 1, nsteps - 1), RtSlot<(u + kRtDepth - 1) % kRtDepth>{});
      compute(st & 1);
      if (st + 1 < nsteps) store((st + 1) & 1, RtSlot<(u + 1) % kRtDepth>{});
      __syncthreads();
    };
    // whole groups of kRtDepth steps without conditions (conditional copies
    // of the step were merged by the compiler into one with a run-time
    // register set, i.e. private memory), then at most kRtDepth - 1 more
    int st0 = 0;
    for (; st0 + kRtDepth <= nsteps; st0 += kRtDepth)
      rt_for<0, kRtDepth>([&](auto U) { step(st0 + decltype(U)::value, U); });
    rt_for<0, kRtDepth - 1>([&](auto U) {  // conditions are the same in every lane
      if (st0 + decltype(U)::value < nsteps) step(st0 + decltype(U)::value, U);
    });
  }

  // acc[i][j] register r: token 64wm + 32i + 8(r/4) + 4(lane/32) + r%4,
  // expert 64wn + 32j + lane%32
  const bool partial = a.router_ks > 1;
  float* out = partial ? a.router_part + int64_t(blockIdx.z) * a.T * a.E : a.logits;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 64 * wn + 32 * j + (lane & 31);
    if (e >= a.E) continue;
    const float bias = (!partial && a.br) ? a.br[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 64 * wm + 32 * i + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (t < a.T) out[int64_t(t) * a.E + e] = acc[i][j][r] + bias;
      }
  }
}

// logits = sum of the K-slice partials in slice order, plus the bias
__global__ void __launch_bounds__(256) k_router_reduce(FwdArgs a) {
  const int64_t n = int64_t(a.T) * a.E;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    float s = 0.0f;
    for (int ks = 0; ks < a.router_ks; ++ks) s += a.router_part[ks * n + i];
    a.logits[i] = s + (a.br ? a.br[i % a.E] : 0.0f);
  }
}

hipError_t launch_router(const FwdArgs& a, hipStream_t st) {
  // the small-batch router also quantises x: 32 blocks per expert workgroup
  if (router_small(a.T, a.d, a.E)) {
    hipLaunchKernelGGL(k_router_small, dim3(a.E), dim3(256), 0, st, a);
  } else {
    dim3 grid((a.T + 127) / 128, (a.E + 127) / 128, a.router_ks);
    hipLaunchKernelGGL(k_router_mfma, grid, dim3(256), 0, st, a);
    if (a.router_ks > 1) {
      const int64_t n = int64_t(a.T) * a.E;
      const int blocks = static_cast<int>(std::min<int64_t>((n + 255) / 256, 4096));
      hipLaunchKernelGGL(k_router_reduce, dim3(blocks), dim3(256), 0, st, a);
    }
  }
  return hipGetLastError();
}

// Many tokens: one wave per token, top-k then the token's MXFP8 row.
__global__ void __launch_bounds__(256) k_topk_quant(FwdArgs a) {
  __shared__ uint2 cand[4][64];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  topk_token(a, t, lane, cand[threadIdx.x >> 6]);
  if (a.a16) return;  // bf16 activations (A16W4): x is used as it is
  const int nb = a.d / 32;
  const uint16_t* xr = a.x + int64_t(t) * a.d;
  for (int b = lane; b < nb; b += 64) {
    float v[32];
    load_block32_bf16(xr + b * 32, v);
    a.x_scales[int64_t(t) * nb + b] =
        static_cast<uint8_t>(quant_block32(v, a.x_codes + int64_t(t) * a.d + b * 32));
  }
}



// ---------------------------------------------------------------------------
// Permutation: pairs (t, j) -> rows grouped by expert, tokens ascending.
// Ranks come from per-chunk bitmasks of the 64 tokens in a chunk, so the
// result is deterministic and needs no ordered atomics.
// ---------------------------------------------------------------------------

// Exclusive scan of n <= 2048 ints held in LDS `v` (in place); returns the total.
// Must be called by all threads of a 1024-thread workgroup.
__device__ int block_exclusive_scan(int* v, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    int i = base + tid;
    int x = i < n ? v[i] : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      int w = lane < 16 ? wave_tot[lane] : 0;
      int wi = w;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        int y = __shfl_up(wi, o, 64);
        if (lane >= o) wi += y;
      }
      if (lane < 16) wave_tot[16 + lane] = wi - w;  // exclusive wave offsets
      if (lane == 15) wave_tot[32] = wi;            // chunk total
    }
    __syncthreads();
    if (i < n) v[i] = carry + wave_tot[16 + wv] + incl - x;
    carry += wave_tot[32];
    __syncthreads();
  }
  return carry;
}

// Offsets, counts and the tile list from per-expert counts held in LDS `cnt`
// (routed experts [0, E)); shared experts contribute T rows each.
__device__ void write_offsets_and_tiles(const FwdArgs& a, int* cnt, int* scan, int* wave_tot) {
  const int tid = threadIdx.x;
  const int nex = a.E + a.S;
  for (int e = tid; e < a.E; e += 1024) scan[e] = cnt[e];
  __syncthreads();
  block_exclusive_scan(scan, a.E, wave_tot);
  for (int e = tid; e < a.E; e += 1024) {
    a.offsets[e] = scan[e];
    a.counts[e] = cnt[e];
  }
  if (tid == 0) a.offsets[a.E] = a.Rr;
  __syncthreads();
  // tiles per expert -> LDS cnt reused as tile counts; scan[] keeps row starts
  for (int ex = tid; ex < nex; ex += 1024) {
    int rows = ex < a.E ? cnt[ex] : a.T;
    cnt[ex] = (rows + a.bm - 1) / a.bm;
    if (ex >= a.E) scan[ex] = a.Rr + (ex - a.E) * a.T;
  }
  __syncthreads();
  // scan tile counts into tile_start (stored in cnt)
  int ntiles = block_exclusive_scan(cnt, nex, wave_tot);
  for (int ex = tid; ex < nex; ex += 1024) a.ex_tiles[ex] = cnt[ex];
  if (tid == 0) a.ex_tiles[nex] = ntiles;
  for (int ex = tid; ex < nex; ex += 1024) {
    int rb = scan[ex];
    int rows = ex < a.E ? (ex + 1 < a.E ? scan[ex + 1] : a.Rr) - rb : a.T;
    int re = rb + rows;
    int first = cnt[ex];
    int nt = (rows + a.bm - 1) / a.bm;
    for (int i = 0; i < nt; ++i) {
      Tile tl;
      tl.ex = ex;
      tl.row_begin = rb + i * a.bm;
      tl.row_end = min(rb + (i + 1) * a.bm, re);
      tl.pad = 0;
      a.tiles[first + i] = tl;
    }
  }
  if (tid == 0) *a.tile_count = ntiles;
}

// Whole permutation in one 1024-thread workgroup (moderate token counts).
struct PermLds {
  int cnt[1032];
  int scan[1032];
  int run[1024];
  unsigned long long mask[1024];
  int wave_tot[40];
};

__device__ void permute_block(const FwdArgs& a, PermLds& L) {
  const int tid = threadIdx.x;
  const int npairs = a.T * a.k;
  for (int e = tid; e < a.E; e += 1024) { L.cnt[e] = 0; L.run[e] = 0; }
  __syncthreads();
  for (int p = tid; p < npairs; p += 1024) atomicAdd(&L.cnt[a.topk_ids[p]], 1);
  __syncthreads();
  write_offsets_and_tiles(a, L.cnt, L.scan, L.wave_tot);
  __syncthreads();
  // scan[e] now holds the first row of routed expert e
  for (int t0 = 0; t0 < a.T; t0 += 64) {
    for (int e = tid; e < a.E; e += 1024) L.mask[e] = 0ull;
    __syncthreads();
    const int tend = min(t0 + 64, a.T);
    const int p0 = t0 * a.k, p1 = tend * a.k;
    for (int p = p0 + tid; p < p1; p += 1024) {
      int t = p / a.k;
      atomicOr(&L.mask[a.topk_ids[p]], 1ull << (t - t0));
    }
    __syncthreads();
    for (int p = p0 + tid; p < p1; p += 1024) {
      int t = p / a.k;
      int e = a.topk_ids[p];
      unsigned long long below = (t - t0) == 0 ? 0ull : (~0ull >> (64 - (t - t0)));
      int row = L.scan[e] + L.run[e] + __popcll(L.mask[e] & below);
      a.row_src[row] = p;
      a.row_token[row] = t;
      a.token_row[p] = row;
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += 1024) L.run[e] += __popcll(L.mask[e]);
    __syncthreads();
  }
}

__global__ void __launch_bounds__(1024) k_permute_small(FwdArgs a) {
  __shared__ PermLds L;
  permute_block(a, L);
}

// Few tokens (router_small: T <= 32): top-k of every token (one wave each)
// with the choices kept in LDS, then the permutation in the same workgroup:
// per-expert counts and token bitmasks by LDS atomics, one scan of the packed
// (rows | tiles << 16) per expert for row and tile starts, and each pair's
// row = expert start + number of earlier tokens with that expert.  x was
// already quantised by the router launch.
__global__ void __launch_bounds__(1024) k_topk_permute_small(FwdArgs a) {
  __shared__ uint2 cand[16][64];
  __shared__ int s_ids[32 * 32];
  __shared__ int cnt[1024];
  __shared__ uint32_t mask[1024];
  __shared__ int wave_tot[40];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < a.E) { cnt[tid] = 0; mask[tid] = 0u; }
  for (int t = wv; t < a.T; t += 16) topk_token(a, t, lane, cand[wv], s_ids);
  __syncthreads();
  const int npairs = a.T * a.k;
  for (int p = tid; p < npairs; p += 1024) {
    const int e = s_ids[p];
    atomicAdd(&cnt[e], 1);
    atomicOr(&mask[e], 1u << (p / a.k));
  }
  __syncthreads();
  const int c = tid < a.E ? cnt[tid] : 0;
  const int ntile = (c + a.bm - 1) / a.bm;
  if (tid < a.E) cnt[tid] = c | (ntile << 16);
  const int total = block_exclusive_scan(cnt, a.E, wave_tot);  // ends with a barrier
  const int rtiles = total >> 16;
  const int nts = (a.T + a.bm - 1) / a.bm;  // tiles per shared expert
  if (tid < a.E) {
    const int row0 = cnt[tid] & 0xFFFF, tile0 = cnt[tid] >> 16;
    a.offsets[tid] = row0;
    a.counts[tid] = c;
    a.ex_tiles[tid] = tile0;
    for (int i = 0; i < ntile; ++i) {
      Tile tl;
      tl.ex = tid;
      tl.row_begin = row0 + i * a.bm;
      tl.row_end = min(row0 + (i + 1) * a.bm, row0 + c);
      tl.pad = 0;
      a.tiles[tile0 + i] = tl;
    }
  }
  if (tid < a.S * nts) {
    const int sx = tid / nts, i = tid % nts;
    const int rb = a.Rr + sx * a.T;
    Tile tl;
    tl.ex = a.E + sx;
    tl.row_begin = rb + i * a.bm;
    tl.row_end = min(rb + (i + 1) * a.bm, rb + a.T);
    tl.pad = 0;
    a.tiles[rtiles + tid] = tl;
  }
  if (tid <= a.S) a.ex_tiles[a.E + tid] = rtiles + tid * nts;
  if (tid == 0) {
    a.offsets[a.E] = a.Rr;
    *a.tile_count = rtiles + a.S * nts;
  }
  for (int p = tid; p < npairs; p += 1024) {
    const int t = p / a.k, e = s_ids[p];
    const int row = (cnt[e] & 0xFFFF) + __popc(mask[e] & ((1u << t) - 1u));
    a.row_src[row] = p;
    a.row_token[row] = t;
    a.token_row[p] = row;
  }
}

// Large token counts: per-chunk masks and counts ...
__global__ void __launch_bounds__(256) k_perm_count(FwdArgs a) {
  __shared__ unsigned long long mask[1024];
  const int c = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < a.E; e += 256) mask[e] = 0ull;
  __syncthreads();
  const int t0 = c * 64, tend = min(t0 + 64, a.T);
  for (int p = t0 * a.k + tid; p < tend * a.k; p += 256) {
    int t = p / a.k;
    atomicOr(&mask[a.topk_ids[p]], 1ull << (t - t0));
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += 256) {
    unsigned long long m = mask[e];
    a.chunk_mask[int64_t(c) * a.E + e] = m;
    a.chunk_base[int64_t(e) * a.nchunks + c] = __popcll(m);
  }
}

// ... per-expert exclusive scan over chunks (one wave per expert) ...
__global__ void __launch_bounds__(256) k_perm_scan_chunks(FwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.E) return;
  int32_t* cb = a.chunk_base + int64_t(e) * a.nchunks;
  int carry = 0;
  for (int c0 = 0; c0 < a.nchunks; c0 += 64) {
    int c = c0 + lane;
    int x = c < a.nchunks ? cb[c] : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (c < a.nchunks) cb[c] = carry + incl - x;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) a.counts[e] = carry;
}

// ... expert offsets and tile list ...
__global__ void __launch_bounds__(1024) k_perm_offsets(FwdArgs a) {
  __shared__ int cnt[1032];
  __shared__ int scan[1032];
  __shared__ int wave_tot[40];
  for (int e = threadIdx.x; e < a.E; e += 1024) cnt[e] = a.counts[e];
  __syncthreads();
  write_offsets_and_tiles(a, cnt, scan, wave_tot);
}

// ... and the scatter.
__global__ void __launch_bounds__(256) k_perm_scatter(FwdArgs a) {
  const int c = blockIdx.x, tid = threadIdx.x;
  const int t0 = c * 64, tend = min(t0 + 64, a.T);
  for (int p = t0 * a.k + tid; p < tend * a.k; p += 256) {
    int t = p / a.k;
    int e = a.topk_ids[p];
    unsigned long long m = a.chunk_mask[int64_t(c) * a.E + e];
    unsigned long long below = (t - t0) == 0 ? 0ull : (~0ull >> (64 - (t - t0)));
    int row = a.offsets[e] + a.chunk_base[int64_t(e) * a.nchunks + c] + __popcll(m & below);
    a.row_src[row] = p;
    a.row_token[row] = t;
    a.token_row[p] = row;
  }
}

// ---------------------------------------------------------------------------
// Router bias balancing step: b_e += rate * sign(T*k/E - c_e), the loads c_e
// from a forward's expert offsets.  "Kimi K3 Tech Intro" names quantile
// balancing for the router without defining it; this is the reading taken.
// The sign is decided in integers (T*k - c_e*E), the addition in fp32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_router_bias_update(const int32_t* __restrict__ offsets, int E,
                                                            int64_t tk, float rate, float* __restrict__ b) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t c = offsets[e + 1] - offsets[e];
  const int64_t d = tk - c * E;
  const float step = d > 0 ? rate : (d < 0 ? -rate : 0.0f);
  b[e] = b[e] + step;
}

hipError_t launch_router_bias_update(const int32_t* offsets, int E, int64_t tk, float rate, float* b,
                                     hipStream_t st) {
  hipLaunchKernelGGL(k_router_bias_update, dim3((E + 255) / 256), dim3(256), 0, st, offsets, E, tk, rate, b);
  return hipGetLastError();
}

hipError_t launch_topk_quant(const FwdArgs& a, hipStream_t st) {
  if (stream_split_phases(a)) return launch_topk_shared_gate_up(a, st);
  if (router_small(a.T, a.d, a.E))
    hipLaunchKernelGGL(k_topk_permute_small, dim3(1), dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(k_topk_quant, dim3((a.T + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_permute(const FwdArgs& a, hipStream_t st) {
  if (router_small(a.T, a.d, a.E))
    return hipSuccess;  // done with the top-k launch
  if (a.T <= kPermSmallMaxTokens) {
    hipLaunchKernelGGL(k_permute_small, dim3(1), dim3(1024), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_perm_count, dim3(a.nchunks), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_scan_chunks, dim3((a.E + 3) / 4), dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_perm_offsets, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(k_perm_scatter, dim3(a.nchunks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j w[t][j] o[row(t,j)] + sum_s o[shared row(s,t)]
// (fixed order: slots ascending = expert id ascending, then shared experts)
// ---------------------------------------------------------------------------

// One thread per 8 output columns of one token (one 16-byte load of bf16 o
// per row); the k expert rows are read in batches of 16 loads in flight and
// summed in slot order, then the shared rows.  The decode kernels leave o in
// permuted-row order (found through token_row); the prefill kernels store it
// in (token, slot) order (TOKMAJOR), so a token's k rows are contiguous.
typedef uint32_t v4u_nt __attribute__((ext_vector_type(4)));

template <bool TOKMAJOR, int NSH>
__global__ void __launch_bounds__(64) k_combine(FwdArgs a) {
  constexpr int C = 8;
  // workgroup = (token, 512-column block), blocks of a token adjacent: the
  // workgroups in flight read whole o rows rather than one 1 KB piece of
  // every row
  const int nblk = (a.d / C + 63) / 64;
  const int t = blockIdx.x / nblk;
  const int cg = (blockIdx.x - t * nblk) * 64 + threadIdx.x;  // column group
  // every lane stays to the end (lanes 0..15 hand the slot weights to the
  // others); lanes past the row load column group 0 and store nothing
  const bool live = cg < a.d / C;
  const int c = live ? cg : 0;
  // o rows are read once: non-temporal loads, kept raw until every load of
  // the pass is out (a conversion right after each load would make the
  // compiler wait on it)
  auto load = [&](int64_t row) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4u_nt*>(a.o16 + row * a.d) + c);
  };
  auto add = [&](const v4u_nt& u, float w, float* acc) {
    const uint32_t q4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(w, __uint_as_float(q4[q] << 16), acc[2 * q]);
      acc[2 * q + 1] = fmaf(w, __uint_as_float(q4[q] & 0xFFFF0000u), acc[2 * q + 1]);
    }
  };
  float r[C], sh[C];
#pragma unroll
  for (int q = 0; q < C; ++q) r[q] = sh[q] = 0.f;
  // Lane l < 32 first reads slot l's weight and row (clamped into the
  // token's k entries; slots past k get weight 0), and every lane takes the
  // values from those lanes: one load each, issued before any o row so that
  // waiting for it waits for nothing else.  Every o load is unconditional
  // (slots past k re-read slot k-1 with weight 0; shared experts past S
  // re-read the last one, or with S = 0 a routed row, masked to 0), so the
  // NSH + 16 row loads go out together instead of one branch and one full
  // wait per load.  Sums run in slot order, then shared-expert order.
  const int lane = threadIdx.x;
  const int jl = min(lane & 31, a.k - 1);
  const uint32_t wl = __float_as_uint(a.topk_w[int64_t(t) * a.k + jl]);
  const int rl = TOKMAJOR ? 0 : a.token_row[int64_t(t) * a.k + jl];
  __builtin_amdgcn_sched_barrier(0);
  v4u_nt us[NSH];
#pragma unroll
  for (int s = 0; s < NSH; ++s) us[s] = load(int64_t(a.Rr + (s < a.S ? s : a.S - 1) * a.T + t));
  for (int j0 = 0; j0 < a.k; j0 += 16) {
    v4u_nt u[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int j = j0 + k < a.k ? j0 + k : a.k - 1;
      u[k] = load(TOKMAJOR ? int64_t(t) * a.k + j : int64_t(__builtin_amdgcn_readlane(rl, j)));
    }
    __builtin_amdgcn_sched_barrier(0);
    float w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = __uint_as_float(__builtin_amdgcn_readlane(wl, j0 + k) & (j0 + k < a.k ? ~0u : 0u));
#pragma unroll
    for (int k = 0; k < 16; ++k) add(u[k], w[k], r);
  }
#pragma unroll
  for (int s = 0; s < NSH; ++s) {
    const uint32_t m = s < a.S ? ~0u : 0u;
    const uint32_t q4[4] = {us[s].x & m, us[s].y & m, us[s].z & m, us[s].w & m};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sh[2 * q] += __uint_as_float(q4[q] << 16);
      sh[2 * q + 1] += __uint_as_float(q4[q] & 0xFFFF0000u);
    }
  }
  uint32_t yb[C / 2];
#pragma unroll
  for (int q = 0; q < C / 2; ++q)
    yb[q] = uint32_t(f32_to_bf16_rne(r[2 * q] + sh[2 * q])) |
            (uint32_t(f32_to_bf16_rne(r[2 * q + 1] + sh[2 * q + 1])) << 16);
  if (!live) return;
  reinterpret_cast<uint4*>(a.y + int64_t(t) * a.d)[c] = make_uint4(yb[0], yb[1], yb[2], yb[3]);
  if (a.y_routed) {
    float4* yr = reinterpret_cast<float4*>(a.y_routed + int64_t(t) * a.d) + (C / 4) * c;
#pragma unroll
    for (int q = 0; q < C / 4; ++q) yr[q] = make_float4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
  }
  if (a.y_shared) {
    float4* ys = reinterpret_cast<float4*>(a.y_shared + int64_t(t) * a.d) + (C / 4) * c;
#pragma unroll
    for (int q = 0; q < C / 4; ++q) ys[q] = make_float4(sh[4 * q], sh[4 * q + 1], sh[4 * q + 2], sh[4 * q + 3]);
  }
}

hipError_t launch_combine(const FwdArgs& a, hipStream_t st) {
  // o rows in (token, slot) order after the prefill kernels, in permuted-row
  // order after the decode ones
  const unsigned grid = static_cast<unsigned>(a.T) * static_cast<unsigned>((a.d / 8 + 63) / 64);
  // shared rows: two loads cover the usual S <= 2, eight any S (unused
  // ones re-read the last row and are masked)
  if (a.bm > kDecodeMaxRows && a.S <= 2)
    hipLaunchKernelGGL((k_combine<true, 2>), dim3(grid), dim3(64), 0, st, a);
  else if (a.bm > kDecodeMaxRows)
    hipLaunchKernelGGL((k_combine<true, 8>), dim3(grid), dim3(64), 0, st, a);
  else if (a.S <= 2)
    hipLaunchKernelGGL((k_combine<false, 2>), dim3(grid), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((k_combine<false, 8>), dim3(grid), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mxmoe
