// LatentMoE tail: y = MXFP8(RMSNorm(z)) W_up^T + s.  "Kimi K3 Tech Intro",
// section 4.3 puts the latent up-projection, RMSNorm and an element-wise add
// after the routed and shared experts; section 4.4 has the routed output go
// through RMSNorm and the up projection while the shared output is added to
// it directly.  The projection reuses the down-GEMM kernels (one "expert",
// K = latent width, N = hidden width); this file holds the RMSNorm + MXFP8
// quantiser in front of it and the add behind it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "internal.h"
#include "mx_device.h"

namespace mxmoe {

// One 256-thread workgroup per token row of z (fp32, `latent` columns).
// Pass 1: sum of squares (float4 loads, fp32, tree reduction over the
// workgroup) -> inv_rms = 1 / sqrt(mean + eps).  Pass 2 (the row is in L2 by
// then): n = z * inv_rms * gamma, quantised per 32-element block by 8 threads
// (4 values each) with the hardware E4M3 conversion after the power-of-two
// scaling, as for every other activation of the layer.  Workgroup t also
// writes row_src[t] = t (the projection's rows are in token order) and
// workgroup 0 the projection's tile list.
// The row's values a thread holds in registers between the two passes (rows
// of up to 8192 columns; wider rows load again in pass 2, from L2).
constexpr int kTailRegF4 = 8;

__global__ void __launch_bounds__(256) k_tail_norm_quant(TailArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l = a.latent;
  const float4* z4 = reinterpret_cast<const float4*>(a.z + int64_t(t) * l);
  const int n4 = l / 4;
  const bool in_regs = n4 <= 256 * kTailRegF4;
  // pass 1: every load of the row issued before the first use; float4 i of
  // sweep p is element block (p*256 + tid), the one pass 2 quantises
  const float4* g4 = reinterpret_cast<const float4*>(a.gamma);
  float4 zr[kTailRegF4], gr[kTailRegF4];
  float ss = 0.f;
  if (in_regs) {
#pragma unroll
    for (int p = 0; p < kTailRegF4; ++p) {
      const int i = p * 256 + tid;
      zr[p] = z4[i < n4 ? i : 0];
      gr[p] = g4[i < n4 ? i : 0];
    }
#pragma unroll
    for (int p = 0; p < kTailRegF4; ++p) {
      if (p * 256 + tid < n4) {
        ss = fmaf(zr[p].x, zr[p].x, ss);
        ss = fmaf(zr[p].y, zr[p].y, ss);
        ss = fmaf(zr[p].z, zr[p].z, ss);
        ss = fmaf(zr[p].w, zr[p].w, ss);
      }
    }
  } else {
    for (int i = tid; i < n4; i += 256) {
      const float4 v = z4[i];
      ss = fmaf(v.x, v.x, ss);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
    }
  }
  ss = group_sum<64>(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  const float ms = ((red[0] + red[1]) + (red[2] + red[3])) / static_cast<float>(l);
  const float inv = 1.0f / sqrtf(ms + a.eps);
  if (tid == 0) {
    if (a.inv_rms) a.inv_rms[t] = inv;
    a.row_src[t] = t;
  }
  // pass 2: 8 threads per block, 32 blocks per sweep of the workgroup (thread
  // tid of sweep p holds float4 p*256 + tid: block 32p + tid/8, part tid%8)
  const int nb = l / 32;
  auto quant = [&](int b0, const float4& v, const float4& g) {
    const int b = b0 + (tid >> 3), j = tid & 7;
    const bool ok = b < nb;                         // the same for the 8 threads of a block
    float q[4] = {v.x * inv * g.x, v.y * inv * g.y, v.z * inv * g.z, v.w * inv * g.w};
    const float amax = group_max<8>(fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3]))));
    const int e = mx8_block_exp(amax);
    const float sc = exp2_int(-e);
    const uint32_t w = e4m3_cvt4(q[0] * sc, q[1] * sc, q[2] * sc, q[3] * sc);
    if (ok) {
      *reinterpret_cast<uint32_t*>(a.codes + int64_t(t) * l + 32 * b + 4 * j) = w;
      if (j == 0) a.scales[int64_t(t) * nb + b] = static_cast<uint8_t>(e + 127);
    }
  };
  if (in_regs) {
    // compile-time sweep index: the registers stay registers
#pragma unroll
    for (int p = 0; p < kTailRegF4; ++p)
      if (32 * p < nb) quant(32 * p, zr[p], gr[p]);  // the same in every thread
  } else {
    for (int b0 = 0; b0 < nb; b0 += 32) {
      const int i4 = min(b0 * 8 + tid, n4 - 1);
      quant(b0, z4[i4], g4[i4]);
    }
  }
  if (t == 0) {
    const int ntiles = (a.T + a.bm - 1) / a.bm;
    for (int i = tid; i < ntiles; i += 256) {
      Tile tl;
      tl.ex = 0;
      tl.row_begin = i * a.bm;
      tl.row_end = min((i + 1) * a.bm, a.T);
      tl.pad = 0;
      a.tiles[i] = tl;
    }
    if (tid == 0) {
      *a.tile_count = ntiles;
      a.ex_tiles[0] = 0;
      a.ex_tiles[1] = ntiles;
    }
  }
}

// y = bf16(o + s): o the projection's bf16 rows, s fp32; 8 columns per thread
__global__ void __launch_bounds__(256) k_tail_add(const uint16_t* __restrict__ o, const float* __restrict__ s,
                                                  uint16_t* __restrict__ y, int64_t n8) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n8; i += int64_t(gridDim.x) * 256) {
    const uint4 ob = reinterpret_cast<const uint4*>(o)[i];
    const float4 s0 = reinterpret_cast<const float4*>(s)[2 * i];
    const float4 s1 = reinterpret_cast<const float4*>(s)[2 * i + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint32_t ow[4] = {ob.x, ob.y, ob.z, ob.w};
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = __uint_as_float(ow[q] << 16) + sv[2 * q];
      const float hi = __uint_as_float(ow[q] & 0xFFFF0000u) + sv[2 * q + 1];
      r[q] = uint32_t(f32_to_bf16_rne(lo)) | (uint32_t(f32_to_bf16_rne(hi)) << 16);
    }
    reinterpret_cast<uint4*>(y)[i] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// Few rows (T <= kTailGemvMaxT): the projection split along K.  Workgroup
// (G, ks) computes the 64 outputs of packed weight group G over K steps
// [ks*spk, min((ks+1)*spk, ns)); its wave w takes steps w, w+4, ... of that
// range -- at most kTailGemvSteps -- and issues every load of them (weights
// non-temporal: read once) before its first MFMA, straight into registers:
// a few hundred workgroups each with all of their bytes in flight at once.
// The 16 MFMA rows are the rows of z (rows past T repeat the last one and
// are not written).  The four waves' sums meet in LDS and are added in wave
// order; the fp32 partial of slice ks goes to part[ks][T][hidden], and
// k_tail_reduce adds the slices in order (plus s) and rounds to bf16.
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u_nt_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f_t tail_mfma(const v8i_t& av, const v8i_t& bv, v4f_t c, uint32_t sa, uint32_t sb) {
  // A: FP8 E4M3 (format 0), B: FP4 E2M1 (format 4); scales in byte 0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, static_cast<int>(sa), 0,
                                                          static_cast<int>(sb));
}

template <bool CANON>
__global__ void __launch_bounds__(256) k_tail_gemv(TailArgs a, float* __restrict__ part, int ks_n) {
  __shared__ v4f_t red[4][4][64];
  const int G = blockIdx.x, ks = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane >> 4, r16 = lane & 15;
  const int K = a.latent, ns = K / 128;
  const int spk = (ns + ks_n - 1) / ks_n;
  const int s0 = ks * spk, s1 = min(ns, s0 + spk);
  // packed: the group's step is 4 KB in lane order, its scales a dword per
  // lane; canonical: lane (g, r) of block j reads row 64G + 16j + r at K
  // bytes 64 st + 16g, and byte g of the dword of that row's blocks
  // 4st .. 4st+3
  const uint8_t* wc = CANON ? a.up_c + (int64_t(G) * 64 + r16) * (K / 2) + 16 * g
                            : a.up_c + int64_t(G) * ns * 4096 + 16 * lane;
  const uint8_t* wsc = CANON ? a.up_s + (int64_t(G) * 64 + r16) * (K / 32) : a.up_s + int64_t(G) * ns * 256 + 4 * lane;
  const int row = min(r16, a.T - 1);
  const uint8_t* ac = a.codes + int64_t(row) * K;
  const uint8_t* asc = a.scales + int64_t(row) * (K / 32);
  uint4 wv[kTailGemvSteps][4], a0[kTailGemvSteps], a1[kTailGemvSteps];
  uint32_t sbw[kTailGemvSteps][CANON ? 4 : 1], sa[kTailGemvSteps];
#pragma unroll
  for (int i = 0; i < kTailGemvSteps; ++i) {
    const int st = s0 + w + 4 * i;
    const int sst = st < s1 ? st : min(s0, ns - 1);  // past the range: a valid step, its values unused
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* src = CANON ? wc + int64_t(16 * j) * (K / 2) + int64_t(sst) * 64 : wc + int64_t(sst) * 4096 + j * 1024;
      const v4u_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_nt_t*>(src));
      wv[i][j] = make_uint4(v.x, v.y, v.z, v.w);
    }
    if constexpr (CANON) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sbw[i][j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsc + int64_t(16 * j) * (K / 32) + int64_t(sst) * 4));
    } else {
      sbw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(wsc + int64_t(sst) * 256));
    }
    a0[i] = *reinterpret_cast<const uint4*>(ac + sst * 128 + 16 * g);
    a1[i] = *reinterpret_cast<const uint4*>(ac + sst * 128 + 64 + 16 * g);
    sa[i] = *reinterpret_cast<const uint32_t*>(asc + 4 * sst);
  }
  v4f_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kTailGemvSteps; ++i) {
    if (s0 + w + 4 * i < s1) {  // the same in every lane
      v8i_t av;
      av[0] = a0[i].x; av[1] = a0[i].y; av[2] = a0[i].z; av[3] = a0[i].w;
      av[4] = a1[i].x; av[5] = a1[i].y; av[6] = a1[i].z; av[7] = a1[i].w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v8i_t bv;
        bv[0] = wv[i][j].x; bv[1] = wv[i][j].y; bv[2] = wv[i][j].z; bv[3] = wv[i][j].w;
        bv[4] = 0; bv[5] = 0; bv[6] = 0; bv[7] = 0;
        acc[j] = tail_mfma(av, bv, acc[j], sa[i] >> (8 * g), CANON ? sbw[i][CANON ? j : 0] >> (8 * g) : sbw[i][0] >> (8 * j));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[w][j][lane] = acc[j];
  __syncthreads();
  // thread (j, l): block j's lane l -- rows 4(l/16) .. +3, column 16j + l%16
  const int j = threadIdx.x >> 6, l = threadIdx.x & 63;
  const v4f_t s = ((red[0][j][l] + red[1][j][l]) + red[2][j][l]) + red[3][j][l];
  const int col = 64 * G + 16 * j + (l & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (l >> 4) + i;
    if (r < a.T) part[(int64_t(ks) * a.T + r) * a.hidden + col] = s[i];
  }
}

// y = bf16(sum of the K slices in order (+ s)); 4 columns per thread
__global__ void __launch_bounds__(256) k_tail_reduce(const float* __restrict__ part, int ks_n,
                                                     const float* __restrict__ s, uint16_t* __restrict__ y,
                                                     int64_t n4) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    float4 v = reinterpret_cast<const float4*>(part)[i];
    for (int k = 1; k < ks_n; ++k) {
      const float4 p = reinterpret_cast<const float4*>(part)[k * n4 + i];
      v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    }
    if (s) {
      const float4 q = reinterpret_cast<const float4*>(s)[i];
      v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
    }
    const uint32_t lo = uint32_t(f32_to_bf16_rne(v.x)) | (uint32_t(f32_to_bf16_rne(v.y)) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16_rne(v.z)) | (uint32_t(f32_to_bf16_rne(v.w)) << 16);
    reinterpret_cast<uint2*>(y)[i] = make_uint2(lo, hi);
  }
}

hipError_t launch_tail(const TailArgs& a, int num_cus, hipStream_t st) {
  hipLaunchKernelGGL(k_tail_norm_quant, dim3(a.T), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T <= kTailGemvMaxT) {
    const int ks_n = tail_gemv_slices(a.latent);
    if (a.wcanon)
      hipLaunchKernelGGL(k_tail_gemv<true>, dim3(a.hidden / 64, ks_n), dim3(256), 0, st, a, a.part, ks_n);
    else
      hipLaunchKernelGGL(k_tail_gemv<false>, dim3(a.hidden / 64, ks_n), dim3(256), 0, st, a, a.part, ks_n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(a.T) * a.hidden / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, int64_t(num_cus) * 4);
    hipLaunchKernelGGL(k_tail_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a.part, ks_n,
                       a.s, a.y, n4);
    return hipGetLastError();
  }
  // the projection: the down-GEMM kernels with one expert, K = latent,
  // N = hidden, rows in token order
  FwdArgs f{};
  f.T = a.T;
  f.d = a.hidden;
  f.dff = a.latent;
  f.E = 1;
  f.k = 1;
  f.S = 0;
  f.Rr = f.R = a.T;
  f.dn_c = a.up_c;
  f.dn_s = a.up_s;
  f.h_codes = a.codes;
  f.h_scales = a.scales;
  f.o16 = a.o16;
  f.row_src = a.row_src;
  f.tiles = a.tiles;
  f.tile_count = a.tile_count;
  f.ex_tiles = a.ex_tiles;
  f.bm = a.bm;
  f.wcanon = a.wcanon;
  f.num_cus = num_cus;
  f.max_tiles = (a.T + a.bm - 1) / a.bm;
  // few tiles: K slices into fp32 partials, summed in order with s
  const int ks = a.bm > kDecodeMaxRows ? tail_ksplit(a.T, a.latent, a.hidden, a.bm) : 1;
  if (ks > 1) {
    f.ksplit = ks;
    f.kpart = a.part;
    e = launch_gemm_down(f, st);
    if (e != hipSuccess) return e;
    const int64_t n4 = int64_t(a.T) * a.hidden / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, int64_t(num_cus) * 4);
    hipLaunchKernelGGL(k_tail_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a.part, ks,
                       a.s, a.y, n4);
    return hipGetLastError();
  }
  e = launch_gemm_down(f, st);
  if (e != hipSuccess || !a.s) return e;
  const int64_t n8 = int64_t(a.T) * a.hidden / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, int64_t(num_cus) * 8);
  hipLaunchKernelGGL(k_tail_add, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a.o16, a.s, a.y, n8);
  return hipGetLastError();
}

}  // namespace mxmoe
