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
__global__ void __launch_bounds__(256) k_tail_norm_quant(TailArgs a) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l = a.latent;
  const float4* z4 = reinterpret_cast<const float4*>(a.z + int64_t(t) * l);
  const int n4 = l / 4;
  float ss = 0.f;
  for (int i = tid; i < n4; i += 256) {
    const float4 v = z4[i];
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
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
  // pass 2: 8 threads per block, 32 blocks per sweep of the workgroup
  const float4* g4 = reinterpret_cast<const float4*>(a.gamma);
  const int nb = l / 32;
  for (int b0 = 0; b0 < nb; b0 += 32) {
    const int b = b0 + (tid >> 3), j = tid & 7;
    const bool ok = b < nb;                         // the same for the 8 threads of a block
    const int i4 = ok ? b * 8 + j : 0;
    const float4 v = z4[i4], g = g4[i4];
    float q[4] = {v.x * inv * g.x, v.y * inv * g.y, v.z * inv * g.z, v.w * inv * g.w};
    const float amax = group_max<8>(fmaxf(fmaxf(fabsf(q[0]), fabsf(q[1])), fmaxf(fabsf(q[2]), fabsf(q[3]))));
    const int e = mx8_block_exp(amax);
    const float sc = exp2_int(-e);
    const uint32_t w = e4m3_cvt4(q[0] * sc, q[1] * sc, q[2] * sc, q[3] * sc);
    if (ok) {
      *reinterpret_cast<uint32_t*>(a.codes + int64_t(t) * l + 32 * b + 4 * j) = w;
      if (j == 0) a.scales[int64_t(t) * nb + b] = static_cast<uint8_t>(e + 127);
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

hipError_t launch_tail(const TailArgs& a, int num_cus, hipStream_t st) {
  hipLaunchKernelGGL(k_tail_norm_quant, dim3(a.T), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
  f.num_cus = num_cus;
  f.max_tiles = (a.T + a.bm - 1) / a.bm;
  e = launch_gemm_down(f, st);
  if (e != hipSuccess || !a.s) return e;
  const int64_t n8 = int64_t(a.T) * a.hidden / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, int64_t(num_cus) * 8);
  hipLaunchKernelGGL(k_tail_add, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a.o16, a.s, a.y, n8);
  return hipGetLastError();
}

}  // namespace mxmoe
