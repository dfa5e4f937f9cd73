// Conversion of canonical MXFP4 matrices into the packed tile order read by
// the grouped GEMMs (layout documented with moe_pack_mx4): the four 16-row x
// 128-wide MFMA operands of a 64-row group and K step become 4 KB contiguous
// in lane order, and their block scales one dword per lane (one byte per
// 16-row block).  With `interleave`, group G holds rows 32G .. 32G+31 of the
// first half of the matrix and the same rows of the second half (gate and up
// rows of the same outputs).  Pure byte movement, done once when the weights
// are loaded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mxmoe {

// canonical row of block j (0..3), row r (0..15) of 64-row group G
__device__ __forceinline__ int64_t packed_row(int64_t G, int j, int r, int64_t rows, int interleave) {
  if (!interleave) return 64 * G + 16 * j + r;
  return (j >> 1) * (rows / 2) + 32 * G + 16 * (j & 1) + r;
}

__global__ void __launch_bounds__(256) k_pack_codes(const uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ codes_p, int64_t mats,
                                                    int64_t rows, int64_t k, int interleave) {
  const int64_t nsteps = k / 128, ngrp = rows / 64;
  const int64_t total = mats * ngrp * nsteps * 4 * 64;  // one 16-byte entry per thread
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int l = static_cast<int>(i & 63);
    int64_t t = i >> 6;
    const int j = static_cast<int>(t & 3);
    t >>= 2;
    const int64_t s = t % nsteps;
    t /= nsteps;
    const int64_t G = t % ngrp, m = t / ngrp;
    const int g = l >> 4, r = l & 15;
    const uint8_t* src = codes + (m * rows + packed_row(G, j, r, rows, interleave)) * (k / 2) + 64 * s + 16 * g;
    reinterpret_cast<uint4*>(codes_p)[i] = *reinterpret_cast<const uint4*>(src);
  }
}

__global__ void __launch_bounds__(256) k_pack_scales(const uint8_t* __restrict__ scales,
                                                     uint8_t* __restrict__ scales_p, int64_t mats,
                                                     int64_t rows, int64_t k, int interleave) {
  const int64_t nb = k / 32, nsteps = k / 128, ngrp = rows / 64;
  const int64_t total = mats * ngrp * nsteps * 64;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int l = static_cast<int>(i & 63);
    int64_t t = i >> 6;
    const int64_t s = t % nsteps;
    t /= nsteps;
    const int64_t G = t % ngrp, m = t / ngrp;
    const int g = l >> 4, r = l & 15;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w |= uint32_t(scales[(m * rows + packed_row(G, j, r, rows, interleave)) * nb + 4 * s + g]) << (8 * j);
    reinterpret_cast<uint32_t*>(scales_p)[i] = w;
  }
}

hipError_t launch_pack_mx4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int64_t rows,
                           int64_t k, int interleave, uint8_t* codes_p, uint8_t* scales_p,
                           hipStream_t st) {
  const int64_t n1 = mats * (rows / 64) * (k / 128) * 4 * 64;
  const int64_t n2 = mats * (rows / 64) * (k / 128) * 64;
  const int64_t g1 = n1 / 256 + 1 > 65536 ? 65536 : n1 / 256 + 1;
  const int64_t g2 = n2 / 256 + 1 > 65536 ? 65536 : n2 / 256 + 1;
  hipLaunchKernelGGL(k_pack_codes, dim3(g1), dim3(256), 0, st, codes, codes_p, mats, rows, k, interleave);
  hipLaunchKernelGGL(k_pack_scales, dim3(g2), dim3(256), 0, st, scales, scales_p, mats, rows, k, interleave);
  return hipGetLastError();
}

}  // namespace mxmoe
