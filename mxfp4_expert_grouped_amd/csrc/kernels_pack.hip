// Conversion of canonical MXFP4 matrices into the packed tile order read by
// the grouped GEMMs (layout documented with moe_pack_mx4): one 16-row x
// 128-wide MFMA step becomes 1 KB contiguous in lane order, the block scales
// one dword per lane per four steps.  Pure byte movement, done once when the
// weights are loaded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace mxmoe {

__global__ void __launch_bounds__(256) k_pack_codes(const uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ codes_p, int64_t mats,
                                                    int64_t rows, int64_t k) {
  const int64_t nsteps = k / 128, nblk = rows / 16;
  const int64_t total = mats * nblk * nsteps * 64;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int l = static_cast<int>(i & 63);
    int64_t t = i >> 6;
    const int64_t s = t % nsteps;
    t /= nsteps;
    const int64_t b = t % nblk, m = t / nblk;
    const int g = l >> 4, r = l & 15;
    const uint8_t* src = codes + (m * rows + 16 * b + r) * (k / 2) + 64 * s + 16 * g;
    reinterpret_cast<uint4*>(codes_p)[i] = *reinterpret_cast<const uint4*>(src);
  }
}

__global__ void __launch_bounds__(256) k_pack_scales(const uint8_t* __restrict__ scales,
                                                     uint8_t* __restrict__ scales_p, int64_t mats,
                                                     int64_t rows, int64_t k) {
  const int64_t nb = k / 32, nq = (k + 511) / 512, nblk = rows / 16;
  const int64_t total = mats * nblk * nq * 64;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int l = static_cast<int>(i & 63);
    int64_t t = i >> 6;
    const int64_t q = t % nq;
    t /= nq;
    const int64_t b = t % nblk, m = t / nblk;
    const int g = l >> 4, r = l & 15;
    const uint8_t* row = scales + (m * rows + 16 * b + r) * nb;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t blk = 16 * q + 4 * j + g;
      if (blk < nb) w |= uint32_t(row[blk]) << (8 * j);
    }
    reinterpret_cast<uint32_t*>(scales_p)[i] = w;
  }
}

hipError_t launch_pack_mx4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int64_t rows,
                           int64_t k, uint8_t* codes_p, uint8_t* scales_p, hipStream_t st) {
  const int64_t n1 = mats * (rows / 16) * (k / 128) * 64;
  const int64_t n2 = mats * (rows / 16) * ((k + 511) / 512) * 64;
  const int64_t g1 = n1 / 256 + 1 > 65536 ? 65536 : n1 / 256 + 1;
  const int64_t g2 = n2 / 256 + 1 > 65536 ? 65536 : n2 / 256 + 1;
  hipLaunchKernelGGL(k_pack_codes, dim3(g1), dim3(256), 0, st, codes, codes_p, mats, rows, k);
  hipLaunchKernelGGL(k_pack_scales, dim3(g2), dim3(256), 0, st, scales, scales_p, mats, rows, k);
  return hipGetLastError();
}

}  // namespace mxmoe
