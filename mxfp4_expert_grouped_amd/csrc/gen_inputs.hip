// GPU twin of the seeded input generator: the MXFP4 expert weights of a
// synthetic layer drawn directly as codes and scales from Philox4x64-10
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC'11).  Holds none of the layer's arithmetic; the recipe is the one of the
// numpy generator, which this must reproduce byte for byte:
//   element byte r: sign = r >> 7, magnitude code from 128 equiprobable slots
//   (10, 20, 19, 16, 20, 18, 16, 9 slots for codes 0..7);
//   block scale byte r: 127 + e_base + (1 if (r & 7) >= 6 else 0).
// Block b of a matrix takes the 32 bytes of counter b under the code key; the
// scales of blocks 32c..32c+31 take the 32 bytes of counter c under the scale key.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 { uint64_t x[4]; };

__device__ __forceinline__ U4 philox4x64_10(uint64_t k0, uint64_t k1, uint64_t c0, uint64_t c1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = c0, x1 = c1, x2 = 0, x3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
    uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
    uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
  }
  U4 o; o.x[0] = x0; o.x[1] = x1; o.x[2] = x2; o.x[3] = x3;
  return o;
}

__device__ __forceinline__ uint32_t mag_code(uint32_t r7) {
  return (r7 >= 10) + (r7 >= 30) + (r7 >= 49) + (r7 >= 65) + (r7 >= 85) + (r7 >= 103) + (r7 >= 119);
}

__global__ void k_gen_codes(uint8_t* __restrict__ codes, int64_t nblocks, uint64_t seed, uint64_t stream) {
  for (int64_t b = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; b < nblocks; b += int64_t(gridDim.x) * blockDim.x) {
    U4 r = philox4x64_10(seed, stream, static_cast<uint64_t>(b), 0);
    uint32_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint64_t v = r.x[w];
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // bytes 2i, 2i+1 of this word -> one output byte
        uint32_t b0 = (v >> (16 * i)) & 0xFF, b1 = (v >> (16 * i + 8)) & 0xFF;
        uint32_t c0 = mag_code(b0 & 0x7F) | ((b0 >> 7) << 3);
        uint32_t c1 = mag_code(b1 & 0x7F) | ((b1 >> 7) << 3);
        packed |= (c0 | (c1 << 4)) << (8 * i);
      }
      out[w] = packed;
    }
    reinterpret_cast<uint4*>(codes)[b] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__global__ void k_gen_scales(uint8_t* __restrict__ scales, int64_t nblocks, uint64_t seed, uint64_t stream, int e_base) {
  const int64_t ncalls = (nblocks + 31) / 32;
  for (int64_t c = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; c < ncalls; c += int64_t(gridDim.x) * blockDim.x) {
    U4 r = philox4x64_10(seed, stream, static_cast<uint64_t>(c), 0);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      int64_t b = c * 32 + j;
      if (b < nblocks) {
        uint32_t byte = (r.x[j / 8] >> (8 * (j % 8))) & 0xFF;
        scales[b] = static_cast<uint8_t>(127 + e_base + ((byte & 7) >= 6 ? 1 : 0));
      }
    }
  }
}

}  // namespace

extern "C" int mxmoe_gen_mx_matrix(uint8_t* codes, uint8_t* scales, int64_t rows, int64_t k,
                                   uint64_t seed, uint64_t code_stream, uint64_t scale_stream,
                                   int e_base, void* stream) {
  if (!codes || !scales || rows <= 0 || k <= 0 || k % 32) return 1;
  if (reinterpret_cast<uintptr_t>(codes) % 16) return 1;
  const int64_t nblocks = rows * (k / 32);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int64_t g1 = (nblocks + 255) / 256; if (g1 > 65536) g1 = 65536;
  int64_t g2 = ((nblocks + 31) / 32 + 255) / 256; if (g2 > 65536) g2 = 65536; if (g2 < 1) g2 = 1;
  hipLaunchKernelGGL(k_gen_codes, dim3(g1), dim3(256), 0, st, codes, nblocks, seed, code_stream);
  hipLaunchKernelGGL(k_gen_scales, dim3(g2), dim3(256), 0, st, scales, nblocks, seed, scale_stream, e_base);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
