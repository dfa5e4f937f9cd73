// GPU twin of the seeded input generator: the MXFP4 expert weights of a
// synthetic layer, N(0, sigma) samples quantised to MXFP4 block by block,
// from Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC'11).  Holds none of the layer's arithmetic; the
// recipe is the one of the numpy generator, which this must reproduce byte
// for byte:
//   block b (32 consecutive elements of a row) takes the 64 bytes of counters
//   2b and 2b+1 under the matrix's key as 32 little-endian 16-bit uniforms u;
//   x = table[u] * sigma in float32 (table: the standard normal quantile at
//   (u + 1/2) / 65536, supplied by the caller);
//   e = floor(log2(max |x|)) - 2 (kept in [-126, 125]; all-zero blocks -127),
//   scale byte e + 127; element code = the E2M1 value nearest |x| / 2^e
//   (ties to the even code, saturating at 6), sign bit x < 0.
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

// E2M1 code of a = |x| / 2^e >= 0: the boundaries 0.25, 1.25, 2.5 and 5 go
// down, 0.75, 1.75 and 3.5 up (to the even mantissa)
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
}

// one thread per 32-element block
__global__ void k_gen_mx(uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t nblocks,
                         uint64_t seed, uint64_t stream, const float* __restrict__ table, float sigma) {
  for (int64_t b = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; b < nblocks; b += int64_t(gridDim.x) * blockDim.x) {
    const U4 r0 = philox4x64_10(seed, stream, 2 * static_cast<uint64_t>(b), 0);
    const U4 r1 = philox4x64_10(seed, stream, 2 * static_cast<uint64_t>(b) + 1, 0);
    float x[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint64_t w = i < 16 ? r0.x[i / 4] : r1.x[(i - 16) / 4];
      const uint32_t u = static_cast<uint32_t>(w >> (16 * (i % 4))) & 0xFFFFu;
      x[i] = __fmul_rn(table[u], sigma);
      amax = fmaxf(amax, fabsf(x[i]));
    }
    int e = -127;
    float inv = 1.0f;
    if (amax != 0.0f) {
      const int eb = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
      e = min(max(eb - 129, -126), 125);
      inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);   // 2^-e, exact
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = e2m1_code(__fmul_rn(fabsf(x[i]), inv)) | (x[i] < 0.0f ? 8u : 0u);
      out[i / 8] |= c << (4 * (i % 8));
    }
    reinterpret_cast<uint4*>(codes)[b] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = static_cast<uint8_t>(e + 127);
  }
}

}  // namespace

// codes [rows, k/2] (16-byte aligned), scales [rows, k/32]; table: 65536
// float32 on the device; returns 0, 1 (bad argument) or 2 (launch error)
extern "C" int mxmoe_gen_mx_matrix(uint8_t* codes, uint8_t* scales, int64_t rows, int64_t k,
                                   uint64_t seed, uint64_t code_stream, const float* table, float sigma,
                                   void* stream) {
  if (!codes || !scales || !table || rows <= 0 || k <= 0 || k % 32) return 1;
  if (reinterpret_cast<uintptr_t>(codes) % 16) return 1;
  const int64_t nblocks = rows * (k / 32);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int64_t g = (nblocks + 255) / 256; if (g > 65536) g = 65536;
  hipLaunchKernelGGL(k_gen_mx, dim3(g), dim3(256), 0, st, codes, scales, nblocks, seed, code_stream, table, sigma);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
