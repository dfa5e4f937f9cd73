// Device-side helpers for the MX formats and wavefront reductions (gfx950).
//
// Formats (OCP Microscaling v1.0, the encodings behind the "MXFP4 weights,
// MXFP8 activations" of the Kimi K3 pages):
//   E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa; max finite 448.
//   E8M0 scale : 2^(k-127).
// Quantisation of a block of 32 values: e = clamp(floor(log2 amax) - 8,
// -127, 127) (amax == 0 -> -127); element code = round-to-nearest-even of
// v * 2^-e on the E4M3 grid, saturated to +-448, sign kept on zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

constexpr int kWave = 64;

// floor(log2 |a|) of a finite float, subnormals included; |a| == 0 -> -150.
__device__ __forceinline__ int floor_log2_f32(float a) {
  uint32_t u = __float_as_uint(a) & 0x7fffffffu;
  int ef = static_cast<int>(u >> 23);
  if (ef > 0) return ef - 127;
  return (u == 0) ? -150 : (31 - __clz(u)) - 149;
}

// Shared exponent of an MXFP8 block from its largest magnitude.
__device__ __forceinline__ int mx8_block_exp(float amax) {
  int e = floor_log2_f32(amax) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^n as a float for n in [-126, 127] (normal range).
__device__ __forceinline__ float exp2_int(int n) {
  return __uint_as_float(static_cast<uint32_t>(n + 127) << 23);
}

// E4M3 code (round-to-nearest-even, saturating to +-448, sign kept, OCP MX
// v1.0) from the conversion instruction: V_CVT_PK_FP8_F32 rounds to nearest
// even and keeps denormals, so with its input clamped to +-448 it gives that
// code for every finite float (compared over all 2^32 bit patterns with a
// bit-level encoder written from the format definition; the bit-exact
// quantiser tests against the oracle cover midpoints, saturation, subnormal
// inputs and signed zeros).  Two values per instruction: bytes 0 and 1.
__device__ __forceinline__ uint32_t e4m3_cvt2(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xFFFFu;
}
// four codes in one dword, byte i from value i
__device__ __forceinline__ uint32_t e4m3_cvt4(float a, float b, float c, float d) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  const float cc = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  const float cd = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, lo, true));
}

// fp32 -> bf16, round to nearest even (finite values)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Reductions across the lanes of a wave (or of aligned lane groups).
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}

// Order-preserving map of a float to an unsigned key (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace mxmoe
