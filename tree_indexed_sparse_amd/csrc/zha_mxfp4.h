// MXFP4 encoding on the GPU (OCP Microscaling Formats v1.0): blocks of 32 elements, E2M1
// elements (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5,
// 2, 3, 4, 6) and one E8M0 scale byte per block (2^(byte - 127)). Used by the router
// encoder and by the FP4 scoring kernels, which quantise the query the same way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zha {

constexpr int kMxBlock = 32;

// E8M0 byte of a block whose largest magnitude is amax: X + 127 with
// X = floor(log2 amax) - 2 (2 = exponent of the largest E2M1 value, 6 = 1.5 * 2^2), read
// from the float's biased exponent e (floor(log2 amax) = e - 127 for a normal float), and
// clamped to X >= -127 (zero and subnormal blocks included). A float's exponent keeps
// X <= 125.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return (uint32_t)(e > 2 ? e - 2 : 0);
}

// 2^-X for an E8M0 byte (X = byte - 127, -127 <= X <= 125): a normal float, so scaling by
// it is exact for every normal input.
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// E2M1 codes of x / 2^X for eight consecutive elements, packed into one word (element i
// in bits 4i .. 4i + 3). x * 2^-X is exact; v_cvt_scalef32_pk_fp4_f32 (scale 1) then
// rounds it to the nearest E2M1 value with ties to the even mantissa, saturates at +-6
// and keeps the sign (zeros included): the format's rounding, checked against the
// definition on every tie and on both sides of the clamp.
__device__ __forceinline__ uint32_t e2m1_pack(const float* x, int n, float inv) {
  uint32_t w = 0;
  if (n > 0) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * inv, x[1] * inv, 1.0f, 0);
  if (n > 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * inv, x[3] * inv, 1.0f, 1);
  if (n > 4) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * inv, x[5] * inv, 1.0f, 2);
  if (n > 6) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * inv, x[7] * inv, 1.0f, 3);
  return w;
}
__device__ __forceinline__ uint32_t e2m1_pack8(const float (&x)[8], float inv) {
  return e2m1_pack(x, 8, inv);
}

// One whole block held by one lane: 32 values -> 16 code bytes (uint4) and the scale byte.
__device__ __forceinline__ uint4 mx_encode_block(const float (&x)[kMxBlock], uint32_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const uint32_t sb = mx_scale_byte(amax);
  const float inv = mx_inv_scale(sb);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[8 * j + i];
    w[j] = e2m1_pack8(v, inv);
  }
  *scale = sb;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace zha
