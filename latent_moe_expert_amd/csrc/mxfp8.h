// MXFP8 activations of the routed experts (K3 report review, quantization-aware
// training section: MXFP4 weights with MXFP8 input activations; shared experts,
// projections and router stay at higher precision).
//
// Element E4M3 (OCP 8-bit floating point): sign, 4 exponent bits (bias 7), 3
// mantissa bits, no infinities, largest magnitude 1.75 * 2^8 = 448, subnormals
// m/8 * 2^-6. Block: 32 consecutive values share an E8M0 scale X = 2^s with
// s = floor(log2 amax) - 8 (8 = exponent of E4M3's largest normal), kept in
// [-126, 127]; each value becomes the E4M3 value nearest to v / X, ties to the
// even mantissa, magnitudes past 448 saturating to 448 (OCP Microscaling v1.0).
//
// Tensor layout on the scaled-MFMA path (rows of K values, K a multiple of 512):
//   data   [row][K] E4M3 codes in K order (k-step k = bytes 128k .. 128k+127; its
//          E8M0 group 4k + q = bytes 128k + 32q .. +31)
//   scales [row][K/512 windows][4][4 B]: window w, dword q, byte s is the scale of
//          group 16w + 4s + q, so MFMA lane group q, which supplies the scale of K
//          block q of a k-step, finds its four scales of the window in one dword (byte
//          s for k-step 4w + s).
// The data rows of h (the down contraction's input) are stored tiled instead
// (atile_offset in mxfp6.h); the bytes of each row are the same.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kFp8WindowScaleBytes = 16;

__host__ __device__ constexpr size_t fp8_row_bytes(int K) { return (size_t)K; }
__host__ __device__ constexpr size_t fp8_scale_row_bytes(int K) { return (size_t)K / 32; }

// Block scale exponent s of a block whose largest magnitude is amax (amax >= 0).
__device__ __forceinline__ int mxfp8_scale_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // 0 for zero and subnormals
  const int s = ef - 127 - 8;
  return ef == 0 ? -126 : (s < -126 ? -126 : s);
}

// Nearest E4M3 value to y (magnitude clamped to 448), as a float; ties to even.
__device__ __forceinline__ float e4m3_round(float y) {
  const float a = fminf(fabsf(y), 448.f);
  float r;
  if (a < 0.015625f) {  // below 2^-6: the subnormal quantum 2^-9 (8 * 2^-9 is the smallest normal)
    r = rintf(a * 512.f) * (1.f / 512.f);
  } else {  // round the 23-bit significand to 3 bits, ties to even
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    r = __uint_as_float(b & 0xfff00000u);
  }
  return copysignf(r, y);
}

// E4M3 code of the nearest value to y (magnitude clamped to 448); ties to even.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);  // 0..8; 8 is the code of 2^-6
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    const int e = (int)(b >> 23) - 127;  // -6..8
    code = ((uint32_t)(e + 7) << 3) | ((b >> 20) & 7u);
  }
  return sign | code;
}

// One block of 32 values: E4M3 codes (byte i of the 8 dwords = value i) and the E8M0 code.
__device__ __forceinline__ void mxfp8_encode_group(const float v[32], uint32_t codes[8], uint32_t& scale_code) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int s = mxfp8_scale_exp(amax);
  scale_code = (uint32_t)(s + 127);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) w |= e4m3_code(ldexpf(v[4 * j + b], -s)) << (8 * b);
    codes[j] = w;
  }
}

// Byte offset of the scale of group g inside a scale row.
__device__ __forceinline__ uint32_t fp8_scale_offset(int g) {
  const int w = g >> 4, s = (g >> 2) & 3, q = g & 3;
  return (uint32_t)(w * kFp8WindowScaleBytes + q * 4 + s);
}

}  // namespace moe
