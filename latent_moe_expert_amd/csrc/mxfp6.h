// MXFP6 (E2M3) activation encoding used as the A operand of the scaled MFMA.
//
// Why: gfx950's scaled MFMA multiplies an FP6 operand by an FP4 operand at the
// FP4 rate, while FP8 x FP4 runs at the (half) FP8 rate. One E2M3 plane keeps
// only 4 significant bits, so each group of 32 activations is carried as two
// planes: hi = E2M3(v / X_hi) and lo = E2M3((v - hi * X_hi) / X_lo), each with
// its own E8M0 scale. The two MFMAs (hi and lo against the same weights) sum to
// about 8 significant bits, the precision of the bf16 activations they replace.
//
// Scale rule (OCP MX v1.0, section 6.3): X = 2^(floor(log2(amax)) - 2), where
// 2 is the exponent of E2M3's largest normal (7.5 = 1.875 * 2^2); codes round to
// nearest even and saturate at 7.5.
//
// E2M3 code (6 bits): sign (bit 5), exponent (bits 4:3, bias 1), mantissa (2:0):
// exponent 0 -> m/8, else (1 + m/8) * 2^(e-1). Magnitude codes are monotonic, so
// for |y| < 2 the code is rint(8|y|), for [2, 4) rint(4|y|) + 8, for [4, 7.5]
// rint(2|y|) + 16.
//
// Packed layout of a group: 32 codes in 24 bytes, code i at bits [6i, 6i+6)
// (little endian), which is the register layout the MFMA reads.
//
// Tensor layout (rows of K values, K a multiple of 512; a window is 16 groups):
//   data   [row][K/128 steps][plane hi|lo][4][24 B]: step k, slot q holds group 4k + q
//   scales [row][K/512 windows][plane hi|lo][4][4 B]: window w, dword q, byte s is the
//          scale of group 16w + 4s + q
// so MFMA lane group q of k-step 4w + s finds its 24 bytes contiguously, and its
// four scales of the window as one aligned dword (byte s for k-step s).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kFp6StepBytes = 192;   // one k-step (128 values) of one row: hi 96 B + lo 96 B
constexpr int kFp6WindowScaleBytes = 32;

__host__ __device__ constexpr size_t fp6_row_bytes(int K) { return (size_t)K * 3 / 2; }
__host__ __device__ constexpr size_t fp6_scale_row_bytes(int K) { return (size_t)K / 16; }

// Scale code (E8M0) of a group with max magnitude `amax`, and 1/X as fp32.
__device__ __forceinline__ uint32_t fp6_scale_code(float amax, float& inv) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // biased exponent, 0 for zero/subnormal
  int code = e - 2;                                           // 2^(floor(log2 amax) - 2), biased
  code = code < 0 ? 0 : code;                                 // amax < 2^-125: values quantize at 2^-127
  inv = __uint_as_float((uint32_t)(254 - code) << 23);        // exact power of two, code <= 253
  return (uint32_t)code;
}

// Round y (already divided by the scale) to E2M3: returns the 6-bit code and the
// value of the code (in units of the scale). Branch-free (lanes of a wave round
// values of different binades): binade e = [t >= 2] + [t >= 4] has spacing 2^(e-3)
// and code offset 8e.
__device__ __forceinline__ uint32_t e2m3_round(float y, float& qv) {
  const float t = fminf(fabsf(y), 7.5f);
  const bool b2 = t >= 2.f, b4 = t >= 4.f;
  const float f = b4 ? 2.f : (b2 ? 4.f : 8.f);
  const float inv = b4 ? 0.5f : (b2 ? 0.25f : 0.125f);
  const uint32_t off = b4 ? 16u : (b2 ? 8u : 0u);
  const float r = rintf(t * f);
  const uint32_t sign = y < 0.f ? 0x80000000u : 0u;
  qv = __uint_as_float(__float_as_uint(r * inv) | sign);
  return ((uint32_t)r + off) | (sign >> 26);
}

// Pack 32 six-bit codes into 6 dwords (code i at bits [6i, 6i+6)).
__device__ __forceinline__ void pack_fp6x32(const uint32_t c[32], uint32_t w[6]) {
#pragma unroll
  for (int j = 0; j < 6; ++j) w[j] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int bit = 6 * i, wi = bit >> 5, sh = bit & 31;
    w[wi] |= c[i] << sh;
    if (sh > 26) w[wi + 1] |= c[i] >> (32 - sh);
  }
}

// Encode one group of 32 values into hi and lo planes (6 dwords each) and their scale codes.
__device__ __forceinline__ void fp6_encode_group(const float v[32], uint32_t hi[6], uint32_t lo[6], uint32_t& s_hi,
                                                 uint32_t& s_lo) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float inv;
  s_hi = fp6_scale_code(amax, inv);
  const float x_hi = __uint_as_float(s_hi ? (s_hi << 23) : 0x00400000u);  // 2^(s_hi - 127)
  uint32_t c[32];
  float r[32];
  float ramax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float qv;
    c[i] = e2m3_round(v[i] * inv, qv);
    r[i] = v[i] - qv * x_hi;  // exact: qv * x_hi and v[i] are within a factor of two or qv = 0
    ramax = fmaxf(ramax, fabsf(r[i]));
  }
  pack_fp6x32(c, hi);
  s_lo = fp6_scale_code(ramax, inv);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float qv;
    c[i] = e2m3_round(r[i] * inv, qv);
  }
  pack_fp6x32(c, lo);
}

// Byte offsets of group g of a row inside the data and scale rows.
__device__ __forceinline__ uint32_t fp6_data_offset(int g, int plane) {
  return (uint32_t)((g >> 2) * kFp6StepBytes + plane * 96 + (g & 3) * 24);
}
__device__ __forceinline__ uint32_t fp6_scale_offset(int g, int plane) {
  const int w = g >> 4, s = (g >> 2) & 3, q = g & 3;
  return (uint32_t)(w * kFp6WindowScaleBytes + plane * 16 + q * 4 + s);
}

}  // namespace moe
