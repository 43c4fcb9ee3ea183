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
// nearest even and saturate at 7.5 (gfx950's scaled conversion instructions do both).
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
//   data   [row][K/128 steps][4][plane hi|lo][24 B]: step k, slot q holds group 4k + q
//   scales [row][K/512 windows][plane hi|lo][4][4 B]: window w, dword q, byte s is the
//          scale of group 16w + 4s + q
// so MFMA lane group q of k-step 4w + s finds both planes of its group as 48
// contiguous, 16-byte aligned bytes (three 16-byte chunks fill the two operands),
// and its four scales of the window as one aligned dword (byte s for k-step s).
// The scales are stored row after row; the data rows are stored row after row (gate/up
// inputs) or tiled (atile_offset; h, the down contraction's input).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kFp6StepBytes = 192;   // one k-step (128 values) of one row: 4 groups x (hi 24 B + lo 24 B)
constexpr int kFp6WindowScaleBytes = 32;

__host__ __device__ constexpr size_t fp6_row_bytes(int K) { return (size_t)K * 3 / 2; }
__host__ __device__ constexpr size_t fp6_scale_row_bytes(int K) { return (size_t)K / 16; }

// Tiled layout of the contraction's A data (FP6 hi/lo or MXFP8 rows alike). Rows come in
// tiles of 16, and inside a tile the rows' bytes are stored chunk-major: 16-byte chunk c of
// the 16 rows, then chunk c + 1. Byte b of row r of a tensor of row_bytes bytes per row is at
//   (r / 16) * 16 * row_bytes + (b / 16) * 256 + (r % 16) * 16 + b % 16.
// One k-step of a tile is then one contiguous block (LDS-DMA moves it unchanged, 1 KB per
// instruction), and the 16 lanes of an MFMA lane group, which read one chunk of 16 rows,
// read 256 contiguous bytes of LDS. A tiled tensor holds a multiple of 16 rows.
__host__ __device__ inline size_t atile_offset(size_t r, size_t b, size_t row_bytes) {
  return (r >> 4) * 16 * row_bytes + (b >> 4) * 256 + (r & 15) * 16 + (b & 15);
}

typedef __attribute__((ext_vector_type(16))) float fp6_f32x16_t;
typedef __attribute__((ext_vector_type(32))) float fp6_f32x32_t;
typedef __attribute__((ext_vector_type(6))) unsigned fp6_u32x6_t;

// Scale code (E8M0) of a group with max magnitude `amax`: 2^(floor(log2 amax) - 2), at
// least 2^-126 (code 1) so that the scale is a normal float (a group whose magnitudes are
// all below 2^-125 is encoded on the 2^-126 grid).
__device__ __forceinline__ uint32_t fp6_scale_code(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // biased exponent, 0 for zero/subnormal
  const int code = e - 2;
  return (uint32_t)(code < 1 ? 1 : code);
}
__device__ __forceinline__ float e8m0_value(uint32_t code) { return __uint_as_float(code << 23); }  // code >= 1

// The two packing conversions, as inline asm with early-clobber outputs: no register of the
// result may also hold an operand. The builtins leave that to the register allocator, which
// may give the 6-dword result of the 2 x 16-value conversion registers inside a source operand.
// Where they start at the same register the results were right, but a result placed four
// registers into the second source (v[6:11] against v[2:17]) gave wrong codes: the
// instruction writes its first result dwords before it has read the rest of that source.
__device__ __forceinline__ fp6_u32x6_t fp6_cvt_2xpk16(fp6_f32x16_t even, fp6_f32x16_t odd, float scale) {
  fp6_u32x6_t r;
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(r) : "v"(even), "v"(odd), "v"(scale));
  return r;
}
__device__ __forceinline__ fp6_f32x32_t fp6_cvt_pk32_to_f32(fp6_u32x6_t codes, float scale) {
  fp6_f32x32_t r;
  asm("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(r) : "v"(codes), "v"(scale));
  return r;
}

// Encode one group of 32 values into hi and lo planes (6 dwords each) and their scale
// codes. v_cvt_scalef32_2xpk16_fp6_f32 rounds x / scale to E2M3 (nearest even, saturating
// at 7.5) and packs src0[j] at code position 2j and src1[j] at 2j + 1;
// v_cvt_scalef32_pk32_f32_fp6 returns code value * scale in position order. Feeding the
// even- and odd-indexed values puts value i at position i.
__device__ __forceinline__ void fp6_encode_group(const float v[32], uint32_t hi[6], uint32_t lo[6], uint32_t& s_hi,
                                                 uint32_t& s_lo) {
  fp6_f32x16_t ev, od;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ev[i] = v[2 * i];
    od[i] = v[2 * i + 1];
    amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  s_hi = fp6_scale_code(amax);
  const float x_hi = e8m0_value(s_hi);
  const fp6_u32x6_t h = fp6_cvt_2xpk16(ev, od, x_hi);
  const fp6_f32x32_t q = fp6_cvt_pk32_to_f32(h, x_hi);
  float ramax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // exact: v and its hi value are within a factor of two of each other, or the hi value is 0
    ev[i] = v[2 * i] - q[2 * i];
    od[i] = v[2 * i + 1] - q[2 * i + 1];
    ramax = fmaxf(ramax, fmaxf(fabsf(ev[i]), fabsf(od[i])));
  }
  s_lo = fp6_scale_code(ramax);
  const fp6_u32x6_t l = fp6_cvt_2xpk16(ev, od, e8m0_value(s_lo));
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    hi[j] = h[j];
    lo[j] = l[j];
  }
}

// Byte offsets of group g of a row inside the data and scale rows.
__device__ __forceinline__ uint32_t fp6_data_offset(int g, int plane) {
  return (uint32_t)((g >> 2) * kFp6StepBytes + (g & 3) * 48 + plane * 24);
}
__device__ __forceinline__ uint32_t fp6_scale_offset(int g, int plane) {
  const int w = g >> 4, s = (g >> 2) & 3, q = g & 3;
  return (uint32_t)(w * kFp6WindowScaleBytes + plane * 16 + q * 4 + s);
}

}  // namespace moe
