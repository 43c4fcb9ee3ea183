// Device helpers shared by the latent-MoE kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

#define MOE_WAVE 64

// bf16 is carried as raw uint16 bit patterns outside the MFMA operands.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Eight MXFP4 elements (one 32-bit word, element 2j in the low nibble of byte j)
// to eight bf16 values times the E8M0 scale. The conversion instruction takes the
// scale from the exponent field of its fp32 operand, so `scale_as_f32` is the raw
// E8M0 code shifted into that field (exact for every code, 255 gives NaN).
// Returns 4 dwords, each two bf16 (lower element in the low half).
__device__ __forceinline__ void fp4x8_to_bf16x8(uint32_t w, float scale_as_f32, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_as_f32, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_as_f32, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_as_f32, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale_as_f32, 3));
}

__device__ __forceinline__ float e8m0_as_f32_exponent(uint32_t code) { return __uint_as_float(code << 23); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// GLU activation of the experts, chosen per launch problem:
//   kGluSilu: SiLU(gate) * up
//   kGluSitu: SiTU, b1 * tanh(SiLU(gate) / b1) * b2 * tanh(up / b2) -- the sigmoid branch and
//             the linear branch each soft-limited by beta * tanh(z / beta) (K3 report review,
//             "SiTU-GLU"; betas 4 and 25 in the K3 configuration, WASTE "Kimi K3, as
//             released", "What is new since Kimi-Linear" item 3); |output| < b1 * b2.
enum GluKind : int { kGluSilu = 0, kGluSitu = 1 };
struct GluAct {
  int kind;
  float b1, b2;     // kGluSitu: beta of the gate branch, beta of the linear (up) branch
  float ib1, ib2;   // 1 / b1, 1 / b2
};

// The epilogues evaluate the activation for every element of h with no matrix work to hide
// it behind, so the divisions use the hardware reciprocal (about 1 ulp) instead of the
// correctly rounded division sequence.
__device__ __forceinline__ float rcp_dev(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float silu_dev(float g) { return g * rcp_dev(1.0f + __expf(-g)); }

// tanh(x) = sign(x) * (1 - 2 / (exp(2|x|) + 1)): one hardware exponential and a reciprocal;
// saturates to +-1 without overflow (exp -> inf gives 1/inf = 0). Absolute error a few fp32
// ulps of 1 (the subtraction from 1), relative error larger only where |tanh x| < 1e-3,
// whose contribution to a GLU output is below 1e-7 * beta in absolute terms.
__device__ __forceinline__ float tanh_dev(float x) {
  const float t = 1.0f - 2.0f * rcp_dev(__expf(2.0f * fabsf(x)) + 1.0f);
  return copysignf(t, x);
}

__device__ __forceinline__ float glu_act(float gate, float up, GluAct a) {
  if (a.kind == kGluSitu) return a.b1 * tanh_dev(silu_dev(gate) * a.ib1) * (a.b2 * tanh_dev(up * a.ib2));
  return silu_dev(gate) * up;
}

__device__ __forceinline__ float sigmoidf_dev(float x) { return 1.0f / (1.0f + __expf(-x)); }

// wave-level sum (wave64)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Two fp32 values split exactly into three bf16 planes each (truncation: f = hi + mid + lo, every
// term a bf16 value, 24 significand bits = 3 x 8), packed two per dword (first value low).
__device__ __forceinline__ void split3x2(float f0, float f1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t h0 = __float_as_uint(f0) & 0xffff0000u, h1 = __float_as_uint(f1) & 0xffff0000u;
  const float r0 = f0 - __uint_as_float(h0), r1 = f1 - __uint_as_float(h1);
  const uint32_t m0 = __float_as_uint(r0) & 0xffff0000u, m1 = __float_as_uint(r1) & 0xffff0000u;
  const float l0 = r0 - __uint_as_float(m0), l1 = r1 - __uint_as_float(m1);
  hi = (h0 >> 16) | h1;
  mid = (m0 >> 16) | m1;
  lo = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xffff0000u);
}

// Streaming 16-byte load that bypasses nothing but marks the data as read-once.
__device__ __forceinline__ u32x4_t load_nt_u32x4(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}
__device__ __forceinline__ u32x4_t load_u32x4(const void* p) { return *(const u32x4_t*)p; }

// ---- buffer resources (raw buffers: an offset past num_records reads 0, with no memory access)
constexpr uint32_t kOob = 0x80000000u;  // offset past any tensor the kernels index
constexpr int kNonTemporal = 2;         // cache policy bit of once-read streams

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ u32x4_t buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kNonTemporal));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
