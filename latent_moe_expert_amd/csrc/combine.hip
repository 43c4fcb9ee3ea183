// Weighted aggregate of the routed experts' outputs and the optional RMSNorm on
// the aggregated latent, before the up-projection (WASTE "Kimi K3, as released",
// "Against the technical report": the latent MoE with RMSNorm before the
// up-projection; K3 report review, "Stable LatentMoE": aggregate -> normalise ->
// up-project).
//
// Gather form: token t reads its k expert outputs at inv_pos[t*k+j] and sums
// w_tj * O in slot order j = 0..k-1 in fp32 (no atomics, deterministic). The
// norm is c / sqrt(mean(c^2) + eps) * g with a fixed-order block reduction.
// Output: bf16 c' (the up-projection's activations) and optionally fp32 c.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxSlots = 64;

__global__ __launch_bounds__(256) void combine_norm_kernel(const float* __restrict__ O, int L,
                                                           const int32_t* __restrict__ inv_pos,
                                                           const float* __restrict__ w, int k,
                                                           const uint16_t* __restrict__ norm, float eps,
                                                           float* __restrict__ c_tap, uint16_t* __restrict__ c_norm) {
  __shared__ int pos[kMaxSlots];
  __shared__ float wt[kMaxSlots];
  __shared__ float red[4];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    pos[threadIdx.x] = inv_pos[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // each thread owns latent columns l = tid + 256*i; keep them in registers (L <= 256*kCols)
  constexpr int kCols = 32;
  float cv[kCols];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    const int l = threadIdx.x + 256 * i;
    float c = 0.f;
    if (l < L) {
      for (int j = 0; j < k; ++j) {
        const int p = pos[j];
        if (p >= 0) c += wt[j] * O[(size_t)p * L + l];
      }
      ss += c * c;
      if (c_tap) c_tap[(size_t)t * L + l] = c;
    }
    cv[i] = c;
  }
  float scale = 1.f;
  if (norm) {
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    scale = rsqrtf(tot / (float)L + eps);
  }
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    const int l = threadIdx.x + 256 * i;
    if (l < L) {
      const float g = norm ? bf16_bits_to_f32(norm[l]) : 1.f;
      c_norm[(size_t)t * L + l] = (uint16_t)f32_to_bf16_bits(norm ? cv[i] * scale * g : cv[i]);
    }
  }
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

}  // namespace

hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const float* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float eps, float* c_tap, uint16_t* c_norm, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap, c_norm);
  return hipGetLastError();
}

}  // namespace moe
