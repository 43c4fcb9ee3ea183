// Weighted aggregate of the routed experts' outputs and the optional RMSNorm on
// the aggregated latent, before the up-projection (WASTE "Kimi K3, as released",
// "Against the technical report": the latent MoE with RMSNorm before the
// up-projection; K3 report review, "Stable LatentMoE": aggregate -> normalise ->
// up-project).
//
// Gather form: token t reads its k expert outputs -- rows t*k .. t*k+k-1 of O when O has
// one row per (token, slot), or rows inv_pos[t*k+j] when O follows the expert-sorted
// layout -- and sums w_tj * O in slot order j = 0..k-1 in fp32 (no atomics,
// deterministic). The
// norm is c / sqrt(mean(c^2) + eps) * g with a fixed-order block reduction.
// Output: bf16 c' (the up-projection's activations) and optionally fp32 c.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxSlots = 64;

// One block per token; thread owns float4 columns v = tid + 256*i (i < KV). Slots
// are taken in groups of G = 32/KV with every load of a group issued before any
// use, then added in slot order (a fixed rounding order). Each row of O is read once,
// with the read-once cache policy: at 8192 tokens (1.88 GB of O) 0.348 ms against 0.373.
template <int KV>
__global__ __launch_bounds__(256) void combine_norm_kernel(const float* __restrict__ O, int L,
                                                           const int32_t* __restrict__ inv_pos,
                                                           const float* __restrict__ w, int k,
                                                           const uint16_t* __restrict__ norm, float eps,
                                                           float* __restrict__ c_tap, uint16_t* __restrict__ c_norm) {
  constexpr int G = 32 / KV;
  __shared__ int pos[kMaxSlots];
  __shared__ float wt[kMaxSlots];
  __shared__ float red[4];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const size_t f = (size_t)t * k + threadIdx.x;
    pos[threadIdx.x] = inv_pos ? inv_pos[f] : (int)f;
    wt[threadIdx.x] = w[f];
  }
  __syncthreads();
  const int nvec = L >> 2;
  f32x4_t acc[KV];
#pragma unroll
  for (int i = 0; i < KV; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += G) {
    f32x4_t v[G][KV];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      const int p = j < k ? pos[j] : -1;
      const f32x4_t* row = (const f32x4_t*)(O + (size_t)(p < 0 ? 0 : p) * L);
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        v[g][i] = (p >= 0 && vi < nvec) ? __builtin_nontemporal_load(row + vi) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      const float wj = j < k ? wt[j] : 0.f;
#pragma unroll
      for (int i = 0; i < KV; ++i) acc[i] += wj * v[g][i];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nvec) {
      ss += acc[i][0] * acc[i][0] + acc[i][1] * acc[i][1] + acc[i][2] * acc[i][2] + acc[i][3] * acc[i][3];
      if (c_tap) *(f32x4_t*)(c_tap + (size_t)t * L + 4 * vi) = acc[i];
    }
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
  for (int i = 0; i < KV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nvec) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g = norm ? bf16_bits_to_f32(norm[4 * vi + e]) : 1.f;
        o[e] = norm ? acc[i][e] * scale * g : acc[i][e];
      }
      uint2 packed = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *(uint2*)(c_norm + (size_t)t * L + 4 * vi) = packed;
    }
  }
}

// Decode batches: block (t, q) owns columns 256q .. 256q + 255 of token t, one per thread,
// and sums the k slots in slot order as above. It writes c (fp32) and, for the up-projection,
// bf16(c * g) (bf16(c) without a norm weight); with the norm it also writes the block's sum
// of c^2 (fixed-order wave and block reduction). The 1 / rms(c) factor is applied to the
// up-projection's output (finish_up), so no block needs another block's columns.
__global__ __launch_bounds__(256) void combine_cols_kernel(const float* __restrict__ O, int L,
                                                           const int32_t* __restrict__ inv_pos,
                                                           const float* __restrict__ w, int k,
                                                           const uint16_t* __restrict__ norm, float* __restrict__ c,
                                                           uint16_t* __restrict__ cg, float* __restrict__ part_sq) {
  constexpr int G = 16;
  __shared__ int pos[kMaxSlots];
  __shared__ float wt[kMaxSlots];
  __shared__ float red[4];
  const int Q = L >> 8;
  const int t = (int)blockIdx.x / Q, qb = (int)blockIdx.x % Q;
  if (threadIdx.x < k) {
    const size_t f = (size_t)t * k + threadIdx.x;
    pos[threadIdx.x] = inv_pos ? inv_pos[f] : (int)f;
    wt[threadIdx.x] = w[f];
  }
  __syncthreads();
  const int col = qb * 256 + threadIdx.x;
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += G) {
    float v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      const int p = j < k ? pos[j] : -1;
      v[g] = p >= 0 ? O[(size_t)p * L + col] : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      acc += (j < k ? wt[j] : 0.f) * v[g];
    }
  }
  const size_t o = (size_t)t * L + col;
  c[o] = acc;
  cg[o] = (uint16_t)f32_to_bf16_bits(norm ? acc * bf16_bits_to_f32(norm[col]) : acc);
  if (norm) {
    const float ss = wave_sum(acc * acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) part_sq[(size_t)t * Q + qb] = ((red[0] + red[1]) + red[2]) + red[3];
  }
}

// The normalised aggregate itself, bf16(c * s * g) with s = 1 / sqrt(sum of the partial sums
// in column-block order / L + eps): the c_norm tap of the decode path.
__global__ __launch_bounds__(256) void norm_from_parts_kernel(const float* __restrict__ c,
                                                              const float* __restrict__ part_sq, int L,
                                                              const uint16_t* __restrict__ norm, float eps,
                                                              uint16_t* __restrict__ out) {
  const int t = blockIdx.x, Q = L >> 8;
  float tot = 0.f;
  for (int i = 0; i < Q; ++i) tot += part_sq[(size_t)t * Q + i];
  const float scale = rsqrtf(tot / (float)L + eps);
  for (int col = threadIdx.x; col < L; col += 256) {
    const size_t o = (size_t)t * L + col;
    out[o] = (uint16_t)f32_to_bf16_bits(c[o] * scale * bf16_bits_to_f32(norm[col]));
  }
}

// RMSNorm of bf16 rows: y = x / sqrt(mean(x^2) + eps) * g (g = 1 without a weight), one
// block per row. Pass 1 sums the squares (each thread its columns in ascending order,
// then a fixed-order wave and block reduction); pass 2 re-reads the row (from L2) and
// writes it, each element read before its own store, so y may be x.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int cols,
                                                      const uint16_t* __restrict__ g, float eps, uint16_t* y) {
  __shared__ float red[4];
  const size_t row = (size_t)blockIdx.x * cols;
  const int nvec = cols >> 2;
  float ss = 0.f;
  for (int v = threadIdx.x; v < nvec; v += 256) {
    const uint2 u = *(const uint2*)(x + row + 4 * v);
    const float a = bf16_bits_to_f32(u.x & 0xffffu), b = bf16_bits_to_f32(u.x >> 16);
    const float c = bf16_bits_to_f32(u.y & 0xffffu), d = bf16_bits_to_f32(u.y >> 16);
    ss += a * a + b * b + c * c + d * d;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float scale = rsqrtf((((red[0] + red[1]) + red[2]) + red[3]) / (float)cols + eps);
  for (int v = threadIdx.x; v < nvec; v += 256) {
    const uint2 u = *(const uint2*)(x + row + 4 * v);
    float o[4] = {bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16), bf16_bits_to_f32(u.y & 0xffffu),
                  bf16_bits_to_f32(u.y >> 16)};
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = g ? o[e] * scale * bf16_bits_to_f32(g[4 * v + e]) : o[e] * scale;
    *(uint2*)(y + row + 4 * v) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const float* __restrict__ src, int cols,
                                                          const int32_t* __restrict__ idx, float* __restrict__ out) {
  const size_t from = (size_t)idx[blockIdx.x] * cols, to = (size_t)blockIdx.x * cols;
  for (int v = threadIdx.x; v < cols / 4; v += 256) *(f32x4_t*)(out + to + 4 * v) = *(const f32x4_t*)(src + from + 4 * v);
}

// O in bf16 (the MFMA path's down output above 64 rows): thread owns 8-column vectors
// v = tid + 256 i (i < KV), one 16-byte read-once load per slot and vector; slots in groups of
// G = 16 / KV with every load of a group issued before any use, summed in slot order in fp32
// as above. At 8192 tokens it reads 0.94 GB of O instead of 1.88 (0.18 ms against 0.35 ms).
template <int KV>
__global__ __launch_bounds__(256) void combine_norm_bf16_kernel(const uint16_t* __restrict__ O, int L,
                                                                const int32_t* __restrict__ inv_pos,
                                                                const float* __restrict__ w, int k,
                                                                const uint16_t* __restrict__ norm, float eps,
                                                                float* __restrict__ c_tap,
                                                                uint16_t* __restrict__ c_norm) {
  constexpr int G = 16 / KV;
  __shared__ int pos[kMaxSlots];
  __shared__ float wt[kMaxSlots];
  __shared__ float red[4];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const size_t f = (size_t)t * k + threadIdx.x;
    pos[threadIdx.x] = inv_pos ? inv_pos[f] : (int)f;
    wt[threadIdx.x] = w[f];
  }
  __syncthreads();
  const int nvec = L >> 3;
  float acc[KV][8];
#pragma unroll
  for (int i = 0; i < KV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int j0 = 0; j0 < k; j0 += G) {
    u32x4_t v[G][KV];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      const int p = j < k ? pos[j] : -1;
      const u32x4_t* row = (const u32x4_t*)(O + (size_t)(p < 0 ? 0 : p) * L);
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int vi = threadIdx.x + 256 * i;
        v[g][i] = (p >= 0 && vi < nvec) ? __builtin_nontemporal_load(row + vi) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j = j0 + g;
      const float wj = j < k ? wt[j] : 0.f;
#pragma unroll
      for (int i = 0; i < KV; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][2 * e] += wj * bf16_bits_to_f32(v[g][i][e] & 0xffffu);
          acc[i][2 * e + 1] += wj * bf16_bits_to_f32(v[g][i][e] >> 16);
        }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += acc[i][e] * acc[i][e];
      if (c_tap) {
        float* ct = c_tap + (size_t)t * L + 8 * vi;
        *(f32x4_t*)ct = f32x4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
        *(f32x4_t*)(ct + 4) = f32x4_t{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
      }
    }
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
  for (int i = 0; i < KV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nvec) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = norm ? bf16_bits_to_f32(norm[8 * vi + e]) : 1.f;
        o[e] = norm ? acc[i][e] * scale * g : acc[i][e];
      }
      *(u32x4_t*)(c_norm + (size_t)t * L + 8 * vi) =
          u32x4_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
  }
}

// Rows of bf16 O widened to fp32 (the O tap of the MFMA path); rows of a negative index are zero.
__global__ __launch_bounds__(256) void gather_rows_bf16_kernel(const uint16_t* __restrict__ src, int cols,
                                                               const int32_t* __restrict__ idx, float* __restrict__ out) {
  const int r = idx[blockIdx.x];
  const size_t to = (size_t)blockIdx.x * cols;
  for (int v = threadIdx.x; v < cols / 4; v += 256) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
    if (r >= 0) {
      const uint2 b = *(const uint2*)(src + (size_t)r * cols + 4 * v);
      x = f32x4_t{bf16_bits_to_f32(b.x & 0xffffu), bf16_bits_to_f32(b.x >> 16), bf16_bits_to_f32(b.y & 0xffffu),
                  bf16_bits_to_f32(b.y >> 16)};
    }
    *(f32x4_t*)(out + to + 4 * v) = x;
  }
}

// bf16 -> fp32, four values per thread (the shared experts' output tap when it is held in bf16)
__global__ __launch_bounds__(256) void widen_bf16_kernel(const uint16_t* __restrict__ src, size_t n4,
                                                         float* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const uint2 b = *(const uint2*)(src + 4 * i);
    *(f32x4_t*)(out + 4 * i) = f32x4_t{bf16_bits_to_f32(b.x & 0xffffu), bf16_bits_to_f32(b.x >> 16),
                                       bf16_bits_to_f32(b.y & 0xffffu), bf16_bits_to_f32(b.y >> 16)};
  }
}

__global__ void fill_f32_kernel(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, int rows, int cols, const uint16_t* g, float eps, uint16_t* y,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x, cols, g, eps, y);
  return hipGetLastError();
}

hipError_t launch_gather_rows_f32(const float* src, int cols, const int32_t* idx, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(256), 0, s, src, cols, idx, out);
  return hipGetLastError();
}

hipError_t launch_widen_bf16(const uint16_t* src, size_t n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  const size_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, src, n / 4, out);
  return hipGetLastError();
}

hipError_t launch_gather_rows_bf16(const uint16_t* src, int cols, const int32_t* idx, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_bf16_kernel, dim3(n), dim3(256), 0, s, src, cols, idx, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const float* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float eps, float* c_tap, uint16_t* c_norm, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int nvec = L / 4;
  const int kv = (nvec + 255) / 256;
  if (kv <= 1)
    hipLaunchKernelGGL(combine_norm_kernel<1>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap, c_norm);
  else if (kv <= 2)
    hipLaunchKernelGGL(combine_norm_kernel<2>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap, c_norm);
  else if (kv <= 4)
    hipLaunchKernelGGL(combine_norm_kernel<4>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap, c_norm);
  else
    hipLaunchKernelGGL(combine_norm_kernel<8>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap, c_norm);
  return hipGetLastError();
}

hipError_t launch_combine_norm_bf16(const uint16_t* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                                    const uint16_t* norm, float eps, float* c_tap, uint16_t* c_norm, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (L % 8) return hipErrorInvalidValue;
  const int kv = (L / 8 + 255) / 256;
  if (kv <= 1)
    hipLaunchKernelGGL(combine_norm_bf16_kernel<1>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap,
                       c_norm);
  else if (kv <= 2)
    hipLaunchKernelGGL(combine_norm_bf16_kernel<2>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap,
                       c_norm);
  else
    hipLaunchKernelGGL(combine_norm_bf16_kernel<4>, dim3(T), dim3(256), 0, s, O, L, inv_pos, w, k, norm, eps, c_tap,
                       c_norm);
  return hipGetLastError();
}

hipError_t launch_combine_cols(const float* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float* c, uint16_t* cg, float* part_sq, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (L % 256 || k > kMaxSlots || !c || !cg || (norm && !part_sq)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_cols_kernel, dim3(T * (L / 256)), dim3(256), 0, s, O, L, inv_pos, w, k, norm, c, cg,
                     part_sq);
  return hipGetLastError();
}

hipError_t launch_norm_from_parts(const float* c, const float* part_sq, int T, int L, const uint16_t* norm, float eps,
                                  uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (L % 256 || !norm) return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_from_parts_kernel, dim3(T), dim3(256), 0, s, c, part_sq, L, norm, eps, out);
  return hipGetLastError();
}

}  // namespace moe
