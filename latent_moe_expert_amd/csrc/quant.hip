// Activation encodings (MXFP6 hi/lo, MXFP8) for the expert contractions, and their work list.
#include "common.h"
#include "kernels.h"
#include "mxfp6.h"
#include "mxfp8.h"

namespace moe {

namespace {

// One thread per group of 32 values: 64 bytes in, 2 x 24 bytes and 2 scale bytes out. The
// block's 256 groups move through LDS: each load instruction reads 1 KB of contiguous rows
// (16 groups x 64 bytes; part r of block group lg at LDS slot 4 lg + (r ^ (lg / 4 % 4)), so
// that the per-group reads are conflict-free), and the 48 output bytes of each group, which
// lie contiguous in the dense FP6 rows, leave as 16-byte stores of consecutive lanes. At 8192
// tokens (z and x, 176 MB in, 132 MB out) 64.5 us against 89 us with one thread reading and
// writing its own group (64-byte strided loads, 8-byte strided stores).
__global__ __launch_bounds__(256) void quant_fp6_kernel(const uint16_t* __restrict__ A, int lda, int rows, int K,
                                                        uint8_t* __restrict__ data, uint8_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[256 * 64];
  const int G = K >> 5;
  const long long ng = (long long)rows * G;
  const long long base = (long long)blockIdx.x * 256;
  const int nv = (int)min(256ll, ng - base);  // valid groups of this block (>= 1)
  const int tid = threadIdx.x;
  const int base_row = (int)(base / G), base_g = (int)(base % G);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j, lg = c >> 2, r = c & 3;
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (lg < nv) {
      const int gg = base_g + lg;
      const int row = base_row + gg / G, g = gg % G;
      x = __builtin_nontemporal_load((const u32x4_t*)(A + (size_t)row * lda + (size_t)g * 32 + r * 8));
    }
    *(u32x4_t*)(tile + (4 * lg + (r ^ ((lg >> 2) & 3))) * 16) = x;
  }
  __syncthreads();
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t x = *(const u32x4_t*)(tile + (4 * tid + (j ^ ((tid >> 2) & 3))) * 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * j + 2 * e] = bf16_bits_to_f32(x[e] & 0xffffu);
      v[8 * j + 2 * e + 1] = bf16_bits_to_f32(x[e] >> 16);
    }
  }
  uint32_t hi[6], lo[6], s_hi, s_lo;
  fp6_encode_group(v, hi, lo, s_hi, s_lo);
  __syncthreads();  // the tile now takes the outputs: group lg's 48 bytes at 48 lg
  u32x4_t* o = (u32x4_t*)(tile + tid * 48);
  o[0] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  o[1] = u32x4_t{hi[4], hi[5], lo[0], lo[1]};
  o[2] = u32x4_t{lo[2], lo[3], lo[4], lo[5]};
  __syncthreads();
  // FP6 rows are dense (fp6_row_bytes(K) = 48 G): group gi's bytes start at 48 gi
  uint8_t* dst = data + (size_t)base * 48;
  for (int b = tid * 16; b < nv * 48; b += 256 * 16) *(u32x4_t*)(dst + b) = *(const u32x4_t*)(tile + b);
  if (tid < nv) {
    const int gg = base_g + tid;
    const int row = base_row + gg / G, g = gg % G;
    uint8_t* srow = scales + (size_t)row * fp6_scale_row_bytes(K);
    srow[fp6_scale_offset(g, 0)] = (uint8_t)s_hi;
    srow[fp6_scale_offset(g, 1)] = (uint8_t)s_lo;
  }
}

__device__ __forceinline__ void load_bf16x32(const uint16_t* p, float v[32]) {
  const u32x4_t* src = (const u32x4_t*)p;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t x = src[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * j + 2 * e] = bf16_bits_to_f32(x[e] & 0xffffu);
      v[8 * j + 2 * e + 1] = bf16_bits_to_f32(x[e] >> 16);
    }
  }
}

// One thread per group of 32 values: the MXFP8 value of each, back in bf16.
__global__ __launch_bounds__(256) void qdq_fp8_kernel(const uint16_t* in, int ld_in, int rows, int K, uint16_t* out,
                                                      int ld_out) {
  const int G = K >> 5;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * G) return;
  const int row = (int)(idx / G), g = (int)(idx % G);
  float v[32];
  load_bf16x32(in + (size_t)row * ld_in + (size_t)g * 32, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int s = mxfp8_scale_exp(amax);
  u32x4_t* dst = (u32x4_t*)(out + (size_t)row * ld_out + (size_t)g * 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4_t x;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = pack_bf16x2(ldexpf(e4m3_round(ldexpf(v[8 * j + 2 * e], -s)), s),
                         ldexpf(e4m3_round(ldexpf(v[8 * j + 2 * e + 1], -s)), s));
    dst[j] = x;
  }
}

// One thread per group of 32 values: 64 bytes in, 32 code bytes and 1 scale byte out.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ A, int lda, int rows, int K,
                                                        uint8_t* __restrict__ data, uint8_t* __restrict__ scales) {
  const int G = K >> 5;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)rows * G) return;
  const int row = (int)(idx / G), g = (int)(idx % G);
  float v[32];
  load_bf16x32(A + (size_t)row * lda + (size_t)g * 32, v);
  uint32_t codes[8], sc;
  mxfp8_encode_group(v, codes, sc);
  u32x4_t* d = (u32x4_t*)(data + (size_t)row * fp8_row_bytes(K) + (size_t)g * 32);
  d[0] = u32x4_t{codes[0], codes[1], codes[2], codes[3]};
  d[1] = u32x4_t{codes[4], codes[5], codes[6], codes[7]};
  scales[(size_t)row * fp8_scale_row_bytes(K) + fp8_scale_offset(g)] = (uint8_t)sc;
}

// Single block: per-expert padded segment offsets (the align layout) and job counts,
// scanned in expert order, then one job per chunk of at most spj valid slots.
constexpr int kJobThreads = 1024;

__global__ __launch_bounds__(kJobThreads) void mx_jobs_kernel(const int32_t* __restrict__ counts, int E, int B,
                                                             int spj, int4* __restrict__ jobs,
                                                             int32_t* __restrict__ n_jobs) {
  __shared__ int s_pad[kJobThreads];
  __shared__ int s_job[kJobThreads];
  const int tid = threadIdx.x;
  const int per = (E + kJobThreads - 1) / kJobThreads;  // experts per thread, contiguous
  const int e0 = tid * per;
  int pad = 0, nj = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = counts[e];
    pad += (c + B - 1) / B * B;
    nj += (c + spj - 1) / spj;
  }
  s_pad[tid] = pad;
  s_job[tid] = nj;
  __syncthreads();
  // inclusive scan (Hillis-Steele), then shift to exclusive
  for (int o = 1; o < kJobThreads; o <<= 1) {
    const int a = tid >= o ? s_pad[tid - o] : 0;
    const int b = tid >= o ? s_job[tid - o] : 0;
    __syncthreads();
    s_pad[tid] += a;
    s_job[tid] += b;
    __syncthreads();
  }
  int slot = s_pad[tid] - pad, job = s_job[tid] - nj;
  if (tid == kJobThreads - 1) *n_jobs = s_job[tid];
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = counts[e];
    for (int f = 0; f < c; f += spj) jobs[job++] = make_int4(slot + f, min(spj, c - f), e, 0);
    slot += (c + B - 1) / B * B;
  }
}

}  // namespace

hipError_t launch_quant_fp6(const uint16_t* A, int lda, int rows, int K, uint8_t* data, uint8_t* scales,
                            hipStream_t s) {
  if (K % 512 || lda % 8 || rows < 0) return hipErrorInvalidValue;
  const long long groups = (long long)rows * (K / 32);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_fp6_kernel, dim3((unsigned)blocks), dim3(256), 0, s, A, lda, rows, K, data, scales);
  return hipGetLastError();
}

hipError_t launch_qdq_fp8(const uint16_t* in, int ld_in, int rows, int K, uint16_t* out, int ld_out,
                          hipStream_t s) {
  if (K % 32 || K < 0 || ld_in % 8 || ld_out % 8 || ld_in < K || ld_out < K || rows < 0) return hipErrorInvalidValue;
  const long long groups = (long long)rows * (K / 32);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qdq_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, ld_in, rows, K, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const uint16_t* A, int lda, int rows, int K, uint8_t* data, uint8_t* scales,
                            hipStream_t s) {
  if (K % 512 || lda % 8 || lda < K || rows < 0) return hipErrorInvalidValue;
  const long long groups = (long long)rows * (K / 32);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups + 255) / 256;
  if (blocks > 0x7fffffffll) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, A, lda, rows, K, data, scales);
  return hipGetLastError();
}

int mx_max_jobs(int pairs, int E, int slots_per_job) {
  // sum_e ceil(c_e / spj) <= sum_e (c_e / spj) + #{e : c_e > 0}
  return pairs / slots_per_job + (pairs < E ? pairs : E) + 1;
}

hipError_t launch_mx_jobs(const int32_t* counts, int E, int B, int slots_per_job, int4* jobs, int32_t* n_jobs,
                          hipStream_t s) {
  if (E < 1 || B < 1 || slots_per_job < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_jobs_kernel, dim3(1), dim3(kJobThreads), 0, s, counts, E, B, slots_per_job, jobs, n_jobs);
  return hipGetLastError();
}

}  // namespace moe
