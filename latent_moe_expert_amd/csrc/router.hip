// Sigmoid router with a selection-only bias and top-k (WASTE "Kimi K3, as
// released": router row of the "Shape" table -- sigmoid, 1 group,
// routed_scaling_factor 1.0 -- and "Against the technical report": the
// correction bias is used for selection only and the weights are renormalised
// over the selected top-k, then multiplied by routed_scaling_factor).
//
// Keys key_e = sigmoid(logit_e) + bias_e become unique 64-bit composites (key
// bits, then the inverted expert id), so the larger composite is the larger key
// with ties going to the lower id. For up to 1024 experts and k <= 16 a block's
// threads hold a token's composites in registers; each wave takes its k largest
// as k successive wave-wide maxima, then one wave takes the k largest of those.
// Otherwise a bitonic sort in LDS orders all of them. Either way the winners are written in
// ascending id order with weights s_e / sum(s_selected) * rsf from the unbiased
// scores, summed in ascending id order.
//
// When the down-projection and router logits arrive as partial sums over K
// slices, a wide kernel first sums them (latent rounded to bf16) in slice order.
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 4096;

// Sums split-K partial planes: the latent rows (rounded to bf16) and the router
// logits (fp32), each element over its slices in slice order (loads issued in
// batches of 8 so that they overlap).
__global__ __launch_bounds__(256) void reduce_planes_kernel(RouteArgs a) {
  const size_t nz = a.z_part ? (size_t)a.T * a.L / 4 : 0;  // float4 groups of the latent
  const size_t nr = a.r_part ? (size_t)a.T * a.E : 0;        // logits, one by one
  const size_t zplane = (size_t)a.T * a.L, rplane = (size_t)a.T * a.E;
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < nz + nr; i += (size_t)gridDim.x * 256) {
    if (i < nz) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < a.sz; s0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = s0 + u < a.sz ? *(const f32x4_t*)(a.z_part + (s0 + u) * zplane + 4 * i) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      *(uint2*)(a.z_out + 4 * i) = uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    } else {
      const size_t j = i - nz;
      float acc = 0.f;
      for (int s0 = 0; s0 < a.sr; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = s0 + u < a.sr ? a.r_part[(s0 + u) * rplane + j] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
      }
      a.logits_out[j] = acc;
    }
  }
}

// Order-preserving map of a float to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One block per token: the keys become unique 64-bit composites
//   (ordered key bits << 32) | (0xffffffff - expert id),
// so "larger composite" means larger key, ties to the lower id. A bitonic sort
// in LDS orders them descending; the first k are the selected experts.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ unsigned long long comp[kMaxE];
  __shared__ float sco[kMaxE];
  __shared__ float sel_s[64];
  __shared__ int sel_e[64];
  __shared__ float total;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int E = a.E, k = a.k;
  int n2 = 64;
  while (n2 < E) n2 <<= 1;  // power of two >= E; padding composites are 0 and sort last
  const float* lg = a.logits + (size_t)t * E;

  for (int e = tid; e < n2; e += 256) {
    unsigned long long c = 0ull;
    if (e < E) {
      const float sc = sigmoidf_dev(lg[e]);
      float kv = sc + (a.bias ? a.bias[e] : 0.f);
      kv = (kv == kv) ? kv : -FLT_MAX;  // a NaN key ranks below every real key
      sco[e] = sc;
      c = ((unsigned long long)ordered_bits(kv) << 32) | (0xffffffffu - (uint32_t)e);
    }
    comp[e] = c;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += 256) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long x = comp[lo], y = comp[hi];
        if ((x < y) == desc) {
          comp[lo] = y;
          comp[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  // the k winners; write them in ascending id order
  if (tid < k) {
    const int e = (int)(0xffffffffu - (uint32_t)(comp[tid] & 0xffffffffull));
    int p = 0;
    for (int j = 0; j < k; ++j) {
      const int o = (int)(0xffffffffu - (uint32_t)(comp[j] & 0xffffffffull));
      p += o < e ? 1 : 0;
    }
    sel_e[p] = e;
    sel_s[p] = sco[e];
  }
  __syncthreads();
  if (tid == 0) {  // ascending id order: a fixed rounding order
    float tot = 0.f;
    for (int p = 0; p < k; ++p) tot += sel_s[p];
    total = tot;
  }
  __syncthreads();
  if (tid < k) {
    a.ids[(size_t)t * k + tid] = sel_e[tid];
    a.w[(size_t)t * k + tid] = sel_s[tid] / total * a.rsf;
  }
}

constexpr int kFastMaxE = 1024;  // experts per token of the register path: 4 per thread of a 256-thread block
constexpr int kFastMaxK = 16;    // its top-k: the four waves' k candidates are one per lane of one wave

// 64-bit max over the wave, returned to every lane. DPP moves (quad permutations, then
// the half-row and row mirrors) give each lane the maximum of its row of 16 lanes without
// going through LDS; the four row maxima are then combined through readlane.
__device__ __forceinline__ unsigned long long max_u64(unsigned long long x, unsigned long long y) {
  return y > x ? y : x;
}
template <int Ctrl>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, Ctrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), Ctrl, 0xf, 0xf, false);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)), max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// The k largest of the composites held by a wave (N per lane), as k successive wave
// maxima; lane j < k gets the j-th largest (0 when the wave holds fewer than k non-zero
// composites) and the score stored beside it.
template <int N>
__device__ __forceinline__ void wave_top(unsigned long long (&c)[N], const float (&sc)[N], int k, int lane,
                                         unsigned long long& my_c, float& my_s) {
  my_c = 0ull;
  my_s = 0.f;
  for (int j = 0; j < k; ++j) {
    unsigned long long m = c[0];
#pragma unroll
    for (int i = 1; i < N; ++i) m = max_u64(m, c[i]);
    m = wave_max_u64(m);
    // the owner (composites are unique, apart from zeros) clears its slot and hands over
    // the score through readlane from the lowest lane holding m
    float v = 0.f;
    bool own = false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (c[i] == m && !own) {
        v = sc[i];
        c[i] = 0ull;
        own = true;
      }
    }
    const unsigned long long ownmask = __ballot(own);
    const int src = ownmask ? __ffsll((long long)ownmask) - 1 : 0;
    v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
    if (lane == j) {
      my_c = m;
      my_s = v;
    }
  }
}

// One token per block. Thread t holds experts e = t + 256 i; each wave keeps its top k,
// then wave 0 takes the top k of the 4k candidates.
__global__ __launch_bounds__(256) void route_fast_kernel(RouteArgs a) {
  __shared__ unsigned long long cand_c[4][kFastMaxK];
  __shared__ float cand_s[4][kFastMaxK];
  __shared__ int sel_e[kFastMaxK];
  __shared__ float sel_s[kFastMaxK];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = blockIdx.x;
  const int E = a.E, k = a.k;
  const size_t row = (size_t)t * E;
  unsigned long long c[4];
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    c[i] = 0ull;  // below every real composite
    sc[i] = 0.f;
    if (e < E) {
      sc[i] = sigmoidf_dev(a.logits[row + e]);
      float kv = sc[i] + (a.bias ? a.bias[e] : 0.f);
      kv = (kv == kv) ? kv : -FLT_MAX;  // a NaN key ranks below every real key
      c[i] = ((unsigned long long)ordered_bits(kv) << 32) | (0xffffffffu - (uint32_t)e);
    }
  }
  unsigned long long my_c;
  float my_s;
  wave_top<4>(c, sc, k, lane, my_c, my_s);
  if (lane < k) {
    cand_c[wave][lane] = my_c;
    cand_s[wave][lane] = my_s;
  }
  __syncthreads();
  if (wave != 0) return;
  unsigned long long c1[1] = {lane < 4 * k ? cand_c[lane / k][lane % k] : 0ull};
  const float s1[1] = {lane < 4 * k ? cand_s[lane / k][lane % k] : 0.f};
  wave_top<1>(c1, s1, k, lane, my_c, my_s);
  const int my_e = (int)(0xffffffffu - (uint32_t)(my_c & 0xffffffffull));
  // ascending id order
  if (lane < k) {
    int p = 0;
    for (int j = 0; j < k; ++j) p += __builtin_amdgcn_readlane(my_e, j) < my_e ? 1 : 0;
    sel_e[p] = my_e;
    sel_s[p] = my_s;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float tot = 0.f;
  for (int p = 0; p < k; ++p) tot += sel_s[p];  // ascending id order: a fixed rounding order
  if (lane < k) {
    a.ids[(size_t)t * k + lane] = sel_e[lane];
    a.w[(size_t)t * k + lane] = sel_s[lane] / tot * a.rsf;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.r_part || a.z_part) {  // finish split-K sums first, in parallel over all elements
    const size_t n = (a.z_part ? (size_t)a.T * a.L / 4 : 0) + (a.r_part ? (size_t)a.T * a.E : 0);
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(reduce_planes_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, a);
  }
  if (a.E <= kFastMaxE && a.k <= kFastMaxK)
    hipLaunchKernelGGL(route_fast_kernel, dim3(a.T), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(route_kernel, dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
