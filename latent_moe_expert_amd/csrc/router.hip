// Sigmoid router with a selection-only bias and top-k (WASTE "Kimi K3, as
// released": router row of the "Shape" table -- sigmoid, 1 group,
// routed_scaling_factor 1.0 -- and "Against the technical report": the
// correction bias is used for selection only and the weights are renormalised
// over the selected top-k, then multiplied by routed_scaling_factor).
//
// Keys key_e = sigmoid(logit_e) + bias_e become unique 64-bit composites (key
// bits, then the inverted expert id), so the larger composite is the larger key
// with ties going to the lower id. For up to 1024 experts and k <= 16 one wave holds
// a token's composites in registers and selects the k largest (route_dev.h).
// Up to 4096 experts a bitonic sort in LDS orders all of them; beyond that (up to 65535) a
// radix select over the keys' 32-bit images finds the k-th largest key and an ordered pass
// takes the keys above it and the lowest ids among those equal to it. Every path writes the
// winners in ascending id order with weights s_e / sum(s_selected) * rsf from the unbiased
// scores, summed in ascending id order.
//
// When the down-projection and router logits arrive as partial sums over K
// slices, a wide kernel first sums them (latent rounded to bf16) in slice order.
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kMaxE = 4096;

// Split-K partial planes summed per element in slice order (loads issued in batches of 8 so
// that they overlap): float4 group i of the latent rows [T * L / 4], rounded to bf16, and
// logit j of [T * E] in fp32.
__device__ __forceinline__ void sum_z_group(const RouteArgs& a, size_t i) {
  const size_t zplane = (size_t)a.T * a.L;
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
}
__device__ __forceinline__ void sum_logit(const RouteArgs& a, size_t j) {
  const size_t rplane = (size_t)a.T * a.E;
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

// All split-K sums in parallel over all elements.
__global__ __launch_bounds__(256) void reduce_planes_kernel(RouteArgs a) {
  const size_t nz = a.z_part ? (size_t)a.T * a.L / 4 : 0;  // float4 groups of the latent
  const size_t nr = a.r_part ? (size_t)a.T * a.E : 0;        // logits, one by one
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < nz + nr; i += (size_t)gridDim.x * 256) {
    if (i < nz)
      sum_z_group(a, i);
    else
      sum_logit(a, i - nz);
  }
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

// Experts beyond the LDS sort (E > kMaxE): one block per token finds the k-th largest key by a
// radix select on the keys' order-preserving 32-bit images (four passes over 8-bit digits, each
// a 256-bin LDS histogram of the keys that match the digits found so far, read from the logits
// row in L2), then takes every key above it and, of the keys equal to it, the lowest ids, in
// one ordered pass over the experts (block prefix sums), which also yields ascending id order.
__device__ __forceinline__ uint32_t radix_key(const RouteArgs& a, const float* lg, int e, float* sig) {
  const float s = sigmoidf_dev(lg[e]);
  float kv = s + (a.bias ? a.bias[e] : 0.f);
  kv = (kv == kv) ? kv : -FLT_MAX;  // a NaN key ranks below every real key
  *sig = s;
  return ordered_bits(kv);
}

// exclusive prefix of f over the block (256 threads, in thread order) and the block total
__device__ __forceinline__ int block_prefix(bool f, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long b = __ballot(f);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(b);
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += wsum[i];
  *total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  __syncthreads();
  return off + in_wave;
}

__global__ __launch_bounds__(256) void route_radix_kernel(RouteArgs a) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ int sel_e[64];
  __shared__ float sel_s[64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  __shared__ float s_tot;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int E = a.E, k = a.k;
  const float* lg = a.logits + (size_t)t * E;
  uint32_t prefix = 0u, mask = 0u;
  int rem = k;  // how many of the keys matching prefix under mask are still to be taken
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      float sg;
      const uint32_t u = radix_key(a, lg, e, &sg);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 4l..4l+3; cum(d) = number of matching keys with digit >= d; the digit
      // taken is the largest d with cum(d) >= rem
      int h[4], lsum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = hist[4 * tid + i];
        lsum += h[i];
      }
      int above = lsum;  // inclusive suffix sum over lanes >= tid
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(above, o, 64);
        if (tid + o < 64) above += v;
      }
      above -= lsum;  // keys with digits in higher lanes
      int best = -1, best_above = 0;
      int cum = above;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (best < 0 && cum + h[i] >= rem) {
          best = 4 * tid + i;
          best_above = cum;
        }
        cum += h[i];
      }
      int d = best;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) d = max(d, __shfl_xor(d, o, 64));
      if (best == d && d >= 0) {
        s_prefix = prefix | ((uint32_t)d << shift);
        s_rem = rem - best_above;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    rem = s_rem;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the k-th largest image; every key above it is taken, and the first rem keys equal
  // to it in id order
  int eq_seen = 0, sel_seen = 0;
  for (int c0 = 0; c0 < E && sel_seen < k; c0 += 256) {
    const int e = c0 + tid;
    float sg = 0.f;
    const uint32_t u = e < E ? radix_key(a, lg, e, &sg) : 0u;
    const bool eq = e < E && u == prefix;
    int n_eq;
    const int eq_rank = block_prefix(eq, wsum, &n_eq);
    const bool sel = e < E && (u > prefix || (eq && eq_seen + eq_rank < rem));
    int n_sel;
    const int idx = sel_seen + block_prefix(sel, wsum, &n_sel);
    if (sel && idx < k) {
      sel_e[idx] = e;
      sel_s[idx] = sg;
    }
    eq_seen += n_eq;
    sel_seen += n_sel;
  }
  __syncthreads();
  if (tid == 0) {  // ascending id order: a fixed rounding order
    float tot = 0.f;
    for (int p = 0; p < k; ++p) tot += sel_s[p];
    s_tot = tot;
  }
  __syncthreads();
  if (tid < k) {
    const float tot = s_tot;
    a.ids[(size_t)t * k + tid] = sel_e[tid];
    a.w[(size_t)t * k + tid] = sel_s[tid] / tot * a.rsf;
  }
}

// One token per wave, four per block (E <= 64 * NPL <= kFastMaxE, k <= kFastMaxK): the waves
// share nothing but the block's LDS arrays, each its own part, and need no block barrier.
// PLANES2: the logits arrive as two split-K partial planes [2][T][E]; the wave sums them in
// slice order from zero (as reduce_planes_kernel does) and stores the sums in logits_out.
template <int NPL, bool PLANES2>
__global__ __launch_bounds__(256) void route_wave_kernel(RouteArgs a) {
  __shared__ float s_lds[4][64 * NPL];
  __shared__ RouteWaveSmem sm[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * 4 + wave;
  if (t >= a.T) return;  // wave-uniform
  const int E = a.E;
  // every load is issued before any is used; experts past E read as zeros
  const float* src = PLANES2 ? a.r_part : a.logits;
  const __amdgpu_buffer_rsrc_t lg_rs = make_rsrc(src + (size_t)t * E, (uint32_t)E * 4);
  const __amdgpu_buffer_rsrc_t l2_rs =
      make_rsrc(PLANES2 ? a.r_part + (size_t)a.T * E + (size_t)t * E : a.logits, PLANES2 ? (uint32_t)E * 4 : 0u);
  const __amdgpu_buffer_rsrc_t bs_rs = make_rsrc(a.bias, a.bias ? (uint32_t)E * 4 : 0u);
  float lg[NPL], l2[NPL], bs[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const uint32_t off = (uint32_t)(lane + 64 * i) * 4;
    lg[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lg_rs, off, 0, 0));
    if (PLANES2) l2[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(l2_rs, off, 0, 0));
    bs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bs_rs, off, 0, 0));
  }
  if constexpr (PLANES2) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      lg[i] = ((0.f + lg[i]) + l2[i]) + 0.f;
      if (e < E) a.logits_out[(size_t)t * E + e] = lg[i];
    }
  }
  unsigned long long c[NPL];
  float sc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    const float sg = sigmoidf_dev(lg[i]);
    float kv = sg + bs[i];
    kv = (kv == kv) ? kv : -FLT_MAX;  // a NaN key ranks below every real key
    c[i] = e < E ? ((unsigned long long)ordered_bits(kv) << 32) | (0xffffffffu - (uint32_t)e) : 0ull;
    sc[i] = e < E ? sg : 0.f;
  }
  route_select_wave<NPL>(c, sc, a.k, a.rsf, lane, s_lds[wave], sm[wave], a.ids + (size_t)t * a.k,
                         a.w + (size_t)t * a.k);
}

// Decode batches with split-K planes (E <= kFastMaxE, k <= kFastMaxK): one launch. Blocks
// 0..T-1 each sum their token's logits over the slices (slice order, as reduce_planes does),
// store them, and form the keys, which one wave of the block then selects from; the blocks
// after them sum the latent rows.
__global__ __launch_bounds__(256) void route_fast_planes_kernel(RouteArgs a) {
  __shared__ unsigned long long c_lds[kFastMaxE];
  __shared__ float s_lds[kFastMaxE];
  __shared__ RouteWaveSmem wsm;
  const int t = blockIdx.x;
  if (t >= a.T) {
    const size_t nz = (size_t)a.T * a.L / 4;
    for (size_t i = (size_t)(t - a.T) * 256 + threadIdx.x; i < nz; i += (size_t)(gridDim.x - a.T) * 256) sum_z_group(a, i);
    return;
  }
  const int E = a.E;
  const __amdgpu_buffer_rsrc_t bs_rs = make_rsrc(a.bias, a.bias ? (uint32_t)E * 4 : 0u);
  float bs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    bs[i] = __builtin_bit_cast(float,
                               __builtin_amdgcn_raw_buffer_load_b32(bs_rs, (uint32_t)(threadIdx.x + 256 * i) * 4, 0, 0));
  const size_t rplane = (size_t)a.T * E, row = (size_t)t * E;
  float lg[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < a.sr; s0 += 8) {
    float v[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + 256 * i;
        v[u][i] = s0 + u < a.sr && e < E ? a.r_part[(s0 + u) * rplane + row + e] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[i] += v[u][i];
  }
  // keys in the summing layout (expert tid + 256 i), handed to one wave through LDS
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x + 256 * i;
    if (e < E) {
      a.logits_out[row + e] = lg[i];
      const float sg = sigmoidf_dev(lg[i]);
      float kv = sg + bs[i];
      kv = (kv == kv) ? kv : -FLT_MAX;  // a NaN key ranks below every real key
      c_lds[e] = ((unsigned long long)ordered_bits(kv) << 32) | (0xffffffffu - (uint32_t)e);
      s_lds[e] = sg;
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;  // one wave selects
  const int lane = threadIdx.x;
  unsigned long long c[16];
  float sc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    c[i] = e < E ? c_lds[e] : 0ull;
    sc[i] = e < E ? s_lds[e] : 0.f;
  }
  route_select_wave<16>(c, sc, a.k, a.rsf, lane, s_lds, wsm, a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k);
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.r_part && a.z_part && a.E <= kFastMaxE && a.k <= kFastMaxK && a.logits_out == a.logits) {
    // one launch: T routing blocks, then a latent-summing block per 256 float4 groups
    const size_t zb = ((size_t)a.T * a.L / 4 + 255) / 256;
    hipLaunchKernelGGL(route_fast_planes_kernel, dim3((unsigned)(a.T + (zb < 4096 ? zb : 4096))), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.k > 64) return hipErrorInvalidValue;
  const bool fast = a.E <= kFastMaxE && a.k <= kFastMaxK;
  // two logit planes and no latent planes (the 2048+-row dense tile splits only the router):
  // the routing waves sum them as they load them
  const bool planes2 = fast && a.r_part && !a.z_part && a.sr == 2 && a.logits_out;
  if ((a.r_part || a.z_part) && !planes2) {  // finish split-K sums first, in parallel over all elements
    const size_t n = (a.z_part ? (size_t)a.T * a.L / 4 : 0) + (a.r_part ? (size_t)a.T * a.E : 0);
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(reduce_planes_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, a);
  }
  if (fast) {
    const dim3 grid((unsigned)((a.T + 3) / 4));
    auto go = [&](auto k2, auto k4, auto k8, auto k16) {
      if (a.E <= 128)
        hipLaunchKernelGGL(k2, grid, dim3(256), 0, s, a);
      else if (a.E <= 256)
        hipLaunchKernelGGL(k4, grid, dim3(256), 0, s, a);
      else if (a.E <= 512)
        hipLaunchKernelGGL(k8, grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(k16, grid, dim3(256), 0, s, a);
    };
    if (planes2)
      go(route_wave_kernel<2, true>, route_wave_kernel<4, true>, route_wave_kernel<8, true>, route_wave_kernel<16, true>);
    else
      go(route_wave_kernel<2, false>, route_wave_kernel<4, false>, route_wave_kernel<8, false>,
         route_wave_kernel<16, false>);
  }
  else if (a.E <= kMaxE)
    hipLaunchKernelGGL(route_kernel, dim3(a.T), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(route_radix_kernel, dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
