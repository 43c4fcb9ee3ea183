// Quantile Balancing: the per-expert selection bias that gives every expert its
// target load (K3 report review, section on Quantile Balancing). With m tokens,
// n experts and k experts per token the target is q = max(1, floor(m*k/n)).
// Each token's threshold alpha is the (k+1)-th largest of its biased keys
// s + b; the margin of token i at expert j is s_ij - alpha_i; an expert's new
// bias is minus the margin quantile that q margins reach, estimated from a
// 1000-bin integer histogram per expert over [-2, 2) (the page's one integer
// all-reduce per layer and step acts on these histograms).
//
// Every float -> integer decision (the threshold selection, a margin's bin) and
// the bin edge that becomes the bias are single IEEE fp32 operations in a fixed
// order, with contraction off, so any exact fp32 evaluation takes the same
// decisions:  key = s + b;  mu = s - alpha;  bin = clamp(floor((mu + 2) * 250));
// bias' = -(-2 + t * 0.004).
//
// Kernels:
//   qb_alpha_kernel  one wave per token: the (k+1)-th largest key by a bitwise
//                    search over order-preserving integer images of the keys
//                    (the largest U with #{keys >= U} >= k+1 is exactly that
//                    order statistic, ties counted with multiplicity), run over
//                    the few keys at or above an exact lower bound.
//   qb_hist_kernel   one block per 4 experts over all tokens: LDS histograms
//                    updated with integer atomics, then stored whole -- no
//                    global atomics, so the counts need no prior clearing.
//   qb_bias_kernel   one wave per expert: the largest bin whose suffix count
//                    reaches q (bins spread 16 per lane, suffix sums in int64).
//                    For a single batch the histogram kernel does the same in
//                    its epilogue, on the LDS histograms it just completed.
#include <math.h>

#include "common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace moe {

namespace {

constexpr int kBins = kQbBins;
constexpr int kHistExperts = 4;  // experts per histogram block (16 KB of LDS)

__device__ __forceinline__ uint32_t qb_ordered(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float qb_unordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// bin of a margin: floor((mu + 2) * 250), clamped to [0, 999]; two fp32 roundings.
// (Plain operators under the pragma above: the __f*_rn helpers are defined in the
// HIP headers, outside its reach, and the compiler fuses them into an FMA.)
__device__ __forceinline__ int qb_bin(float mu) {
  float v = (mu + 2.0f) * 250.0f;
  v = fminf(fmaxf(v, 0.0f), (float)(kBins - 1));
  return (int)v;  // v >= 0: truncation is the floor
}

// Largest U with #{lanes: v_lane >= U, and U within the bits below `bit`} >= k1,
// given that the answer's bits above `bit` equal those of `prefix`.
__device__ __forceinline__ uint32_t qb_search_lanes(uint32_t v, int k1, uint32_t prefix, int bit) {
  for (; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    if (__popcll(__ballot(v >= cand)) >= k1) prefix = cand;
  }
  return prefix;
}

constexpr int kCandCap = 256;  // keys kept per token for the final search (else search them all)

// The bitwise search over the first `count` (<= 64 * NC) keys of an LDS list.
template <int NC>
__device__ __forceinline__ uint32_t qb_search_chunks(const uint32_t* keys, int count, int lane, int k1, uint32_t prefix,
                                                     int bit) {
  uint32_t c[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) c[j] = j * 64 + lane < count ? keys[j * 64 + lane] : 0u;
  for (; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j) cnt += __popcll(__ballot(c[j] >= cand));
    if (cnt >= k1) prefix = cand;
  }
  return prefix;
}

// PL keys per lane (n <= 64 * PL). Four tokens per block of 256 threads.
// 1. tau = the k1-th largest of the 64 lane maxima. The k1 lanes whose maximum is
//    >= tau hold k1 distinct keys >= tau, so alpha >= tau; alpha <= hi, the largest
//    key. alpha therefore shares the leading bits common to tau and hi.
// 2. The keys >= tau are compacted into LDS (usually a few dozen).
// 3. A bitwise search over the remaining bits: the largest U with #{keys >= U}
//    >= k1. Restricting the count to keys >= tau changes no decision: for
//    U > tau it drops nothing, and for U <= tau both counts are >= k1.
// VEC (n a multiple of 4): lane l holds keys 256 i + 4 l + c, read as 16-byte loads (a row of
// 896 scores is 4 load instructions instead of 14; the kernel is bound by its load
// instructions); else keys 64 i + l, read as 4-byte loads. The searches below depend only on
// the multiset of keys, not on which lane holds which.
template <int PL, bool BIAS, bool VEC>
__global__ __launch_bounds__(256) void qb_alpha_kernel(const float* __restrict__ s, const float* __restrict__ bias,
                                                       int m, int n, int k1, float* __restrict__ alpha) {
  __shared__ uint32_t cand_keys[4][kCandCap];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + w;
  if (t >= m) return;
  // Every load is issued before any is used: buffer loads over the row (past its end
  // they return 0 without a memory access), one lane offset and constant offsets.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + (size_t)t * n, (uint32_t)n * 4u);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, BIAS ? (uint32_t)n * 4u : 0u);
  uint32_t u[PL];
  if constexpr (VEC) {
    constexpr int P4 = PL / 4;
    u32x4_t sv[P4], bv[P4];
#pragma unroll
    for (int i = 0; i < P4; ++i) sv[i] = buf_load16(rs, lane * 16, i * 1024);
#pragma unroll
    for (int i = 0; i < P4; ++i) bv[i] = BIAS ? buf_load16(rb, lane * 16, i * 1024) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < P4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)  // 0 lies below the image of every key (that of -inf is 0x007fffff)
        u[4 * i + c] = 256 * i + 4 * lane + c < n
                           ? qb_ordered(__uint_as_float(sv[i][c]) + __uint_as_float(bv[i][c]))
                           : 0u;
  } else {
    float sv[PL], bv[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i)
      sv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, i * 256, 0));
#pragma unroll
    for (int i = 0; i < PL; ++i)
      bv[i] =
          BIAS ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, lane * 4, i * 256, 0)) : 0.0f;
#pragma unroll
    for (int i = 0; i < PL; ++i)  // 0 lies below the image of every key (that of -inf is 0x007fffff)
      u[i] = i * 64 + lane < n ? qb_ordered(sv[i] + bv[i]) : 0u;
  }
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < PL; ++i) mx = max(mx, u[i]);
  uint32_t hi = mx, lo_m = mx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    lo_m = min(lo_m, (uint32_t)__shfl_xor((int)lo_m, o, 64));
  }
  // wave-uniform from here on: keep the searches in scalar registers and branches
  hi = __builtin_amdgcn_readfirstlane(hi);
  lo_m = __builtin_amdgcn_readfirstlane(lo_m);
  // tau lies in [lo_m, hi]: it shares their leading bits
  uint32_t tau = 0u;
  if (k1 <= 64) {
    const int d0 = lo_m == hi ? 32 : __clz(lo_m ^ hi);
    tau = d0 == 32 ? hi : qb_search_lanes(mx, k1, d0 ? lo_m & (0xffffffffu << (32 - d0)) : 0u, 31 - d0);
  }
  if (tau == hi) {  // alpha = tau
    if (lane == 0) alpha[t] = qb_unordered(tau);
    return;
  }
  const int d = __clz(tau ^ hi);                       // leading bits shared by tau and hi (< 32)
  const uint32_t prefix = d ? tau & (0xffffffffu << (32 - d)) : 0u;
  const uint32_t lo = tau ? tau : 1u;                  // padding (0) is never a candidate
  const unsigned long long below = (1ull << lane) - 1ull;
  int count = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const bool keep = u[i] >= lo;
    const unsigned long long mask = __ballot(keep);
    const int pos = count + __popcll(mask & below);
    if (keep && pos < kCandCap) cand_keys[w][pos] = u[i];
    count += __popcll(mask);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t res;
  switch ((count + 63) >> 6) {
    case 1: res = qb_search_chunks<1>(cand_keys[w], count, lane, k1, prefix, 31 - d); break;
    case 2: res = qb_search_chunks<2>(cand_keys[w], count, lane, k1, prefix, 31 - d); break;
    case 3: res = qb_search_chunks<3>(cand_keys[w], count, lane, k1, prefix, 31 - d); break;
    case 4: res = qb_search_chunks<4>(cand_keys[w], count, lane, k1, prefix, 31 - d); break;
    default: {  // more candidates than the buffer holds: search all keys
      res = prefix;
      for (int bit = 31 - d; bit >= 0; --bit) {
        const uint32_t cand = res | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < PL; ++i) cnt += __popcll(__ballot(u[i] >= cand));
        if (cnt >= k1) res = cand;
      }
    }
  }
  if (lane == 0) alpha[t] = qb_unordered(res);
}

// New bias of one expert from its bins (global or LDS), one wave: lane l holds bins
// [16 l, 16 l + 16); the largest bin whose suffix count reaches q (suffix sums in
// int64); NaN when no bin does.
__device__ __forceinline__ float qb_bias_of(const int32_t* bins, int lane, long long q) {
  int c[16];
  long long lane_sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bin = lane * 16 + i;
    c[i] = bin < kBins ? bins[bin] : 0;
    lane_sum += c[i];
  }
  // exclusive suffix sum over the lanes above this one
  long long incl = lane_sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long v = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += v;
  }
  long long run = incl - lane_sum;
  int best = -1;
#pragma unroll
  for (int i = 15; i >= 0; --i) {
    run += c[i];
    if (best < 0 && run >= q) best = lane * 16 + i;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, 64));
  const float p = (float)best * 0.004f;
  const float edge = -2.0f + p;
  return best < 0 ? __uint_as_float(0x7fc00000u) : -edge;
}

// Block b takes experts [4 g, 4 g + 4) over all m tokens; g is chosen so that the
// eight groups sharing a 128-byte line of a score row run on one XCD (blocks are
// dealt to the 8 XCDs round-robin). A lane takes one row's four scores (one
// 16-byte load) per pass; eight passes' loads are issued before any margin is
// counted (clamped indices, no branches around the loads).
template <bool VEC>
__global__ __launch_bounds__(1024) void qb_hist_kernel(const float* __restrict__ s, const float* __restrict__ alpha,
                                                       int m, int n, int per_xcd, int32_t* __restrict__ hist,
                                                       long long q, float* __restrict__ new_bias) {
  __shared__ int h[kHistExperts * kBins];
  const int b = blockIdx.x;
  const int g = (b & 7) * per_xcd + (b >> 3);
  const int e0 = g * kHistExperts;
  if (e0 >= n) return;
  for (int i = threadIdx.x; i < kHistExperts * kBins; i += 1024) h[i] = 0;
  __syncthreads();
  const int ne = min(kHistExperts, n - e0);
  constexpr int kUnroll = 8;
  for (int t0 = threadIdx.x; t0 < m; t0 += 1024 * kUnroll) {
    float v[kUnroll][kHistExperts], a[kUnroll];
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int t = min(t0 + r * 1024, m - 1);
      a[r] = alpha[t];
      const float* p = s + (size_t)t * n + e0;
      if (VEC) {
        const f32x4_t x = *(const f32x4_t*)p;
#pragma unroll
        for (int q = 0; q < kHistExperts; ++q) v[r][q] = x[q];
      } else {
#pragma unroll
        for (int q = 0; q < kHistExperts; ++q) v[r][q] = p[min(q, ne - 1)];
      }
    }
#pragma unroll
    for (int r = 0; r < kUnroll; ++r)
#pragma unroll
      for (int q = 0; q < kHistExperts; ++q)
        if (q < ne && t0 + r * 1024 < m) atomicAdd(&h[q * kBins + qb_bin(v[r][q] - a[r])], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ne * kBins; i += 1024) hist[(size_t)e0 * kBins + i] = h[i];
  // the block holds its experts' complete histograms: with a target, their new bias too
  const int w = threadIdx.x >> 6;
  if (new_bias && w < ne) {
    const float b = qb_bias_of(&h[w * kBins], threadIdx.x & 63, q);
    if ((threadIdx.x & 63) == 0) new_bias[e0 + w] = b;
  }
}

// One wave per expert, four per block.
__global__ __launch_bounds__(256) void qb_bias_kernel(const int32_t* __restrict__ hist, int n, long long q,
                                                      float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const float b = qb_bias_of(hist + (size_t)j * kBins, lane, q);
  if (lane == 0) out[j] = b;
}

}  // namespace

hipError_t launch_qb_histogram(const float* scores, const float* bias, int m, int n, int k, float* alpha,
                               int32_t* hist, long long q, float* new_bias, hipStream_t st) {
  if (m > 0) {
    const dim3 grid((m + 3) / 4);
    const bool vec = n % 4 == 0;
    auto* f = n <= 1024 ? (bias ? (vec ? qb_alpha_kernel<16, true, true> : qb_alpha_kernel<16, true, false>)
                                : (vec ? qb_alpha_kernel<16, false, true> : qb_alpha_kernel<16, false, false>))
                        : (bias ? (vec ? qb_alpha_kernel<64, true, true> : qb_alpha_kernel<64, true, false>)
                                : (vec ? qb_alpha_kernel<64, false, true> : qb_alpha_kernel<64, false, false>));
    hipLaunchKernelGGL(f, grid, dim3(256), 0, st, scores, bias, m, n, k + 1, alpha);
  }
  const int groups = (n + kHistExperts - 1) / kHistExperts;
  // a multiple of 8 groups per XCD, so the 8 groups of one 128-byte line share an L2
  const int per_xcd = 8 * ((groups + 63) / 64);
  auto* h = n % 4 == 0 ? qb_hist_kernel<true> : qb_hist_kernel<false>;
  hipLaunchKernelGGL(h, dim3(8 * per_xcd), dim3(1024), 0, st, scores, alpha, m, n, per_xcd, hist, q, new_bias);
  return hipGetLastError();
}

hipError_t launch_qb_bias(const int32_t* hist, int n, long long q, float* new_bias, hipStream_t st) {
  hipLaunchKernelGGL(qb_bias_kernel, dim3((n + 3) / 4), dim3(256), 0, st, hist, n, q, new_bias);
  return hipGetLastError();
}

}  // namespace moe
