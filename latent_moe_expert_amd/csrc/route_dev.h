// Top-k selection of one token's router keys by one wave (gfx950, wave64), used by the
// per-token route kernel and the decode route launch that also sums split-K planes.
//
// Keys key_e = sigmoid(logit_e) + bias_e become unique 64-bit composites (ordered key bits,
// then the inverted expert id), so the larger composite is the larger key with ties going to
// the lower id (WASTE "Kimi K3, as released", "Against the technical report": the bias only
// selects; the weights are the unbiased scores renormalised over the selected k, times
// routed_scaling_factor).
#pragma once
#include <float.h>

#include "common.h"

namespace moe {

// Order-preserving map of a float to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kFastMaxE = 1024;  // experts per token of the register path: 16 per lane of one wave
constexpr int kFastMaxK = 16;    // its top-k

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

// ---- One wave per token: up to 64 * NPL experts (expert e = lane + 64 i in register i).
//
// The k-th largest of the 64 lane maxima, tau, bounds the k-th largest composite from below
// (k lanes hold a composite >= tau), so the k winners are among the composites >= tau. Those
// are compacted into 64 LDS slots (usually a few dozen) and bitonic-sorted across the wave;
// when more than 64 reach tau, k successive wave maxima over all composites are taken instead.
// The selected set is the k largest (unique) composites.

// lane ^ X within the wave: DPP for 1, 2 and 8 (quad permutations, row rotation by 8),
// ds_swizzle for 4 and 16, a permute for 32
template <int X>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v) {
  if constexpr (X == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  else if constexpr (X == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  else if constexpr (X == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);
  else if constexpr (X == 4 || X == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (X << 10));
  else return (uint32_t)__shfl_xor((int)v, X, 64);
}

template <int SIZE, int STRIDE>
__device__ __forceinline__ unsigned long long bitonic_step_u64(unsigned long long v, int lane) {
  const uint32_t lo = xor_lane_u32<STRIDE>((uint32_t)v);
  const uint32_t hi = xor_lane_u32<STRIDE>((uint32_t)(v >> 32));
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  // the lower lane of a pair keeps the larger value in a descending run (lane & SIZE == 0)
  const bool keep_max = ((lane & STRIDE) == 0) == ((lane & SIZE) == 0);
  return (keep_max == (o > v)) ? o : v;
}

// One composite per lane, returned sorted descending across the 64 lanes.
template <int SIZE = 2, int STRIDE = 1>
__device__ __forceinline__ unsigned long long wave_sort_desc_u64(unsigned long long v, int lane) {
  if constexpr (SIZE > 64) {
    return v;
  } else {
    v = bitonic_step_u64<SIZE, STRIDE>(v, lane);
    if constexpr (STRIDE > 1)
      return wave_sort_desc_u64<SIZE, STRIDE / 2>(v, lane);
    else
      return wave_sort_desc_u64<SIZE * 2, SIZE>(v, lane);
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct RouteWaveSmem {
  unsigned long long cand[64];
  int sel_e[kFastMaxK];
  float sel_s[kFastMaxK];
};

// Top-k (k <= kFastMaxK) of one token's composites c (zero past E) with their unbiased scores
// sc; writes the winners in ascending id order with weights s_e / sum(s_selected) * rsf, the
// sum taken in ascending id order. s_lds holds the wave's scores by expert id afterwards.
template <int NPL>
__device__ __forceinline__ void route_select_wave(unsigned long long (&c)[NPL], const float (&sc)[NPL], int k,
                                                  float rsf, int lane, float* __restrict__ s_lds,
                                                  RouteWaveSmem& sm, int32_t* __restrict__ ids_out,
                                                  float* __restrict__ w_out) {
  unsigned long long m = c[0];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    s_lds[lane + 64 * i] = sc[i];
    if (i) m = max_u64(m, c[i]);
  }
  const unsigned long long tau = readlane_u64(wave_sort_desc_u64(m, lane), k - 1);
  int n = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool cand = c[i] >= tau;  // tau is a real composite: padding (zero) never qualifies
    const unsigned long long b = __ballot(cand);
    const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
    if (cand && pos < 64) sm.cand[pos] = c[i];
    n += __popcll(b);
  }
  wave_sync_lds();
  unsigned long long my_c;
  if (n <= 64) {
    my_c = wave_sort_desc_u64(lane < n ? sm.cand[lane] : 0ull, lane);
  } else {
    float unused;
    wave_top<NPL>(c, sc, k, lane, my_c, unused);
  }
  const int my_e = (int)(0xffffffffu - (uint32_t)(my_c & 0xffffffffull));
  if (lane < k) {
    int p = 0;
    for (int j = 0; j < k; ++j) p += __builtin_amdgcn_readlane(my_e, j) < my_e ? 1 : 0;
    sm.sel_e[p] = my_e;
    sm.sel_s[p] = s_lds[my_e];
  }
  wave_sync_lds();
  float tot = 0.f;
  for (int p = 0; p < k; ++p) tot += sm.sel_s[p];  // ascending id order: a fixed rounding order
  if (lane < k) {
    ids_out[lane] = sm.sel_e[lane];
    w_out[lane] = sm.sel_s[lane] / tot * rsf;
  }
}

}  // namespace moe
