// Sigmoid router with a selection-only bias and top-k (WASTE "Kimi K3, as
// released": router row of the "Shape" table -- sigmoid, 1 group,
// routed_scaling_factor 1.0 -- and "Against the technical report": the
// correction bias is used for selection only and the weights are renormalised
// over the selected top-k, then multiplied by routed_scaling_factor).
//
// One wave per token. Lane l owns experts l, l+64, l+128, ... and keeps their
// keys in LDS; k rounds of (local best, wave arg-max) pick the winners, ties
// going to the lower expert id. The k ids are then written in ascending id
// order with their weights s_j / sum(s_sel) * rsf (unbiased scores).
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void better(float& bk, int& bi, float k2, int i2) {
  // larger key wins; equal keys -> lower id
  if (k2 > bk || (k2 == bk && i2 < bi)) { bk = k2; bi = i2; }
}

__global__ __launch_bounds__(64) void router_topk_kernel(const float* __restrict__ logits, int ld,
                                                         const float* __restrict__ bias, int E, int k,
                                                         float rsf, int32_t* __restrict__ ids,
                                                         float* __restrict__ wout) {
  extern __shared__ float keys[];  // [E]
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* lg = logits + (size_t)t * ld;
  for (int e = lane; e < E; e += 64) {
    const float s = sigmoidf_dev(lg[e]);
    const float key = s + (bias ? bias[e] : 0.f);
    keys[e] = (key == key) ? key : -FLT_MAX;  // a NaN key never wins
  }
  // each lane only touches its own entries below, so no barrier is needed
  int my_sel = -1;
  for (int r = 0; r < k; ++r) {
    float bk = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = lane; e < E; e += 64) better(bk, bi, keys[e], e);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float k2 = __shfl_xor(bk, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      better(bk, bi, k2, i2);
    }
    // bi is uniform now; -INFINITY entries are taken ones (keys are > -inf otherwise)
    if (bi < 0 || bi >= E) bi = 0;  // cannot happen for finite keys and k <= E
    if ((bi & 63) == lane) keys[bi] = -INFINITY;
    if (lane == r) my_sel = bi;
  }
  // ascending id order: rank among the selected
  int rank = 0;
  for (int i = 0; i < k; ++i) {
    const int other = __shfl(my_sel, i, 64);
    rank += (lane < k && other < my_sel) ? 1 : 0;
  }
  const float s = (lane < k) ? sigmoidf_dev(lg[my_sel]) : 0.f;
  // sum of the selected scores, in selection order (a fixed rounding order)
  float ssum = 0.f;
  for (int i = 0; i < k; ++i) ssum += __shfl(s, i, 64);
  if (lane < k) {
    ids[(size_t)t * k + rank] = my_sel;
    wout[(size_t)t * k + rank] = s / ssum * rsf;
  }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int ld_logits, const float* select_bias, int T, int E, int k,
                              float rsf, int32_t* ids, float* w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_topk_kernel, dim3(T), dim3(64), (size_t)E * sizeof(float), s, logits, ld_logits,
                     select_bias, E, k, rsf, ids, w);
  return hipGetLastError();
}

}  // namespace moe
