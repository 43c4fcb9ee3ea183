// Dense projections of the latent-MoE layer on MFMA (bf16 x bf16 -> fp32).
//
// The latent MoE adds two dense matmuls per layer (WASTE "Kimi K3, as released",
// "What is new since Kimi-Linear", item 1): routed_expert_down_proj 7168->3584
// and routed_expert_up_proj 3584->7168. The router logits x . W_r^T use the same
// activations, so the down-projection and the router run as one launch with two
// weight segments (K3 report review, serving section: the down-projection is
// fused with the router).
//
// Small-M kernel: each block owns 16 weight rows and up to 16*MT tokens; its four
// waves split the K loop (k-steps of 128 interleaved across waves) and reduce the
// partial tiles through LDS in a fixed order, so results are run-to-run
// deterministic. Each lane reads 32 consecutive K values of one weight row per
// k-step; MFMA lane group q = lane/16 supplies K sub-range [32q, 32q+32) of the
// step, which both operands agree on, so no data shuffles are needed.
//
// fp32 router weights are split exactly into three bf16 planes (truncation:
// w = hi + mid + lo with every term a bf16 value), so x . w is computed from
// exact bf16 products accumulated in fp32.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void split3(float f0, float f1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  uint32_t u0 = __float_as_uint(f0), u1 = __float_as_uint(f1);
  uint32_t h0 = u0 & 0xffff0000u, h1 = u1 & 0xffff0000u;
  float r0 = f0 - __uint_as_float(h0), r1 = f1 - __uint_as_float(h1);
  uint32_t m0 = __float_as_uint(r0) & 0xffff0000u, m1 = __float_as_uint(r1) & 0xffff0000u;
  float l0 = r0 - __uint_as_float(m0), l1 = r1 - __uint_as_float(m1);
  hi = (h0 >> 16) | h1;
  mid = (m0 >> 16) | m1;
  lo = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xffff0000u);
}

template <int MT>
__global__ __launch_bounds__(256) void dense_small_kernel(DenseArgs a, int nb0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int blk = blockIdx.x;
  const int si = blk < nb0 ? 0 : 1;
  const DenseSeg sg = a.seg[si];
  const int row0 = (si == 0 ? blk : blk - nb0) * 16;
  const int m0 = blockIdx.y * 16 * MT;
  const int K = a.K;
  const int nsteps = K >> 7;

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // rows past N (a weight segment whose N is not a multiple of 16) read row N-1
  // and their results are never stored
  const size_t wrow = (size_t)min(row0 + nl, sg.N - 1);
  for (int s = wave; s < nsteps; s += 4) {
    const int kb = s * 128 + q * 32;
    u32x4_t av[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m0 + mt * 16 + nl;
      if (m < a.M) {
        const uint16_t* ap = a.A + (size_t)m * a.lda + kb;
#pragma unroll
        for (int j = 0; j < 4; ++j) av[mt][j] = load_u32x4(ap + 8 * j);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) av[mt][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    if (!sg.w_f32) {
      const uint16_t* wp = (const uint16_t*)sg.W + wrow * K + kb;
      u32x4_t bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = load_nt_u32x4(wp + 8 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[mt][j]), as_bf16x8(bv[j]), acc[mt], 0, 0, 0);
    } else {
      const float* wp = (const float*)sg.W + wrow * K + kb;
      u32x4_t raw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) raw[j] = load_nt_u32x4(wp + 4 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h4[4], m4[4], l4[4];
        const u32x4_t r0 = raw[2 * j], r1 = raw[2 * j + 1];
        split3(__uint_as_float(r0[0]), __uint_as_float(r0[1]), h4[0], m4[0], l4[0]);
        split3(__uint_as_float(r0[2]), __uint_as_float(r0[3]), h4[1], m4[1], l4[1]);
        split3(__uint_as_float(r1[0]), __uint_as_float(r1[1]), h4[2], m4[2], l4[2]);
        split3(__uint_as_float(r1[2]), __uint_as_float(r1[3]), h4[3], m4[3], l4[3]);
        const u32x4_t hi = {h4[0], h4[1], h4[2], h4[3]};
        const u32x4_t mid = {m4[0], m4[1], m4[2], m4[3]};
        const u32x4_t lo = {l4[0], l4[1], l4[2], l4[3]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[mt][j]), as_bf16x8(hi), acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[mt][j]), as_bf16x8(mid), acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[mt][j]), as_bf16x8(lo), acc[mt], 0, 0, 0);
        }
      }
    }
  }

  __shared__ float red[4][MT][4][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][mt][r][lane] = acc[mt][r];
  __syncthreads();

  for (int i = threadIdx.x; i < MT * 256; i += 256) {
    const int mt = i >> 8, r = (i >> 6) & 3, ln = i & 63;
    const float v = ((red[0][mt][r][ln] + red[1][mt][r][ln]) + red[2][mt][r][ln]) + red[3][mt][r][ln];
    const int m = m0 + mt * 16 + 4 * (ln >> 4) + r;
    const int n = row0 + (ln & 15);
    if (m >= a.M || n >= sg.N) continue;
    if (sg.mode == kStoreBf16) {
      ((uint16_t*)sg.out)[(size_t)m * sg.ldo + n] = (uint16_t)f32_to_bf16_bits(v);
    } else if (sg.mode == kStoreF32) {
      ((float*)sg.out)[(size_t)m * sg.ldo + n] = v;
    } else {
      const float add = sg.addend ? sg.addend[(size_t)m * sg.ld_add + n] : 0.f;
      ((uint16_t*)sg.out)[(size_t)m * sg.ldo + n] = (uint16_t)f32_to_bf16_bits(v + add);
      if (sg.tap) sg.tap[(size_t)m * sg.ld_tap + n] = v;
    }
  }
}

}  // namespace

hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const int nb0 = (a.seg[0].N + 15) / 16;
  const int nb = nb0 + (a.nseg > 1 ? (a.seg[1].N + 15) / 16 : 0);
  int mt = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  dim3 grid(nb, (a.M + 16 * mt - 1) / (16 * mt));
  if (mt == 1)
    hipLaunchKernelGGL(dense_small_kernel<1>, grid, dim3(256), 0, s, a, nb0);
  else if (mt == 2)
    hipLaunchKernelGGL(dense_small_kernel<2>, grid, dim3(256), 0, s, a, nb0);
  else
    hipLaunchKernelGGL(dense_small_kernel<4>, grid, dim3(256), 0, s, a, nb0);
  return hipGetLastError();
}

}  // namespace moe
