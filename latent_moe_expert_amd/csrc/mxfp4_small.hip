// Grouped MXFP4 contractions for small token counts per expert (decode).
//
// Weights stay in the shipped MXFP4 layout (WASTE "Kimi K3, as released",
// shard-header listing and "Gate 3 repeated on real K3 experts"): a matrix
// [N, K] is U8 [N, K/2] with two E2M1 nibbles per byte, low nibble first, plus
// one E8M0 exponent per 32 consecutive weights of a row, U8 [N, K/32].
//
// Work unit: one 16-slot block of the expert-sorted layout (or 16 rows of a
// dense batch) x a band of weight rows. In each k-step of 128, lane (n = l%16,
// q = l/16) loads 16 bytes = one whole scale group (32 weights) of weight row n,
// plus its E8M0 code, and converts them with the scaled FP4->bf16 instruction
// (exact for every code); the matching 32 activations of token n come straight
// from global memory as bf16. Four bf16 MFMA 16x16x32 consume the group: lane
// group q supplies K sub-range [32q, 32q+32) of the step for both operands, so
// the contraction needs no shuffles. One pass streams every weight byte exactly
// once per 16 tokens; decode is bound by those bytes (the experts' I/O is the
// per-token cost the pages measure).
//
// GLU variant: a wave holds tiles of the gate (w1) and up (w3) rows with the
// same indices, so the epilogue applies act(gate) * up in registers and writes
// bf16 h; the plain variant (w2, or the shared down) writes fp32.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <bool GLU, int NTW>
__global__ __launch_bounds__(256) void mx_small_kernel(MxArgs a) {
  constexpr int CH = GLU ? 2 * NTW : NTW;  // 16-row weight tiles per wave per k-step
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int blk = blockIdx.y;

  int expert = 0;
  if (a.routed) {
    if (blk * 16 >= *a.num_post) return;
    expert = a.expert_ids[blk / a.tiles_per_block];  // layout blocks of B = 16*tiles_per_block slots
    if (expert < 0) return;
  } else if (blk * 16 >= a.M) {
    return;
  }
  const int row0 = (blockIdx.x * 4 + wave) * NTW * 16;  // first weight row of this wave
  if (row0 >= a.N) return;

  // activation row feeding MFMA row nl
  int arow = -1;
  {
    const int pos = blk * 16 + nl;
    if (a.routed) {
      const int sid = a.sorted_ids[pos];
      if (sid < a.pairs) arow = a.a_by_pos ? pos : sid / a.topk;
    } else if (pos < a.M) {
      arow = pos;
    }
  }
  const uint16_t* aptr = arow >= 0 ? a.A + (size_t)arow * a.lda + q * 32 : nullptr;

  const int K = a.K;
  const int nsteps = K >> 7;
  const size_t kb2 = (size_t)K / 2, ks32 = (size_t)K / 32;
  const uint8_t* wbase[CH];
  const uint8_t* sbase[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int tile = GLU ? (c % NTW) : c;
    const uint8_t* Wm = (GLU && c >= NTW) ? a.W2 : a.W;
    const uint8_t* Sm = (GLU && c >= NTW) ? a.S2 : a.S;
    const size_t row = (size_t)(row0 + tile * 16 + nl);
    wbase[c] = Wm + (size_t)expert * a.w_stride + row * kb2 + q * 16;
    sbase[c] = Sm + (size_t)expert * a.s_stride + row * ks32 + q;
  }

  f32x4_t acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // software pipeline: loads of step s+1 are issued before the math of step s
  u32x4_t wcur[CH], wnxt[CH];
  uint32_t scur[CH], snxt[CH];
  u32x4_t acur[4], anxt[4];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    wcur[c] = load_nt_u32x4(wbase[c]);
    scur[c] = sbase[c][0];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acur[j] = aptr ? load_u32x4(aptr + 8 * j) : u32x4_t{0u, 0u, 0u, 0u};

  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        wnxt[c] = load_nt_u32x4(wbase[c] + (size_t)(s + 1) * 64);
        snxt[c] = sbase[c][(s + 1) * 4];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        anxt[j] = aptr ? load_u32x4(aptr + (size_t)(s + 1) * 128 + 8 * j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float sc = e8m0_as_f32_exponent(scur[c]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t bw[4];
        fp4x8_to_bf16x8(wcur[c][j], sc, bw);
        const u32x4_t bv = {bw[0], bw[1], bw[2], bw[3]};
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(acur[j]), as_bf16x8(bv), acc[c], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        wcur[c] = wnxt[c];
        scur[c] = snxt[c];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acur[j] = anxt[j];
    }
  }

  // epilogue: lane holds D[m = 4q + r][n = nl] of each tile
  bool valid[4];
  int opos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = blk * 16 + 4 * q + r;
    opos[r] = pos;
    valid[r] = a.routed ? (a.sorted_ids[pos] < a.pairs) : (pos < a.M);
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int col = row0 + t * 16 + nl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!valid[r]) continue;
      if (GLU) {
        const float h = glu_act(acc[t][r], acc[NTW + t][r]);
        ((uint16_t*)a.out)[(size_t)opos[r] * a.ldo + col] = (uint16_t)f32_to_bf16_bits(h);
      } else {
        ((float*)a.out)[(size_t)opos[r] * a.ldo + col] = acc[t][r];
      }
    }
  }
}

template <bool GLU, int NTW>
hipError_t launch_t(const MxArgs& a, hipStream_t s) {
  const int rows_per_block = 4 * NTW * 16;
  dim3 grid((a.N + rows_per_block - 1) / rows_per_block, a.max_blocks);
  hipLaunchKernelGGL((mx_small_kernel<GLU, NTW>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_small(const MxArgs& a, hipStream_t s) {
  if (a.max_blocks <= 0) return hipSuccess;
  const bool glu = a.W2 != nullptr;
  // narrower bands when few token blocks would leave the chip idle
  const bool narrow = a.max_blocks * (a.N / (glu ? 128 : 256)) < 512;
  if (glu) return narrow ? launch_t<true, 1>(a, s) : launch_t<true, 2>(a, s);
  return narrow ? launch_t<false, 1>(a, s) : launch_t<false, 4>(a, s);
}

}  // namespace moe
