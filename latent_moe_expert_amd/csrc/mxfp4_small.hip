// Grouped MXFP4 contractions for small token counts per expert (decode).
//
// Weights stay in the shipped MXFP4 layout (WASTE "Kimi K3, as released",
// shard-header listing and "Gate 3 repeated on real K3 experts"): a matrix
// [N, K] is U8 [N, K/2] with two E2M1 nibbles per byte, low nibble first, plus
// one E8M0 exponent per 32 consecutive weights of a row, U8 [N, K/32].
//
// Work unit: one 16-slot tile of the expert-sorted layout (or 16 rows of a
// dense batch) x 64 weight rows per wave (GLU: 32 gate rows and the same 32 up
// rows; plain: 64 rows), 4 waves per block, full K per wave; the routed tiles
// of a launch's last round take half the weight rows per wave. The block loads
// the tile's activations once per step into a shared, swizzled LDS tile.
//
// Memory path. Decode streams each touched expert's bytes once, so the kernel
// lives on HBM efficiency. Every weight load instruction of a wave covers 8
// whole rows x 128 contiguous bytes (256 weights = two k-steps of a row): on
// MI355X that pattern streams as fast as a contiguous copy, while the MFMA's
// native fragment (16 rows x 64 bytes per instruction) measured about 27%
// slower. The bytes go through a wave-private LDS tile, XOR-swizzled so that
// both the 16-byte writes and the MFMA fragment reads are bank-conflict free,
// and no barrier is needed for them. Activations come in through buffer loads:
// slots without a token get an out-of-range offset, read as zeros with no
// memory traffic.
//
// Math. Lane (n = l%16, q = l/16) of an MFMA fragment holds one whole E8M0
// group (32 weights of row n); the scaled FP4->bf16 conversion applies the
// group's scale exactly, and four bf16 MFMA 16x16x32 consume the group against
// the matching 32 activations (lane group q supplies the same K sub-range in
// both operands, so no reordering of K is visible in the result).
//
// Rows: a routed problem reads its A row of slot position pos as the slot's token,
// the position itself or the flat slot index (RowMode), and writes its output row at
// the position or the flat slot index; the layer keeps h and O one row per
// (token, slot), so their size follows T * k, not the padded layout.
//
// GLU variant: the epilogue applies act(gate) * up in registers and writes
// bf16 h (with MXFP8 activations: each row's 32 columns of a wave are one
// block, rounded to their MXFP8 values first); the plain variant (w2, or the
// shared down) writes fp32.
#include "common.h"
#include "kernels.h"
#include "mxfp8.h"

namespace moe {

namespace {

// NTW: 16-row weight tiles per wave (GLU: NTW/2 gate tiles and the same up tiles). One block:
// 4 waves, one 16-slot tile `blk` of problem `a` against the column band `band`.
template <bool GLU, int NTW>
__device__ __forceinline__ void mx_small_block(const MxProblem& a, int band, int blk, uint8_t (*lds_w)[4 * 16 * 128],
                                               uint8_t (*lds_a)[16 * 512]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nl = lane & 15, q = lane >> 4;
  uint8_t* lds = lds_w[wave];

  // block-uniform exits only (the loop below has block barriers)
  int expert = 0;
  if (a.routed) {
    if (blk * 16 >= *a.num_post) return;
    expert = a.expert_ids[blk / a.tiles_per_block];  // layout blocks of B = 16*tiles_per_block slots
    if (expert < 0) return;
  } else if (blk * 16 >= a.M) {
    return;
  }
  constexpr int kColsPerWave = GLU ? 8 * NTW : 16 * NTW;
  const int col0 = (band * 4 + wave) * kColsPerWave;  // N is a multiple of the block's columns

  const int K = a.K;
  const uint32_t kb2 = (uint32_t)K / 2, ks32 = (uint32_t)K / 32;
  const uint32_t mat_bytes = (uint32_t)a.N * kb2, mat_scales = (uint32_t)a.N * ks32;
  const __amdgpu_buffer_rsrc_t w_lo = make_rsrc(a.W + (size_t)expert * a.w_stride, mat_bytes);
  const __amdgpu_buffer_rsrc_t s_lo = make_rsrc(a.S + (size_t)expert * a.s_stride, mat_scales);
  const __amdgpu_buffer_rsrc_t w_hi = GLU ? make_rsrc(a.W2 + (size_t)expert * a.w_stride, mat_bytes) : w_lo;
  const __amdgpu_buffer_rsrc_t s_hi = GLU ? make_rsrc(a.S2 + (size_t)expert * a.s_stride, mat_scales) : s_lo;

  // Wave tile t (16 rows) starts at row col0 + 16*tt(t) of its matrix, tt(t) = t&1 (GLU: t<2 gate,
  // t>=2 up) or t (plain). Load l (0..7) of a double step covers the wave's slots 8l..8l+7;
  // lane = (slot 8l + lane/8, 16-byte chunk lane%8). Row offsets are uniform per l.
  auto tt = [](int t) { return GLU ? t % (NTW / 2) : t; };
  const uint32_t gbase = (uint32_t)(col0 + (lane >> 3)) * kb2 + (lane & 7) * 16;
  // LDS: slot j, chunk c lives at j*128 + ((c ^ (j & 7)) * 16); for load l, j & 7 = lane >> 3
  const uint32_t wbase = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16);
  // fragment of tile t, step h: slot 16t + nl, chunk 4h + q
  const uint32_t rbase0 = nl * 128 + (((q) ^ (nl & 7)) * 16);
  const uint32_t rbase1 = nl * 128 + (((4 + q) ^ (nl & 7)) * 16);
  const uint32_t sbase = (uint32_t)(col0 + nl) * ks32;  // scales: 8 bytes per row per double step

  // activation tile: thread tid fills slot tid/16, chunks tid%16 and tid%16 + 16 (16 bytes each)
  uint32_t aoff_fill;
  {
    const int slot = tid >> 4;
    const int pos = blk * 16 + slot;
    int arow = -1;
    if (a.routed) {
      const int sid = a.sorted_ids[pos];
      if (sid < a.pairs) arow = a.a_row == kRowPos ? pos : (a.a_row == kRowFlat ? sid : sid / a.topk);
    } else if (pos < a.M) {
      arow = pos;
    }
    aoff_fill = arow >= 0 ? ((uint32_t)arow * (uint32_t)a.lda) * 2 + (tid & 15) * 16 : kOob;
  }
  const uint32_t a_step = aoff_fill == kOob ? 0u : 512u;
  const int fslot = tid >> 4, fc = tid & 15;
  const uint32_t afill0 = fslot * 512 + (((fc) ^ fslot) * 16);
  const uint32_t afill1 = fslot * 512 + (((fc + 16) ^ fslot) * 16);
  // fragment reads: lane (nl, q), step h, MFMA j: chunk h*16 + 4q + j of slot nl
  uint32_t aread[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aread[j] = nl * 512 + (((4 * q + j) ^ nl) * 16);
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(a.A, 0x7fffffffu);

  f32x4_t acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    u32x4_t w[2 * NTW];
    uint2 sc[NTW];
  };
  u32x4_t anext[2];
  // A double step past the end loads from a zero-size resource (zeros, no memory traffic), so
  // every step issues the same loads with no branch: a load under a branch makes the
  // compiler wait for every load in flight before the next use of any of them.
  const __amdgpu_buffer_rsrc_t none = make_rsrc(a.W, 0u);
  auto issue = [&](Stage& st, int d) {
    const bool on = d < (K >> 8);
    {  // activations first: they are waited on before this step's weights
      const uint32_t ao = aoff_fill + (uint32_t)d * a_step;
      anext[0] = buf_load16(on ? a_rs : none, ao);
      anext[1] = buf_load16(on ? a_rs : none, aoff_fill == kOob ? kOob : ao + 256);
    }
    const uint32_t vo = gbase + (uint32_t)d * 128;  // 256 weights of a row per double step
#pragma unroll
    for (int l = 0; l < 2 * NTW; ++l) {
      const int t = l >> 1;
      const uint32_t so = (uint32_t)(16 * tt(t) + 8 * (l & 1)) * kb2;
      st.w[l] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                on ? ((GLU && t >= NTW / 2) ? w_hi : w_lo) : none, vo, so, kNonTemporal));
    }
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const uint32_t so = (uint32_t)(16 * tt(t)) * ks32 + (uint32_t)d * 8;
      st.sc[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                               on ? ((GLU && t >= NTW / 2) ? s_hi : s_lo) : none, sbase, so, 0));
    }
  };
  auto fill_a = [&](int buf) {
    *(u32x4_t*)(lds_a[buf] + afill0) = anext[0];
    *(u32x4_t*)(lds_a[buf] + afill1) = anext[1];
  };
  auto consume = [&](const Stage& st, int buf) {
#pragma unroll
    for (int l = 0; l < 2 * NTW; ++l) *(u32x4_t*)(lds + l * 1024 + wbase) = st.w[l];
    const uint8_t* at = lds_a[buf];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = *(const u32x4_t*)(at + h * 256 + aread[j]);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const u32x4_t wf = *(const u32x4_t*)(lds + t * 2048 + (h ? rbase1 : rbase0));
        const uint32_t code = ((h ? st.sc[t].y : st.sc[t].x) >> (8 * q)) & 0xffu;
        const float sc = e8m0_as_f32_exponent(code);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t bw[4];
          fp4x8_to_bf16x8(wf[j], sc, bw);
          const u32x4_t bv = {bw[0], bw[1], bw[2], bw[3]};
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x[j]), as_bf16x8(bv), acc[t], 0, 0, 0);
        }
      }
    }
  };

  // Pipeline: step d's weights sit in registers and its activations in lds_a[d & 1] while
  // step d+1's loads are in flight; one barrier per step publishes the next activation tile.
  const int nd = K >> 8;  // double steps (K is a multiple of 256)
  // Steps past the last one load zeros and fill an activation buffer that is not read again.
  Stage s0, s1;
  issue(s0, 0);
  fill_a(0);
  __syncthreads();
  int d = 0;
  for (; d + 2 <= nd; d += 2) {
    issue(s1, d + 1);
    consume(s0, d & 1);
    fill_a((d + 1) & 1);
    __syncthreads();
    issue(s0, d + 2);
    consume(s1, (d + 1) & 1);
    fill_a((d + 2) & 1);
    __syncthreads();
  }
  if (d < nd) consume(s0, d & 1);

  // epilogue: lane holds D[m = 4q + r][n = nl] of each tile
  bool valid[4];
  int opos[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = blk * 16 + 4 * q + r;
    const int sid = a.routed ? a.sorted_ids[pos] : 0;
    opos[r] = a.routed && a.out_row == kRowFlat ? sid : pos;
    valid[r] = a.routed ? (sid < a.pairs) : (pos < a.M);
  }
  if (GLU) {
    // with NTW == 4 a wave's 32 columns of a row are one MXFP8 group: lanes 16q..16q+15 (tiles 0
    // and 1) of row 4q + r (the launcher runs MXFP8 outputs with NTW == 4 only)
    float hv[NTW / 2][4];
#pragma unroll
    for (int t = 0; t < NTW / 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[t][r] = glu_act(acc[t][r], acc[t + NTW / 2][r], a.act);
    if (NTW == 4 && a.out_fp8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = fmaxf(fabsf(hv[0][r]), fabsf(hv[1][r]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        const int sx = mxfp8_scale_exp(m);
#pragma unroll
        for (int t = 0; t < NTW / 2; ++t) hv[t][r] = ldexpf(e4m3_round(ldexpf(hv[t][r], -sx)), sx);
      }
    }
#pragma unroll
    for (int t = 0; t < NTW / 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (valid[r])
          ((uint16_t*)a.out)[(size_t)opos[r] * a.ldo + col0 + t * 16 + nl] = (uint16_t)f32_to_bf16_bits(hv[t][r]);
  } else {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (valid[r]) ((float*)a.out)[(size_t)opos[r] * a.ldo + col0 + t * 16 + nl] = acc[t][r];
  }
}

// Block -> (problem, column band, 16-slot tile); problem 0 first. With half_tiles > 0 the last
// min(half_tiles, V) valid tiles of problem 1 (V = its valid 16-slot tiles, known on the device)
// run as blocks of half the columns (NTW = 2), placed after every full-width block, so the launch
// ends on blocks half as long. Per-block timestamps at decode16 (three blocks resident per compute
// unit, 768 in all): as the last full-width blocks finish, the compute units go idle over about one block duration (30-38 us), which cost ~17 us
// of the gate/up launch and ~13 us of the down launch against their steady 6.1 TB/s; with the
// half-width tail the launches took 431 and 224 us against 435 and 226 (decode step 0.716
// against 0.720 ms). All blocks half-width measured slower (0.729 ms): per weight byte a
// half-width block reads its activation tile twice as often.
template <bool GLU, bool HALF>
__global__ __launch_bounds__(256) void mx_small_kernel(MxArgs args, int blocks0, int bands0, int bands1, int full1,
                                                       int half_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[4][4 * 16 * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][16 * 512];
  const bool second = (int)blockIdx.x >= blocks0;
  const int local = second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x;
  const MxProblem& a = args.p[second ? 1 : 0];
  if (HALF && second) {
    const int V = min((*a.num_post + 15) >> 4, a.max_blocks), X = min(half_tiles, V);
    if (local >= full1) {  // half-width blocks: tile V - X + h / (2 bands1)
      const int h = local - full1, t = h / (2 * bands1);
      if (t >= X) return;
      mx_small_block<GLU, 2>(a, h % (2 * bands1), V - X + t, lds_w, lds_a);
      return;
    }
    if (local / bands1 >= V - X) return;  // its tile runs as half-width blocks
  }
  const int bands = second ? bands1 : bands0;
  mx_small_block<GLU, 4>(a, local % bands, local / bands, lds_w, lds_a);
}

}  // namespace

hipError_t launch_mx_small(const MxArgs& a, hipStream_t s) {
  const bool glu = a.p[0].W2 != nullptr;
  const int cols_per_block = 4 * (glu ? 32 : 64);
  int bands[2] = {0, 0}, blocks[2] = {0, 0};
  for (int i = 0; i < a.nprob; ++i) {
    // every wave of a block takes part in the block barriers: no partial column bands
    if (a.p[i].N % cols_per_block || a.p[i].K % 256) return hipErrorInvalidValue;
    bands[i] = a.p[i].N / cols_per_block;
    blocks[i] = a.p[i].max_blocks > 0 ? bands[i] * a.p[i].max_blocks : 0;
  }
  // The routed problem's last tiles as half-width blocks, about kTailBlocks full blocks' worth
  // (decode16 step 0.720, 0.713, 0.716 and 0.717 ms with 0, 512, 768 and 1024; 256 no better than
  // 512). Not for MXFP8 outputs of h, whose groups are one full-width wave's 32 columns.
  constexpr int kTailBlocks = 512;
  const int r = a.nprob - 1;
  const bool half = a.p[r].routed && !(glu && a.p[r].out_fp8) && bands[r] > 0;
  const int half_tiles = half ? (kTailBlocks + bands[r] - 1) / bands[r] : 0;
  const long long extra = half ? (long long)half_tiles * 2 * bands[r] : 0;
  const long long total = (long long)blocks[0] + blocks[1] + extra;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffll) return hipErrorInvalidValue;
  // with one problem it is problem "1" of the kernel's mapping (blocks0 = 0)
  const int b0 = a.nprob > 1 ? blocks[0] : 0, bd0 = a.nprob > 1 ? bands[0] : 1, bd1 = bands[r], full1 = blocks[r];
  MxArgs args = a;
  if (a.nprob == 1) args.p[1] = a.p[0];
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(256), 0, s, args, b0, bd0, bd1, full1, half_tiles);
  };
  if (glu) {
    if (half) go(mx_small_kernel<true, true>);
    else go(mx_small_kernel<true, false>);
  } else {
    if (half) go(mx_small_kernel<false, true>);
    else go(mx_small_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace moe
