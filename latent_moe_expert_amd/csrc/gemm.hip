// Dense projections for batches of more than 64 tokens: C = A . W^T in bf16 MFMA.
//
// The layer's two dense matmuls (down-projection with the router logits, and the
// up-projection; WASTE "Kimi K3, as released", section "Shape", and the K3
// report review, "Stable LatentMoE") are plain contractions over K-contiguous
// rows: A [M, K] activations, W [N, K] weights, both row-major.
//
// Tile: 128 x 128 outputs per block, 4 waves in 2 x 2, each 64 x 64 (4 x 4 MFMA
// 16x16x32 bf16 tiles), K in steps of 64 (one 128-byte line per row). Operand
// tiles go to LDS by LDS-DMA, full lines per row, into a ring of four stages
// three k-steps ahead; each stage is its own LDS array with a compile-time index,
// and the waits are explicit counts (every k-step issues the same 8 loads per
// thread). The 16-byte chunks of a row are XOR-rotated by (row / 2) % 8, which
// makes the MFMA fragment reads (16 rows x 16 bytes per lane group) bank-conflict
// free.
//
// Grid order: contiguous ranges of logical tiles per XCD (grid position mod 8);
// logical tiles run in groups of 8 M tiles with M fastest, so the blocks an XCD
// runs together share W tiles and reuse A tiles across N from its L2 (one M tile
// at a time across all of N streamed the weights once per M tile).
//
// fp32 weights (the router, fp32 on the K3 checkpoint) are first split exactly
// into three bf16 planes hi + mid + lo (24 significand bits = 3 x 8) stored as
// one [N, 3K] matrix; the contraction then runs over 3K with A's column k mod K,
// which gives the fp32-weight product with fp32 accumulation.
#include <algorithm>
#include <queue>
#include <type_traits>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGM = 8;  // M tiles per group of the grid order
constexpr int kLargeM = 2048;  // from this many rows on, the 256 x 224 tile
constexpr int kTile = kBM * kBK * 2;           // bytes of one operand tile in a stage
constexpr int kGemmDma = 2 * kTile / 16 / 256;  // 16-byte LDS-DMA chunks per thread per k-step (A and W)
static_assert(kGemmDma == 8, "");

template <int I>
using icg = std::integral_constant<int, I>;

#define MOE_GEMM_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | ((((n) >> 4) & 3) << 14))

__device__ __forceinline__ void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keeps the loads issued before it ahead of the LDS reads and MFMAs that follow: left to
// itself the scheduler sinks the next stage's LDS-DMA loads below the current stage's
// compute, and the wait at the end of the k-step then finds them all still in flight.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void dma16g(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff,
                                           0, 0);
}

// LDS position of 16-byte chunk c (0..7) of tile row r
__host__ __device__ constexpr int g_pos(int c, int r) { return c ^ ((r >> 1) & 7); }

// LDS position of 16-byte chunk c (0..3) of a 64-byte tile row r: rows 4 apart share a bank
// cycle, so the chunk is XOR-rotated by (r / 4) % 4
__host__ __device__ constexpr int g_pos2(int c, int r) { return c ^ ((r >> 2) & 3); }

// One of the two segments as a value, chosen field by field (a select between references to
// the kernel argument makes the compiler copy the arguments to scratch and index them there).
// Every field of GemmSeg is copied; r starts zeroed so that a field left out reads as zero.
__device__ __forceinline__ GemmSeg pick_seg(const GemmArgs& a, bool second) {
  const GemmSeg& x = a.seg[0];
  const GemmSeg& y = a.seg[1];
  GemmSeg r{};
  r.W = second ? y.W : x.W;
  r.N = second ? y.N : x.N;
  r.K = second ? y.K : x.K;
  r.kwrap = second ? y.kwrap : x.kwrap;
  r.mode = second ? y.mode : x.mode;
  r.out = second ? y.out : x.out;
  r.ldo = second ? y.ldo : x.ldo;
  r.addend = second ? y.addend : x.addend;
  r.ld_add = second ? y.ld_add : x.ld_add;
  r.tap = second ? y.tap : x.tap;
  r.ld_tap = second ? y.ld_tap : x.ld_tap;
  r.splits = second ? y.splits : x.splits;
  r.w_f32 = second ? y.w_f32 : x.w_f32;
  r.addend16 = second ? y.addend16 : x.addend16;
  return r;
}

// Epilogue of both tiles, the weights having been the MFMA's A operand: acc[i][j][r] is
// D[row0 + 16 i][col0 + 16 j + r]. One loop per output form (a branch on the form inside the
// tile loops made the 256 x 224 tile spill its accumulators), each storing a lane's four
// columns as one 8- or 16-byte store (with one 16-byte addend load) when the row strides and N
// allow it, else element by element.
template <int MI, int NJ, typename F>
__device__ __forceinline__ void gemm_tiles(const f32x4_t (&acc)[MI][NJ], int M, int N, int row0, int col0, F f) {
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = row0 + 16 * i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = col0 + 16 * j;
      if (col < N) f(row, col, acc[i][j]);
    }
  }
}

template <int MI, int NJ>
__device__ __forceinline__ void gemm_epilogue_rows(const f32x4_t (&acc)[MI][NJ], const GemmSeg& sg, int M, int row0,
                                                   int col0, int slice) {
  const int N = sg.N;
  const bool add = sg.mode == kAddStoreBf16;
  const bool vec = sg.ldo % 4 == 0 && N % 4 == 0 && (!add || !(sg.addend || sg.addend16) || sg.ld_add % 4 == 0) &&
                   (!add || !sg.tap || sg.ld_tap % 4 == 0);
  uint16_t* outh = (uint16_t*)sg.out;
  if (add && sg.addend16) {  // bf16 addend
    const uint16_t* ad = sg.addend16;
    float* tap = sg.tap;
    if (vec)
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
        const uint2 b = *(const uint2*)(ad + (size_t)row * sg.ld_add + col);
        const f32x4_t y = v + f32x4_t{bf16_bits_to_f32(b.x & 0xffffu), bf16_bits_to_f32(b.x >> 16),
                                      bf16_bits_to_f32(b.y & 0xffffu), bf16_bits_to_f32(b.y >> 16)};
        *(uint2*)(outh + (size_t)row * sg.ldo + col) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        if (tap) *(f32x4_t*)(tap + (size_t)row * sg.ld_tap + col) = v;
      });
    else
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e >= N) continue;
          const float a = bf16_bits_to_f32(ad[(size_t)row * sg.ld_add + col + e]);
          outh[(size_t)row * sg.ldo + col + e] = (uint16_t)f32_to_bf16_bits(v[e] + a);
          if (tap) tap[(size_t)row * sg.ld_tap + col + e] = v[e];
        }
      });
  } else if (add) {
    const float* ad = sg.addend;
    float* tap = sg.tap;
    if (vec)
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
        const f32x4_t a = ad ? *(const f32x4_t*)(ad + (size_t)row * sg.ld_add + col) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        const f32x4_t y = v + a;
        *(uint2*)(outh + (size_t)row * sg.ldo + col) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        if (tap) *(f32x4_t*)(tap + (size_t)row * sg.ld_tap + col) = v;
      });
    else
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e >= N) continue;
          const float a = ad ? ad[(size_t)row * sg.ld_add + col + e] : 0.f;
          outh[(size_t)row * sg.ldo + col + e] = (uint16_t)f32_to_bf16_bits(v[e] + a);
          if (tap) tap[(size_t)row * sg.ld_tap + col + e] = v[e];
        }
      });
  } else if (sg.mode == kStoreF32 || sg.mode == kPartF32) {
    float* outf = (float*)sg.out + (sg.mode == kPartF32 ? (size_t)slice * M * sg.ldo : 0);
    if (vec)
      gemm_tiles(acc, M, N, row0, col0,
                 [&](int row, int col, const f32x4_t& v) { *(f32x4_t*)(outf + (size_t)row * sg.ldo + col) = v; });
    else
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < N) outf[(size_t)row * sg.ldo + col + e] = v[e];
      });
  } else {
    if (vec)
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
        *(uint2*)(outh + (size_t)row * sg.ldo + col) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      });
    else
      gemm_tiles(acc, M, N, row0, col0, [&](int row, int col, const f32x4_t& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < N) outh[(size_t)row * sg.ldo + col + e] = (uint16_t)f32_to_bf16_bits(v[e]);
      });
  }
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[2 * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t st1[2 * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t st2[2 * kTile];
  __shared__ __attribute__((aligned(16))) uint8_t st3[2 * kTile];
  auto stage = [&](auto I_) -> uint8_t* {
    constexpr int I = decltype(I_)::value % 4;
    if constexpr (I == 0) return st0;
    else if constexpr (I == 1) return st1;
    else if constexpr (I == 2) return st2;
    else return st3;
  };
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- block -> (segment, K slice, M tile, N tile): segment 0's blocks first, each
  // segment's K slices one after another
  const int tm = (args.M + kBM - 1) / kBM;
  int tns[2] = {0, 0}, nbs[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i < args.nseg) {
      tns[i] = (args.seg[i].N + kBN - 1) / kBN;
      nbs[i] = tm * tns[i] * max(1, args.seg[i].splits);
    }
  }
  const int total = nbs[0] + nbs[1];
  const int per = (total + 7) >> 3;
  const int lb = (int)blockIdx.x >> 3;
  if (lb >= per) return;
  const int L = ((int)blockIdx.x & 7) * per + lb;
  if (L >= total) return;
  const bool second = L >= nbs[0];
  const GemmSeg sg = pick_seg(args, second);
  const int tn = second ? tns[1] : tns[0];
  const int local = second ? L - nbs[0] : L;
  const int slice = local / (tm * tn), tl = local % (tm * tn);
  // grouped order: groups of kGM M tiles, M fastest inside a group, so the blocks that run
  // together on an XCD share their W tiles (and each A tile is reused across N in L2)
  const int grp = tl / (kGM * tn), rem = tl % (kGM * tn);
  const int gm = min(kGM, tm - grp * kGM);
  const int mt = grp * kGM + rem % gm, nt = rem / gm;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int K = sg.K, kwrap = sg.kwrap;
  // The ring, shared by both weight formats. K-step ks reads stage ks % 4; it issues the loads
  // of ks + 3 into the stage read by ks - 1, then waits for stage ks + 1 (issued in ks - 2: two
  // k-steps' loads follow it). Steps past nks load zeros (a K slice need not be a multiple of 4
  // steps). bf16 weights: k-steps of 64 K, A and W rows of 128 bytes (4 + 4 loads per thread).
  // fp32 weights: k-steps of 32 K, A rows of 64 bytes and W rows of 128 bytes (2 + 4 loads);
  // each fp32 fragment pair is split exactly into three bf16 planes, one MFMA each.
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto core = [&](auto F32_) {
    constexpr bool F32 = decltype(F32_)::value;
    constexpr int kKs = F32 ? 32 : 64;        // K values per k-step
    constexpr int kAL = F32 ? 2 : 4;          // A loads per thread per k-step
    constexpr int kDma = kAL + 4;             // + 4 W loads
    constexpr uint32_t kWes = F32 ? 4u : 2u;  // bytes per weight
    // this block's k-steps: [kb0, kb0 + nks) (a K slice, or all of K)
    const int nks_all = K / kKs, nsl = max(1, sg.splits);
    const int kper = (nks_all + nsl - 1) / nsl;
    const int kb0 = slice * kper;
    const int nks = max(0, min(nks_all, kb0 + kper) - kb0);

    // LDS-DMA of one k-step: A chunk t = tid + 256 i (i < kAL) is row t / (kKs / 8) of the A
    // tile at LDS byte 16 t; W chunk t = tid + 256 i is row t / 8 of the W tile at byte
    // kTile + 16 t; the global chunk of each LDS position undoes the XOR (its own inverse).
    const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(args.A, (uint32_t)args.M * (uint32_t)args.lda * 2u);
    const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(sg.W, (uint32_t)sg.N * (uint32_t)K * kWes);
    const __amdgpu_buffer_rsrc_t none = make_rsrc(sg.W, 0u);
    uint32_t goff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      if (i < kAL) {
        const int t = tid + 256 * i;
        const int r = F32 ? t >> 2 : t >> 3, pos = F32 ? t & 3 : t & 7;
        const int c = F32 ? g_pos2(pos, r) : g_pos(pos, r);
        const int row = m0 + r;
        goff[i] = row < args.M ? ((uint32_t)row * (uint32_t)args.lda + 8u * c) * 2u : kOob;
      } else {
        const int t = tid + 256 * (i - kAL), r = t >> 3, pos = t & 7;
        const int c = g_pos(pos, r);
        const int row = n0 + r;
        goff[i] = row < sg.N ? ((uint32_t)row * (uint32_t)K + (16u / kWes) * c) * kWes : kOob;
      }
    }
    auto dma = [&](uint8_t* st, int j, bool on) {  // kDma loads of the block's k-step j
      const int ks = kb0 + j;
      const uint32_t ka = (uint32_t)((ks * kKs) % kwrap) * 2u, kw = (uint32_t)(ks * kKs) * kWes;
#pragma unroll
      for (int i = 0; i < kDma; ++i)
        dma16g(on ? (i < kAL ? a_rs : w_rs) : none,
               st + (i < kAL ? 0 : kTile) + (i < kAL ? i : i - kAL) * 4096 + wave * 1024, goff[i],
               i < kAL ? ka : kw);
    };

    auto compute = [&](const uint8_t* st) {
      if constexpr (!F32) {
        // lane (nl, q) of A tile mi reads row 64 wm + 16 mi + nl, chunk 4 kk + q
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint32_t ard = (uint32_t)((wm * 64 + nl) * 128 + g_pos(4 * kk + q, nl) * 16);
          const uint32_t brd = (uint32_t)(kTile + (wn * 64 + nl) * 128 + g_pos(4 * kk + q, nl) * 16);
          u32x4_t av[4], bv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) av[i] = *(const u32x4_t*)(st + ard + i * 16 * 128);
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[j] = *(const u32x4_t*)(st + brd + j * 16 * 128);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] =  // weights as the MFMA's A operand: acc[i][j] holds the tile transposed
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bv[j]), as_bf16x8(av[i]), acc[i][j], 0, 0, 0);
        }
      } else {
        // A: row 64 wm + 16 mi + nl of 64-byte rows, chunk q (K 8q .. 8q + 7); W: the same K of
        // row 64 wn + 16 nj + nl as fp32, chunks 2q and 2q + 1 of its 128-byte row
        const uint32_t ard = (uint32_t)((wm * 64 + nl) * 64 + g_pos2(q, nl) * 16);
        const uint32_t brd0 = (uint32_t)(kTile + (wn * 64 + nl) * 128 + g_pos(2 * q, nl) * 16);
        const uint32_t brd1 = (uint32_t)(kTile + (wn * 64 + nl) * 128 + g_pos(2 * q + 1, nl) * 16);
        u32x4_t av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = *(const u32x4_t*)(st + ard + i * 16 * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t w0 = *(const u32x4_t*)(st + brd0 + j * 16 * 128);
          const u32x4_t w1 = *(const u32x4_t*)(st + brd1 + j * 16 * 128);
          uint32_t h4[4], m4[4], l4[4];
          split3x2(__uint_as_float(w0[0]), __uint_as_float(w0[1]), h4[0], m4[0], l4[0]);
          split3x2(__uint_as_float(w0[2]), __uint_as_float(w0[3]), h4[1], m4[1], l4[1]);
          split3x2(__uint_as_float(w1[0]), __uint_as_float(w1[1]), h4[2], m4[2], l4[2]);
          split3x2(__uint_as_float(w1[2]), __uint_as_float(w1[3]), h4[3], m4[3], l4[3]);
          const u32x4_t hi = {h4[0], h4[1], h4[2], h4[3]};
          const u32x4_t mi = {m4[0], m4[1], m4[2], m4[3]};
          const u32x4_t lo = {l4[0], l4[1], l4[2], l4[3]};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(hi), as_bf16x8(av[i]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(mi), as_bf16x8(av[i]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lo), as_bf16x8(av[i]), acc[i][j], 0, 0, 0);
          }
        }
      }
    };

    dma(stage(icg<0>{}), 0, nks > 0);
    dma(stage(icg<1>{}), 1, nks > 1);
    dma(stage(icg<2>{}), 2, nks > 2);
    MOE_GEMM_WAIT_VM_LGKM0(2 * kDma);
    gemm_barrier();
    for (int k4 = 0; k4 < nks; k4 += 4) {
      auto step = [&](auto S_) {
        constexpr int S = decltype(S_)::value;
        const int ks = k4 + S;
        dma(stage(icg<S + 3>{}), ks + 3, ks + 3 < nks);
        issue_fence();
        compute(stage(S_));
        MOE_GEMM_WAIT_VM_LGKM0(2 * kDma);
        gemm_barrier();
      };
      step(icg<0>{});
      step(icg<1>{});
      step(icg<2>{});
      step(icg<3>{});
    }
    // the last k-steps issued zero-filling loads into the ring: they must land before the
    // block ends and its LDS goes to another block
    MOE_GEMM_WAIT_VM_LGKM0(0);
  };
  if (sg.w_f32)
    core(std::true_type{});
  else
    core(std::false_type{});

  // epilogue: lane (nl, q) holds D[m = 16 i + nl][n = 16 j + 4 q + r], r = 0..3, of tile (i, j)
  gemm_epilogue_rows<4, 4>(acc, sg, args.M, m0 + wm * 64 + nl, n0 + wn * 64 + 4 * q, slice);
}

// ---- Large batches: 256 x 224 outputs per block, 8 waves (2 per SIMD) in 4 x 2, each
// 64 x 112 (4 x 7 MFMA tiles). Per 64 K the block moves 60 KB for 7.3 MFLOP, about half the
// bytes per flop of the 128 x 128 tile, whose four waves (one per SIMD) need more load
// bandwidth per compute unit than the memory path gives. 224 columns divide the layer's
// widths (7168 = 32 x 224, 3584 = 16 x 224, 896 = 4 x 224): at an 8192-token prefill the
// up-projection is 1024 tiles, four full rounds of the 256 compute units, where 256-column
// tiles made 896 (3.5 rounds, the last half idle), and the router's 896 rows need no
// half-empty tile. K goes in steps of 32 (64 bytes of every row) through a ring of four
// 32 KB stages, three k-steps ahead, so 96 KB stay in flight per compute unit. Tiles are
// dealt to the XCDs round-robin (tile = grid position), the segment with the longer K
// first, and inside a segment in groups of 8 M tiles with M fastest, so one XCD holds the
// tiles of one M residue class and reuses their A rows across N from its L2.
constexpr int kBM2 = 256, kBN2 = 224, kBK2 = 32;
constexpr int kTile2 = kBM2 * kBK2 * 2;            // 16 KB: one operand tile of a stage
constexpr int kDma2 = 2 * kTile2 / 16 / 512;       // 16-byte LDS-DMA chunks per thread per k-step
static_assert(kDma2 == 4, "");


__global__ __launch_bounds__(512) void gemm256_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t sa0[2 * kTile2];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[2 * kTile2];
  __shared__ __attribute__((aligned(16))) uint8_t sa2[2 * kTile2];
  __shared__ __attribute__((aligned(16))) uint8_t sa3[2 * kTile2];
  auto stage = [&](auto I_) -> uint8_t* {
    constexpr int I = decltype(I_)::value % 4;
    if constexpr (I == 0) return sa0;
    else if constexpr (I == 1) return sa1;
    else if constexpr (I == 2) return sa2;
    else return sa3;
  };
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nl = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- block -> (segment, K slice, M tile, N tile): the segment with the longer K slices
  // first, each segment's K slices one after another
  const int tm = (args.M + kBM2 - 1) / kBM2;
  const GemmSeg& s0 = args.seg[0];
  const GemmSeg& s1 = args.seg[1];
  const int sl0 = max(1, s0.splits), sl1 = args.nseg > 1 ? max(1, s1.splits) : 1;
  const int st0 = (s0.K / kBK2 + sl0 - 1) / sl0, st1 = args.nseg > 1 ? (s1.K / kBK2 + sl1 - 1) / sl1 : 0;
  const bool f1 = st1 > st0;  // segment 1 first
  const int tnf = ((f1 ? s1.N : s0.N) + kBN2 - 1) / kBN2;
  const int tno = args.nseg > 1 ? ((f1 ? s0.N : s1.N) + kBN2 - 1) / kBN2 : 0;
  const int nbf = tm * tnf * (f1 ? sl1 : sl0);
  const int nbo = args.nseg > 1 ? tm * tno * (f1 ? sl0 : sl1) : 0;
  int L = (int)blockIdx.x;
  if (L >= nbf + nbo) return;
  const bool first = L < nbf;
  if (!first) L -= nbf;
  const int tn = first ? tnf : tno;
  const int slice = L / (tm * tn);
  L %= tm * tn;
  const int grp = L / (kGM * tn), rem = L % (kGM * tn);
  const int gm = min(kGM, tm - grp * kGM);
  const int mt = grp * kGM + rem % gm, nt = rem / gm;
  const GemmSeg sg = pick_seg(args, first == f1);
  const int m0 = mt * kBM2, n0 = nt * kBN2;
  const int K = sg.K, kwrap = sg.kwrap;
  // this block's k-steps: [kb0, kb0 + nks) (a K slice, or all of K)
  const int nks_all = K / kBK2, nsl = max(1, sg.splits);
  const int kper = (nks_all + nsl - 1) / nsl;
  const int kb0 = slice * kper;
  const int nks = max(0, min(nks_all, kb0 + kper) - kb0);

  // ---- LDS-DMA of one k-step: load i < 2 carries A chunk t = tid + 512 i, else W chunk
  // t = tid + 512 (i - 2); chunk t is row t / 4 of its tile at LDS position t % 4. The W
  // tile has 224 rows: the chunks of rows 224..255 load zeros into the unused LDS rows.
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(args.A, (uint32_t)args.M * (uint32_t)args.lda * 2u);
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(sg.W, (uint32_t)sg.N * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t none = make_rsrc(sg.W, 0u);
  uint32_t goff[kDma2];
#pragma unroll
  for (int i = 0; i < kDma2; ++i) {
    const int t = tid + 512 * (i & 1), r = t >> 2, pos = t & 3;
    const int c = g_pos2(pos, r);  // the XOR is its own inverse
    if (i < 2) {
      const int row = m0 + r;
      goff[i] = row < args.M ? ((uint32_t)row * (uint32_t)args.lda + 8u * c) * 2u : kOob;
    } else {
      const int row = n0 + r;
      goff[i] = r < kBN2 && row < sg.N ? ((uint32_t)row * (uint32_t)K + 8u * c) * 2u : kOob;
    }
  }
  auto dma = [&](uint8_t* st, int j, bool on) {  // kDma2 loads of the block's k-step j
    const int ks = kb0 + j;
    const uint32_t ka = (uint32_t)((ks * kBK2) % kwrap) * 2u, kw = (uint32_t)(ks * kBK2) * 2u;
#pragma unroll
    for (int i = 0; i < kDma2; ++i)
      dma16g(on ? (i < 2 ? a_rs : w_rs) : none, st + (i < 2 ? 0 : kTile2) + (i & 1) * 8192 + wave * 1024, goff[i],
             i < 2 ? ka : kw);
  };

  // fragment reads: lane (nl, q) of A tile mi reads row 64 wm + 16 mi + nl, chunk q; of W
  // tile j row 112 wn + 16 j + nl
  constexpr int kMI = 4, kNJ = 7;
  const uint32_t ard = (uint32_t)((wm * 64 + nl) * 64 + g_pos2(q, nl) * 16);
  const uint32_t brd = (uint32_t)(kTile2 + (wn * 112 + nl) * 64 + g_pos2(q, nl) * 16);
  f32x4_t acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[i][j]));
    }

  auto compute = [&](const uint8_t* st) {
    u32x4_t bv[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) bv[j] = *(const u32x4_t*)(st + brd + j * 16 * 64);
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const u32x4_t av = *(const u32x4_t*)(st + ard + i * 16 * 64);
#pragma unroll
      for (int j = 0; j < kNJ; ++j)  // weights as the MFMA's A operand: acc[i][j] holds the tile transposed
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(bv[j]), as_bf16x8(av), acc[i][j], 0, 0, 0);
    }
  };

  // ring: k-step ks reads stage ks % 4; it issues the loads of ks + 3 into the stage read
  // by ks - 1, then waits for stage ks + 1 (issued in ks - 2: 2 x kDma2 loads follow it).
  // Steps past nks load zeros (a K slice need not be a multiple of 4 steps).
  dma(stage(icg<0>{}), 0, nks > 0);
  dma(stage(icg<1>{}), 1, nks > 1);
  dma(stage(icg<2>{}), 2, nks > 2);
  MOE_GEMM_WAIT_VM_LGKM0(2 * kDma2);
  gemm_barrier();
  for (int k4 = 0; k4 < nks; k4 += 4) {
    auto step = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      const int ks = k4 + S;
      dma(stage(icg<S + 3>{}), ks + 3, ks + 3 < nks);
      issue_fence();
      compute(stage(S_));
      MOE_GEMM_WAIT_VM_LGKM0(2 * kDma2);
      gemm_barrier();
    };
    step(icg<0>{});
    step(icg<1>{});
    step(icg<2>{});
    step(icg<3>{});
  }
  // the last k-steps issued zero-filling loads into the ring: they must land before the
  // block ends and its LDS goes to another block
  MOE_GEMM_WAIT_VM_LGKM0(0);

  // epilogue: lane (nl, q) holds D[m = 16 i + nl][n = 16 j + 4 q + r], r = 0..3, of tile (i, j):
  // four consecutive columns of one row, stored (and the addend loaded) 8 or 16 bytes at a time
  // when the row strides allow it. Rows past M and columns past N are skipped.
  gemm_epilogue_rows<kMI, kNJ>(acc, sg, args.M, m0 + wm * 64 + nl, n0 + wn * 112 + 4 * q, slice);
}

// fp32 [N, K] -> bf16 [N, 3K]: row n = hi(k) | mid(k) | lo(k), w = hi + mid + lo exactly.
// Eight consecutive weights per thread (K % 8 == 0): two 16-byte read-once loads and one
// 16-byte store per plane (at 8192 tokens of the K3 router, 25.7 MB in and 38.5 MB out, ~12 us
// against 21 us with one weight and three 2-byte stores per thread).
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ W, int N, int K,
                                                     uint16_t* __restrict__ out) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= (long long)N * K) return;
  const int n = (int)(i / K), k = (int)(i % K);
  const u32x4_t a = load_nt_u32x4(W + i), b = load_nt_u32x4(W + i + 4);
  const uint32_t f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split3x2(__uint_as_float(f[2 * j]), __uint_as_float(f[2 * j + 1]), hi[j], mid[j], lo[j]);
  uint16_t* row = out + (size_t)n * 3 * K;
  *(u32x4_t*)(row + k) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  *(u32x4_t*)(row + K + k) = u32x4_t{mid[0], mid[1], mid[2], mid[3]};
  *(u32x4_t*)(row + 2 * K + k) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
}

}  // namespace

// The 256 x 224 tile for large batches, the 128 x 128 tile (split over K where its tiles
// leave compute units idle) below: splitting every segment of the larger tile cost more in
// partial planes than its lower load traffic per flop saved; it splits only the router
// segment, where that balances the rounds (gemm_large_split).
bool use_tile256(int M) { return M >= kLargeM; }

void gemm_split_plan(int M, int nseg, const int* N, const int* K, int num_cu, int* splits) {
  // every block one compute unit (either tile's LDS ring takes 128 KB): the fewest k-steps
  // per block for which all blocks fit at once, each segment's K cut into slices of about
  // that many steps
  const bool big = use_tile256(M);
  const int bm = big ? kBM2 : kBM, bn = big ? kBN2 : kBN, bk = big ? kBK2 : kBK;
  const long long tm = (M + bm - 1) / bm;
  long long tiles[2] = {0, 0}, steps[2] = {0, 0};
  for (int i = 0; i < nseg; ++i) {
    tiles[i] = tm * ((N[i] + bn - 1) / bn);
    steps[i] = K[i] / bk;
  }
  for (long long spb = 4;; spb += 4) {
    long long blocks = 0;
    for (int i = 0; i < nseg; ++i) blocks += tiles[i] * ((steps[i] + spb - 1) / spb);
    if (blocks <= num_cu || spb >= steps[0] + steps[1]) {
      for (int i = 0; i < nseg; ++i) splits[i] = (int)((steps[i] + spb - 1) / spb);
      return;
    }
  }
}

// 256 x 224 tiles (2048+ rows): one block fills a compute unit, so the launch runs as list
// scheduling of its tiles, in grid order, over the compute units. A router segment whose K is
// three times the other's (its three bf16 planes) leaves the last round partly idle; cut into
// two K slices (fp32 partial planes, summed before routing) its tiles balance the rounds. The
// split is taken when the simulated schedule is at least 8% shorter: at 8192 tokens of the K3
// layer 784 against 896 k-step units (the partial planes add ~60 MB of traffic).
static long long schedule_steps(long long tiles_a, long long steps_a, long long tiles_b, long long steps_b, int num_cu) {
  // tiles of the longer k-step count first, as gemm256_kernel orders its segments
  if (steps_b > steps_a) {
    std::swap(tiles_a, tiles_b);
    std::swap(steps_a, steps_b);
  }
  std::priority_queue<long long, std::vector<long long>, std::greater<long long>> cu;
  for (int i = 0; i < num_cu; ++i) cu.push(0);
  long long end = 0;
  auto run = [&](long long n, long long len) {
    for (long long t = 0; t < n; ++t) {
      const long long f = cu.top() + len;
      cu.pop();
      cu.push(f);
      end = std::max(end, f);
    }
  };
  run(tiles_a, steps_a);
  run(tiles_b, steps_b);
  return end;
}

int gemm_large_split(int M, const int* N, const int* K, int num_cu) {
  if (!use_tile256(M)) return 1;
  const long long tm = (M + kBM2 - 1) / kBM2;
  const long long t0 = tm * ((N[0] + kBN2 - 1) / kBN2), t1 = tm * ((N[1] + kBN2 - 1) / kBN2);
  const long long s0 = K[0] / kBK2, s1 = K[1] / kBK2;
  if (s1 % 2 || t0 + 2 * t1 > 0x7fffff) return 1;
  const long long whole = schedule_steps(t0, s0, t1, s1, num_cu);
  const long long halves = schedule_steps(t0, s0, 2 * t1, s1 / 2, num_cu);
  return halves * 100 <= whole * 92 ? 2 : 1;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.nseg < 1 || a.nseg > 2 || a.M < 0 || a.lda % 8) return hipErrorInvalidValue;
  const bool big = use_tile256(a.M);
  const int bm = big ? kBM2 : kBM, bn = big ? kBN2 : kBN, bk = big ? kBK2 : kBK;
  long long blocks = 0;
  const long long tm = (a.M + bm - 1) / bm;
  for (int i = 0; i < a.nseg; ++i) {
    const GemmSeg& g = a.seg[i];
    if (g.K % (4 * kBK) || g.kwrap % kBK || g.kwrap > a.lda || g.K % g.kwrap || g.N <= 0) return hipErrorInvalidValue;
    if ((long long)g.N * g.K * (g.w_f32 ? 4 : 2) >= (1ll << 31)) return hipErrorInvalidValue;
    if (g.w_f32 && (big || g.kwrap != g.K)) return hipErrorInvalidValue;  // fp32 weights: the 128 x 128 tile
    if (g.splits < 0 || g.splits > g.K / (g.w_f32 ? 32 : bk) || (g.mode == kPartF32) != (g.splits > 1))
      return hipErrorInvalidValue;
    blocks += tm * ((g.N + bn - 1) / bn) * (g.splits > 1 ? g.splits : 1);
  }
  if ((long long)a.M * a.lda * 2 >= (1ll << 31)) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7ffffff0ll) return hipErrorInvalidValue;
  if (big) {
    hipLaunchKernelGGL(gemm256_kernel, dim3((unsigned)blocks), dim3(512), 0, s, a);
    return hipGetLastError();
  }
  const long long grid = (blocks + 7) / 8 * 8;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split3(const float* W, int N, int K, uint16_t* out, hipStream_t s) {
  const long long n = (long long)N * K;
  if (n <= 0) return hipSuccess;
  if (K % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s, W, N, K, out);
  return hipGetLastError();
}

}  // namespace moe
