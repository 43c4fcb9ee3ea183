// Grouped MXFP4 contractions on gfx950's scaled MFMA (prefill-sized token counts).
//
// Each routed expert holds its tokens' rows contiguously in the expert-sorted
// layout (moe_align_block_size, pages: "Kimi K3, as released", tensor listing;
// the vLLM-style align block). A job is one chunk of at most 192 slots of one
// expert; a block computes one job against one 256-row tile of the expert's
// weights with the full K, so every weight byte is read from HBM once per chunk,
// and almost every expert of an 8192-token batch fits in one chunk.
//
// Operands. v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16x128 A tile by a
// 128x16 B tile, each lane holding 32 consecutive K values of one row (lane
// group q = lane/16 owns K block q) and one E8M0 scale for them; both operands
// have this lane layout, so either can take the weights. The weights go into the
// MFMA straight from their shipped layout: a lane's 32 weights are one E8M0 group,
// 16 bytes of a row, so the MXFP4 bytes and their scale bytes are used unchanged.
// The GLU contraction passes the activations as A (a lane's outputs are four slots
// of one h column, so the gate and up of a column meet in one lane); the plain one
// passes the weights as A (a lane's outputs are four consecutive columns of one
// slot: 16-byte stores; its epilogue measured 5.2 us against 5.8 us per block with
// 4-byte stores at an 8192-token prefill). The activations are, per problem, either
// in the FP6 E2M3 hi/lo encoding (mxfp6.h; hi and lo each take one MFMA at the
// FP4 rate) or, with MXFP8 activations, as E4M3 codes (mxfp8.h; one MFMA at the
// FP8 rate, two thirds of the bytes per k-step).
//
// K order. K-step k gives lane group q the E8M0 group 4k + q, so one weight load
// instruction covers 64 contiguous bytes of each of 16 rows. A lane's scales for
// the four k-steps of a window (512 K values) are bytes q, 4+q, 8+q, 12+q of its
// row's 16 window scale bytes; they are gathered once per window into one dword
// (opsel s picks byte s). The activation encoding stores its scales in that
// gathered order already.
//
// Activation layouts. Gate/up (GLU): the A rows are the tokens' rows, stored row after
// row and gathered through the sorted token ids; each staged row is rotated in LDS (a_rot).
// Down (plain): A is h, which the GLU epilogue writes tiled (mxfp6.h, atile_offset: 16-row
// tiles, chunk-major inside a tile) in slot order. A job starts at a multiple of 16 slots,
// so one k-step of its rows is NT contiguous blocks of 16 x 192 bytes (FP6) or 16 x 128
// (FP8): every LDS-DMA instruction moves 1 KB of contiguous memory, and the LDS tile comes
// out chunk-major, where the 16 lanes of a lane group read one chunk of 16 rows as 256
// contiguous bytes, the pattern at which gfx950's LDS serves ds_read_b128 without bank
// conflicts. Measured at an 8192-token prefill on one GPU: the down launch 2.55 ms tiled
// against 2.66 ms gathered; the gate/up launch tiled 5.30 ms against 5.46, but its rows
// then have to be copied per slot first (750 MB, 0.17-0.2 ms), which cancels that gain,
// so gate/up keeps the gathered rows. The scales stay row after row.
//
// Dataflow per block (8 waves, 2 per SIMD). The A rows of a k-step (192 rows x
// 192 bytes FP6 or 128 FP8) go to LDS by LDS-DMA loads
// (no registers), into a ring of four stages, three k-steps ahead of their use;
// every wave reads all of them, one barrier per k-step. Each wave owns 32 weight
// rows (GLU: 16 gate + the same 16 up rows) and loads them straight into MFMA
// registers, one window ahead (default cache policy: the four k-steps of a window
// read the two halves of the same lines). Two waves per SIMD keep its MFMA pipe
// fed while the other wave's memory instructions wait for the load pipeline; each
// k-step's memory instructions are spread over its row tiles for the same reason.
// Jobs are dealt to the XCDs round-robin and the blocks of one job are adjacent
// in its XCD's order, so the job's activation rows are served from that XCD's L2.
//
// Waits. vmcnt retires loads in issue order, so waiting for a stage also waits
// for every load issued before it; the ring depth sets how old those loads are.
// The waits are explicit counts (every k-step issues the same loads, none under
// a runtime branch), and each ring stage is its own LDS array with a
// compile-time index, so the compiler can tell that a stage being read is not
// the target of the loads in flight.
//
// Epilogue. Plain: fp32 rows, routed ones at the slot's position (a job's rows are then
// one contiguous block; writing them at the flat slot index instead, scattered, measured
// 2.78 ms against 2.51 ms for the down launch at an 8192-token prefill). GLU: h = act(gate)*up
// goes through LDS and is written directly in the encoding (FP6 hi/lo or MXFP8)
// that the down contraction reads.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mxfp6.h"
#include "mxfp8.h"

namespace moe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMF = kMfmaSlotsPerJob / 16;  // row tiles per job
constexpr int kRows = kMfmaSlotsPerJob;     // 192

// Activation formats of the A operand. Per row and k-step (128 K values): FP6 hi/lo takes
// 12 chunks of 16 bytes (two planes of 4 x 24 bytes), MXFP8 8 chunks (4 x 32 bytes); per
// row and window (512 K values) their scales take 32 and 16 bytes.
template <bool FP8>
struct AFmt {
  static constexpr int kChunks = FP8 ? 8 : 12;         // 16-byte chunks per row per k-step
  static constexpr int kArow = kChunks * 16;           // LDS bytes per staged row
  static constexpr int kStep = FP8 ? 128 : kFp6StepBytes;
  static constexpr int kWinScale = FP8 ? kFp8WindowScaleBytes : kFp6WindowScaleBytes;
  static constexpr int kSChunks = kWinScale / 16;      // 16-byte scale chunks per row per window
  static constexpr int kPlanes = FP8 ? 1 : 2;          // MFMAs per (row tile, B tile, k-step)
  static constexpr int kAStage = kRows * kArow;        // bytes per A stage
  static constexpr int kADmaMax = (kRows * kChunks + kThreads - 1) / kThreads;
  // the last LDS-DMA round of a stage may cover only part of the block; the waves past
  // the stage's end load zeros into a dummy area instead (same load count in every wave)
  static constexpr int kADummy = kADmaMax * kThreads * 16 - kAStage;
  __host__ __device__ static size_t row_bytes(int K) { return FP8 ? fp8_row_bytes(K) : fp6_row_bytes(K); }
  __host__ __device__ static size_t scale_row_bytes(int K) {
    return FP8 ? fp8_scale_row_bytes(K) : fp6_scale_row_bytes(K);
  }
};
using F6 = AFmt<false>;
using F8 = AFmt<true>;
// the kernel's LDS is laid out for FP6 hi/lo, the larger format
constexpr int kAStage = F6::kAStage;
constexpr int kSDma = 1;                    // 16-byte scale chunks per thread per window
constexpr int kSStage = kSDma * kThreads * 16;
constexpr int kADummy = F6::kADummy;
constexpr int kHRow = 132;                  // floats per row of the GLU epilogue tile
constexpr int kHRowsPerArray = 48;          // rows of h per ring array in the GLU epilogue
static_assert(F6::kADummy >= 0 && F6::kADummy % 1024 == 0 && F6::kAStage % 1024 == 0, "A stage");
static_assert(F8::kADummy == 0 && F8::kAStage % 1024 == 0 && F8::kAStage + kSStage <= kAStage + kSStage,
              "FP8 stage inside the FP6 arrays");
static_assert(kRows * F6::kSChunks <= kSDma * kThreads && kRows * F8::kSChunks <= kSDma * kThreads, "scale chunks");
static_assert(kHRowsPerArray * kHRow * 4 <= kAStage && 4 * kHRowsPerArray >= kRows, "GLU epilogue tile");
static_assert(4 * kAStage + kSStage + kADummy <= 160 * 1024, "LDS");

template <int I>
using ic = std::integral_constant<int, I>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at 15:14)
#define MOE_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | ((((n) >> 4) & 3) << 14))

// Workgroup barrier of the ring. Each wave establishes completion of its own
// LDS-DMA loads with an explicit vmcnt wait first; __syncthreads() would wait for
// every outstanding load. The empty asm statements keep the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff,
                                           0, 0);
}

// LDS position of 16-byte chunk c of a staged row whose index within its 16-row tile is
// nl. The 16 lanes of a lane group read the same chunk index of 16 rows; each row is
// rotated so that those 16 reads fall on 16 different 16-byte bank slots.
// FP6: a lane group's operands are chunks 3q..3q+2 (16 bytes of hi, then 8 of hi and 8
// of lo, then 16 of lo); rows are 12 chunks long. FP8: chunks q and 4+q; rows are 8
// chunks long.
// Measured on gfx950 (a ds_read_b128 probe, 4 waves per CU): the LDS reaches its full
// rate only when each group of 16 lanes reads one contiguous 256-byte block (22 clocks
// per wave instruction); these rotated reads take 32, as do unrotated ones, and the
// gate/up kernel's counters show bank conflicts in 35% of its cycles. A chunk-major tile
// of the gathered rows cut that to 13.5%, but its LDS-DMA then gathers 16 rows x 64 bytes
// per instruction and the launch ran 14% slower; the tiled layout of h (above) gives the
// down launch chunk-major LDS tiles with contiguous DMA reads.
template <bool FP8>
__host__ __device__ constexpr int a_rot(int nl) {
  return FP8 ? ((nl >> 1) & 7) : (((nl >> 1) & 3) ^ ((nl >> 3) & 1));
}
template <bool FP8>
__host__ __device__ constexpr int a_chunk_pos(int c, int nl) {
  return (c + a_rot<FP8>(nl)) % AFmt<FP8>::kChunks;
}

// One job (at most NT row tiles of 16) against one column tile. NT is a compile-time
// bucket of the job's row count: every loop below is straight-line code, so each
// k-step issues a fixed set of loads and the compiler's waits are exact.
template <bool GLU, int NT, bool FP8>
__device__ __forceinline__ void mx_job(const MfmaProblem& a, int first, int nvalid, int expert, int ntile,
                                       uint8_t (&lds_a0)[kAStage + kSStage], uint8_t (&lds_a1)[kAStage],
                                       uint8_t (&lds_a2)[kAStage], uint8_t (&lds_a3)[kAStage],
                                       uint8_t* lds_dummy) {
  using Fm = AFmt<FP8>;
  constexpr int kADma = (NT * 16 * Fm::kChunks + kThreads - 1) / kThreads;  // LDS-DMA loads per thread per k-step
  static_assert(kADma <= Fm::kADmaMax, "stage");
  constexpr int kArow = Fm::kArow;
  constexpr int kFStage = Fm::kAStage;  // A bytes of a stage; the window's scales follow stage 0's
  auto stage = [&](auto I_) -> uint8_t* {
    constexpr int I = decltype(I_)::value % 4;
    if constexpr (I == 0) return lds_a0;
    else if constexpr (I == 1) return lds_a1;
    else if constexpr (I == 2) return lds_a2;
    else return lds_a3;
  };
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nl = lane & 15, q = lane >> 4;

  const int K = a.K;
  const uint32_t arow_bytes = (uint32_t)Fm::row_bytes(K), asrow_bytes = (uint32_t)Fm::scale_row_bytes(K);
  auto a_row = [&](int j) -> int {  // scale row of job slot j, -1 past the valid slots
    if (j >= nvalid) return -1;
    if (!a.routed || a.a_by_pos) return first + j;
    return a.sorted_ids[first + j] / a.topk;
  };

  // ---- A stage by LDS-DMA; chunk t = tid + 512 i lands at LDS byte 16 t.
  // Gathered rows (GLU): LDS byte 16 t is position t % kChunks of staged row j = t / kChunks,
  // which receives the row's global chunk whose rotated position that is; k-step ks starts
  // ks * kStep bytes into a row.
  // Tiled (plain): chunk t is byte 16 t of the job's tiles' blocks for the k-step (tile
  // t / (16 kChunks), chunk t / 16 % kChunks of row t % 16); k-step ks starts 16 kStep * ks
  // bytes into a tile.
  constexpr int kCh = Fm::kChunks;
  constexpr uint32_t kAStepOff = GLU ? (uint32_t)Fm::kStep : 16u * Fm::kStep;  // buffer offset per k-step
  uint32_t goff[kADma];
#pragma unroll
  for (int i = 0; i < kADma; ++i) {
    const int t = tid + kThreads * i;
    if constexpr (GLU) {
      const int j = t / kCh, pos = t % kCh;
      const int c = (pos + kCh - a_rot<FP8>(j & 15)) % kCh;
      const int r = j < NT * 16 ? a_row(j) : -1;
      goff[i] = r >= 0 ? (uint32_t)r * arow_bytes + 16u * c : kOob;
    } else {
      const int mf = t / (16 * kCh), j = 16 * mf + (t & 15);
      goff[i] = j < NT * 16 && j < nvalid
                    ? (uint32_t)((first >> 4) + mf) * 16u * arow_bytes + (uint32_t)(t % (16 * kCh)) * 16u
                    : kOob;
    }
  }
  uint32_t sgoff[kSDma];
#pragma unroll
  for (int i = 0; i < kSDma; ++i) {
    const int t = tid + kThreads * i, j = t / Fm::kSChunks, c = t % Fm::kSChunks;
    const int r = j < NT * 16 ? a_row(j) : -1;
    sgoff[i] = r >= 0 ? (uint32_t)r * asrow_bytes + 16u * c : kOob;
  }
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(a.Aq, (uint32_t)a.a_rows * arow_bytes);
  const __amdgpu_buffer_rsrc_t as_rs = make_rsrc(a.Aqs, (uint32_t)a.s_rows * asrow_bytes);

  // ---- weights: two B tiles per wave, lane (nl, q) of tile nf reads row rows(nf) + nl.
  // GLU: tile 0 = 16 gate rows, tile 1 = the same 16 up rows; plain: 32 consecutive rows.
  const uint32_t kb2 = (uint32_t)K / 2, ks32 = (uint32_t)K / 32;
  const uint32_t mat_bytes = (uint32_t)a.N * kb2, mat_scales = (uint32_t)a.N * ks32;
  const __amdgpu_buffer_rsrc_t w_lo = make_rsrc(a.W + (size_t)expert * a.w_stride, mat_bytes);
  const __amdgpu_buffer_rsrc_t s_lo = make_rsrc(a.S + (size_t)expert * a.s_stride, mat_scales);
  const __amdgpu_buffer_rsrc_t w_hi = GLU ? make_rsrc(a.W2 + (size_t)expert * a.w_stride, mat_bytes) : w_lo;
  const __amdgpu_buffer_rsrc_t s_hi = GLU ? make_rsrc(a.S2 + (size_t)expert * a.s_stride, mat_scales) : s_lo;
  const int row0 = GLU ? ntile * 128 + wave * 16 : ntile * 256 + wave * 32;
  uint32_t bvoff[2], svoff[2];
#pragma unroll
  for (int nf = 0; nf < 2; ++nf) {
    const uint32_t row = (uint32_t)(row0 + (GLU ? 0 : 16 * nf) + nl);
    bvoff[nf] = row * kb2 + 16u * q;
    svoff[nf] = row * ks32;
  }
  auto w_rs = [&](int nf) { return (GLU && nf == 1) ? w_hi : w_lo; };
  auto s_rs = [&](int nf) { return (GLU && nf == 1) ? s_hi : s_lo; };
  // byte selector of v_perm_b32 gathering byte q of each of two dwords into the low half
  const uint32_t qsel = 0x0c0c0000u | ((uint32_t)(4 + q) << 8) | (uint32_t)q;

  // A load that is not needed (past the last k-step or window) goes to a zero-size
  // resource: it reads zeros without touching memory, and the load count stays fixed.
  // The weight loads keep the default cache policy: the four k-steps of a window read
  // interleaved 16-byte pieces of the same lines, which must survive in L2 between them.
  const __amdgpu_buffer_rsrc_t none = make_rsrc(a.W, 0u);
  u32x4_t b[4][2];  // [k-step in window][B tile]
  uint32_t sb[2];   // gathered scale dwords of the current window
  u32x4_t sbn[2];   // the next window's 16 scale bytes per row
  auto load_b = [&](int w, int s, bool on) {  // 2 loads
#pragma unroll
    for (int nf = 0; nf < 2; ++nf)
      b[s][nf] = buf_load16(on ? w_rs(nf) : none, bvoff[nf], (uint32_t)(256 * w + 64 * s));
  };
  auto load_sb = [&](int w, bool on) {  // 2 loads
#pragma unroll
    for (int nf = 0; nf < 2; ++nf) sbn[nf] = buf_load16(on ? s_rs(nf) : none, svoff[nf], (uint32_t)(16 * w));
  };
  // byte s of the result = byte q of dword s (the scale of group 4s + q)
  auto gather_sb = [&]() {
#pragma unroll
    for (int nf = 0; nf < 2; ++nf) {
      const uint32_t lo = __builtin_amdgcn_perm(sbn[nf][1], sbn[nf][0], qsel);
      const uint32_t hi = __builtin_amdgcn_perm(sbn[nf][3], sbn[nf][2], qsel);
      sb[nf] = lo | (hi << 16);
    }
  };
  // LDS-DMA round i of this wave: 1 KB at byte i * 8192 + wave * 1024 of the stage, or of the
  // dummy area past the stage's end (those lanes carry no row: their goff is out of range)
  auto a_dst_of = [&](uint8_t* st, int i) -> uint8_t* {
    const int o = i * (kThreads * 16) + wave * 1024;
    return (i + 1) * (kThreads * 16) <= kFStage || o < kFStage ? st + o : lds_dummy + (o - kFStage);
  };
  auto dma_a = [&](uint8_t* st, int ks, bool on) {  // kADma loads
#pragma unroll
    for (int i = 0; i < kADma; ++i) dma16(on ? a_rs : none, a_dst_of(st, i), goff[i], (uint32_t)ks * kAStepOff);
  };
  auto dma_s = [&](int w, bool on) {  // kSDma loads
#pragma unroll
    for (int i = 0; i < kSDma; ++i)
      dma16(on ? as_rs : none, lds_a0 + kFStage + wave * 1024 + i * (kThreads * 16), sgoff[i],
            (uint32_t)(w * Fm::kWinScale));
  };

  // Each accumulator starts from its own opaque zero: with one shared constant as the
  // loop-entry value of every accumulator, the register allocator renames MFMA results
  // and copies them back on every iteration.
  f32x4_t acc[NT][2];
#pragma unroll
  for (int mf = 0; mf < NT; ++mf)
#pragma unroll
    for (int nf = 0; nf < 2; ++nf) {
      acc[mf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(acc[mf][nf]));
    }

  // FP6: lane (nl, q) reads its group as chunks 3q .. 3q+2 (48 bytes, hi then lo plane).
  // FP8: an FP8 operand register's first 16 bytes hold K 16q .. 16q+15 of the k-step and
  // its last 16 bytes K 64+16q .. 64+16q+15, while K block b (32b .. 32b+31) is scaled by
  // lane group b's scale; lane group q therefore reads chunks q and 4+q, and group
  // 4k + q's scale stays with lane group q.
  constexpr int kRd = FP8 ? 2 : 3;
  uint32_t aoff[kRd];
#pragma unroll
  for (int u = 0; u < kRd; ++u) {
    const int c = FP8 ? q + 4 * u : 3 * q + u;
    // gathered: chunk c of row nl at its rotated position; tiled: chunk c of the 16 rows, row nl
    aoff[u] = GLU ? (uint32_t)(nl * kArow + a_chunk_pos<FP8>(c, nl) * 16) : (uint32_t)(c * 256 + nl * 16);
  }
  // activation scale dwords of the window, read at its start: the scale area (in stage 0)
  // receives the next window's scales from k-step 1 of the window on
  constexpr int kP = Fm::kPlanes;
  uint32_t sA[NT][kP];

  // FP6: four reads per tile: the middle chunk is read as two halves, so each operand is
  // one 16-byte and one 8-byte read straight into its registers (the empty asm keeps the
  // two halves from being merged into one read whose halves would then be copied).
  // FP8: two 16-byte reads, the operand's two halves.
  auto read_a = [&](const uint8_t* st, int mf, i32x8_t* av) {
    const uint8_t* base = st + mf * 16 * kArow;
    if constexpr (FP8) {
      const i32x4_t x0 = *(const i32x4_t*)(base + aoff[0]);
      const i32x4_t x1 = *(const i32x4_t*)(base + aoff[1]);
      av[0] = i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      return;
    }
    const i32x4_t x0 = *(const i32x4_t*)(base + aoff[0]);
    const int2 h1 = *(const int2*)(base + aoff[1]);
    asm volatile("" ::: "memory");
    const int2 l1 = *(const int2*)(base + aoff[1] + 8);
    const i32x4_t x2 = *(const i32x4_t*)(base + aoff[2]);
    av[0] = i32x8_t{x0[0], x0[1], x0[2], x0[3], h1.x, h1.y, 0, 0};
    av[1] = i32x8_t{l1.x, l1.y, x2[0], x2[1], x2[2], x2[3], 0, 0};
  };
  // Tile mf's MFMAs run while tile mf+1's operands are read; the barriers per tile keep
  // the compiler from hoisting all tiles' reads. Two register sets, picked by tile parity,
  // so no operand is copied. mem(mf) issues the memory operations assigned to tile mf.
  auto compute = [&](auto S_, const uint8_t* st, auto&& mem) {
    constexpr int S = decltype(S_)::value;
    i32x8_t av[2][kP];  // [row tile parity][plane]
    read_a(st, 0, av[0]);
    static_for<0, NT>([&](auto MF) {
      constexpr int mf = decltype(MF)::value;
      if constexpr (mf + 1 < NT) read_a(st, mf + 1, av[(mf + 1) & 1]);
      mem(MF);
#pragma unroll
      for (int p = 0; p < kP; ++p)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const u32x4_t bw = b[S][nf];
          const i32x8_t bv = {(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3], 0, 0, 0, 0};
          // Formats: 0 = FP8 E4M3, 2 = FP6 E2M3 (activations), 4 = FP4 E2M1 (weights).
          // GLU: activations as the MFMA's A operand, so a lane's four outputs are four slots of
          // one h column (the gate and up of that column sit in the same lane). Plain: weights
          // as the A operand, so a lane's four outputs are four consecutive output columns of one
          // slot and the epilogue writes 16 bytes per lane.
          if constexpr (GLU)
            acc[mf][nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                av[mf & 1][p], bv, acc[mf][nf], FP8 ? 0 : 2, 4, S, (int)sA[mf][p], S, (int)sb[nf]);
          else
            acc[mf][nf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bv, av[mf & 1][p], acc[mf][nf], 4, FP8 ? 0 : 2, S, (int)sb[nf], S, (int)sA[mf][p]);
        }
      // The memory clobber pins the LDS reads (IR passes may move loads across the
      // scheduling barrier, which touches no memory); the scheduling barrier then keeps
      // the MFMAs between them.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Pipeline. K-step ks (window w = ks/4, step S = ks%4) uses A stage S. Each k-step
  // issues, in order: at S == 1 the activation scales of window w+1 (kSDma loads into
  // stage 0's scale area), the A stage of ks+3 (kADma loads into stage (S+3)%4, read by
  // k-step ks-1), the weights of k-step (S+3)%4 (2 loads: window w at S == 0, else w+1;
  // those registers were last read by the previous k-step) and at S == 0 the weight
  // scales of window w+1 (2). Before the barrier that ends k-step ks, the A stage of ks+1
  // (issued in k-step ks-2) must be complete, and with it everything issued before it;
  // the loads issued after it may stay in flight (the compiler waits for the weight
  // registers where they are read).
  const int nw = K >> 9;
  const int nks = nw * 4;
  constexpr int kStepLoads[4] = {kADma + 4, kSDma + kADma + 2, kADma + 2, kADma + 2};  // by S
  constexpr int kStepTail[4] = {4, 2, 2, 2};  // loads of a k-step issued after its A stage
  // Prologue: the weight scales of window 0, then the loads of k-steps -3, -2, -1 in the
  // order those k-steps issue them (S = 1, 2, 3): the activation scales of window 0, A stage
  // 0 and the weights of k-step 0, A stage 1 and the weights of k-step 1, A stage 2 and the
  // weights of k-step 2. The waits at the ends of k-steps 0 and 1 then count exactly the
  // loads issued after stages 1 and 2, as in every later k-step (a wait that allows more
  // outstanding loads than were issued after the stage would not cover the stage).
  load_sb(0, true);
  dma_s(0, true);
  dma_a(stage(ic<0>{}), 0, true);
  load_b(0, 0, true);
  dma_a(stage(ic<1>{}), 1, nks > 1);
  load_b(0, 1, true);
  dma_a(stage(ic<2>{}), 2, nks > 2);
  load_b(0, 2, true);
  static_assert(kStepTail[1] == 2 && kStepTail[2] == 2 && kStepTail[3] == 2 && kStepLoads[2] == kADma + 2 &&
                    kStepLoads[3] == kADma + 2,
                "prologue order");
  // stage 0 and the scales before it complete: the loads after it are those of k-steps -2 and
  // -1 and the weights of k-step 0
  MOE_WAIT_VM_LGKM0(kStepTail[1] + kStepLoads[2] + kStepLoads[3]);
  ring_barrier();
  gather_sb();

  for (int w = 0; w < nw; ++w) {
    {
      const uint8_t* ss = lds_a0 + kFStage + nl * Fm::kWinScale + q * 4;
#pragma unroll
      for (int mf = 0; mf < NT; ++mf)
#pragma unroll
        for (int p = 0; p < kP; ++p) sA[mf][p] = *(const uint32_t*)(ss + mf * 16 * Fm::kWinScale + p * 16);
    }
    const bool more_w = w + 1 < nw;
    auto step = [&](auto S_) {
      constexpr int S = decltype(S_)::value;
      const int ks = 4 * w + S;
      constexpr int nS = S == 1 ? kSDma : 0;
      constexpr int nOps = nS + kADma + 2 + (S == 0 ? 2 : 0);
      constexpr int per = (nOps + NT - 1) / NT;
      constexpr int bs = (S + 3) % 4;
      const int bw_win = S == 0 ? w : w + 1;
      const bool b_on = S == 0 ? true : more_w;
      uint8_t* const a_dst = stage(ic<S + 3>{});
      const bool a_on = ks + 3 < nks;
      auto mem = [&](auto MF) {
        constexpr int mf = decltype(MF)::value;
        static_for<mf * per, (mf + 1) * per < nOps ? (mf + 1) * per : nOps>([&](auto O) {
          constexpr int o = decltype(O)::value;
          if constexpr (o < nS) {
            dma16(more_w ? as_rs : none, lds_a0 + kFStage + wave * 1024 + o * (kThreads * 16), sgoff[o],
                  (uint32_t)((w + 1) * Fm::kWinScale));
          } else if constexpr (o < nS + kADma) {
            constexpr int i = o - nS;
            dma16(a_on ? a_rs : none, a_dst_of(a_dst, i), goff[i], (uint32_t)(ks + 3) * kAStepOff);
          } else if constexpr (o < nS + kADma + 2) {
            constexpr int nf = o - nS - kADma;
            b[bs][nf] = buf_load16(b_on ? w_rs(nf) : none, bvoff[nf], (uint32_t)(256 * bw_win + 64 * bs));
          } else {
            constexpr int nf = o - nS - kADma - 2;
            sbn[nf] = buf_load16(more_w ? s_rs(nf) : none, svoff[nf], (uint32_t)(16 * (w + 1)));
          }
        });
      };
      compute(S_, stage(S_), mem);
      // loads issued after the A stage of ks+1: tail of ks-2, all of ks-1 and ks
      MOE_WAIT_VM_LGKM0(kStepTail[(S + 2) % 4] + kStepLoads[(S + 3) % 4] + kStepLoads[S]);
      ring_barrier();
    };
    step(ic<0>{});
    step(ic<1>{});
    step(ic<2>{});
    step(ic<3>{});
    gather_sb();
  }
  // the last k-steps issued zero-filling stage loads into the ring: drain them before reuse
  MOE_WAIT_VM_LGKM0(0);
  ring_barrier();

  if (!GLU) {
    // lane (nl, q) of tile (mf, nf) holds slot 16 mf + nl, output columns 16 nf + 4 q .. + 3
    const int col0 = row0;
#pragma unroll
    for (int mf = 0; mf < NT; ++mf) {
      const int j = 16 * mf + nl;
      if (j < nvalid) {
        const int orow = a.routed && a.out_flat ? a.sorted_ids[first + j] : first + j;
        const size_t ob = (size_t)orow * a.ldo + col0 + 4 * q;
        if (a.outh) {  // bf16 rows: 8 bytes per lane and tile
#pragma unroll
          for (int nf = 0; nf < 2; ++nf)
            *(uint2*)(a.outh + ob + 16 * nf) =
                uint2{pack_bf16x2(acc[mf][nf][0], acc[mf][nf][1]), pack_bf16x2(acc[mf][nf][2], acc[mf][nf][3])};
        } else {
#pragma unroll
          for (int nf = 0; nf < 2; ++nf) *(f32x4_t*)(a.outf + ob + 16 * nf) = acc[mf][nf];
        }
      }
    }
  } else {
    // h tile through LDS in one pass (rows 48i.. in ring array i), then one thread per
    // (row, group of 32 columns): the eight waves' 16 columns of a row form its 4 groups.
    const uint32_t orow_bytes = (uint32_t)Fm::row_bytes(a.N), osrow_bytes = (uint32_t)Fm::scale_row_bytes(a.N);
    auto hrow = [&](int j) -> float* {
      const int arr = j / kHRowsPerArray;
      uint8_t* base = arr == 0 ? lds_a0 : (arr == 1 ? lds_a1 : (arr == 2 ? lds_a2 : lds_a3));
      return (float*)base + (j - arr * kHRowsPerArray) * kHRow;
    };
#pragma unroll
    for (int mf = 0; mf < NT; ++mf)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hrow(16 * mf + 4 * q + r)[wave * 16 + nl] = glu_act(acc[mf][0][r], acc[mf][1][r], a.act);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (NT * 64 + kThreads - 1) / kThreads; ++i) {
      const int t = tid + kThreads * i;
      const int j = t >> 2, g4 = t & 3;
      if (j < NT * 16 && j < nvalid) {
        float v[32];
        const f32x4_t* src = (const f32x4_t*)(hrow(j) + 32 * g4);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const f32x4_t x = src[u];
          v[4 * u] = x[0];
          v[4 * u + 1] = x[1];
          v[4 * u + 2] = x[2];
          v[4 * u + 3] = x[3];
        }
        const int g = ntile * 4 + g4;
        if constexpr (FP8) {
          uint32_t codes[8], sc;
          mxfp8_encode_group(v, codes, sc);
          const size_t r = (size_t)(first + j);
          *(u32x4_t*)(a.outq + atile_offset(r, 32u * g, orow_bytes)) = u32x4_t{codes[0], codes[1], codes[2], codes[3]};
          *(u32x4_t*)(a.outq + atile_offset(r, 32u * g + 16, orow_bytes)) =
              u32x4_t{codes[4], codes[5], codes[6], codes[7]};
          a.outqs[(size_t)(first + j) * osrow_bytes + fp8_scale_offset(g)] = (uint8_t)sc;
          continue;
        }
        uint32_t hi[6], lo[6], s_hi, s_lo;
        fp6_encode_group(v, hi, lo, s_hi, s_lo);
        // the group's 48 bytes (hi, then lo) are chunks 3g .. 3g+2 of its row
        const size_t r = (size_t)(first + j);
        const uint32_t b = fp6_data_offset(g, 0);
        *(u32x4_t*)(a.outq + atile_offset(r, b, orow_bytes)) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
        *(u32x4_t*)(a.outq + atile_offset(r, b + 16, orow_bytes)) = u32x4_t{hi[4], hi[5], lo[0], lo[1]};
        *(u32x4_t*)(a.outq + atile_offset(r, b + 32, orow_bytes)) = u32x4_t{lo[2], lo[3], lo[4], lo[5]};
        uint8_t* srow = a.outqs + (size_t)(first + j) * osrow_bytes;
        srow[fp6_scale_offset(g, 0)] = (uint8_t)s_hi;
        srow[fp6_scale_offset(g, 1)] = (uint8_t)s_lo;
      }
    }
  }
}

// Activation formats of a launch's problems: every problem FP6 hi/lo, every problem MXFP8,
// or problem 0 FP6 and problem 1 MXFP8 (the shared experts next to MXFP8 routed experts).
// Each combination is its own kernel, so a kernel holds only the job code it runs.
enum LaunchFormats { kAllFp6 = 0, kAllFp8 = 1, kFp6ThenFp8 = 2 };

template <bool GLU, int FMTS>
__global__ __launch_bounds__(kThreads) void mx_mfma_kernel(MfmaArgs args) {
  // stage 0 also holds the activation scales of its window (its k-step starts the window)
  __shared__ __attribute__((aligned(16))) uint8_t lds_a0[kAStage + kSStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a1[kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a2[kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_a3[kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_dummy[kADummy > 0 ? kADummy : 16];

  // ---- block -> (problem, job, column tile). Jobs are dealt to XCDs round-robin (job j
  // to grid positions = j mod 8, which the hardware places on XCD j mod 8); inside an XCD
  // the column tiles of a job are consecutive (the job's activation rows stay in that
  // XCD's L2), and problem 0's jobs (the long dense rows) come before problem 1's.
  const int xcd = (int)blockIdx.x & 7, lb = (int)blockIdx.x >> 3;
  int nj0, nj1 = 0, nt0, nt1 = 1;
  {
    const MfmaProblem& p = args.p[0];
    nt0 = p.N / (GLU ? 128 : 256);
    nj0 = p.routed ? *p.n_jobs : (p.M + kRows - 1) / kRows;
  }
  if (args.nprob > 1) {
    const MfmaProblem& p = args.p[1];
    nt1 = p.N / (GLU ? 128 : 256);
    nj1 = p.routed ? *p.n_jobs : (p.M + kRows - 1) / kRows;
  }
  const int mine0 = nj0 > xcd ? (nj0 - xcd + 7) >> 3 : 0;  // jobs j = xcd + 8i of problem 0
  const int mine1 = nj1 > xcd ? (nj1 - xcd + 7) >> 3 : 0;
  const int b0 = mine0 * nt0;
  if (lb >= b0 + mine1 * nt1) return;
  const bool second = lb >= b0;
  const MfmaProblem& a = args.p[second ? 1 : 0];
  const int local = second ? lb - b0 : lb;
  const int nt = second ? nt1 : nt0;
  const int job = xcd + 8 * (local / nt), ntile = local % nt;
  int first, nvalid, expert = 0;
  if (a.routed) {
    const int4 jb = a.jobs[job];
    first = jb.x;
    nvalid = jb.y;
    expert = jb.z;
  } else {
    first = job * kRows;
    nvalid = min(kRows, a.M - first);
  }
  const int nmf = (nvalid + 15) >> 4;
  const bool fp8 = FMTS == kAllFp8 || (FMTS == kFp6ThenFp8 && second);
  if (FMTS != kAllFp6 && fp8) {
    if (nmf <= 2)
      mx_job<GLU, 2, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    else if (nmf <= 4)
      mx_job<GLU, 4, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    else if (nmf <= 6)
      mx_job<GLU, 6, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    else if (nmf <= 8)
      mx_job<GLU, 8, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    else if (nmf <= 10)
      mx_job<GLU, 10, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    else
      mx_job<GLU, kMF, true>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
    return;
  }
  if constexpr (FMTS == kAllFp8) return;
  if (nmf <= 2)
    mx_job<GLU, 2, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
  else if (nmf <= 4)
    mx_job<GLU, 4, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
  else if (nmf <= 6)
    mx_job<GLU, 6, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
  else if (nmf <= 8)
    mx_job<GLU, 8, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
  else if (nmf <= 10)
    mx_job<GLU, 10, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
  else
    mx_job<GLU, kMF, false>(a, first, nvalid, expert, ntile, lds_a0, lds_a1, lds_a2, lds_a3, lds_dummy);
}

}  // namespace

hipError_t launch_mx_mfma(const MfmaArgs& a, hipStream_t s) {
  if (a.nprob < 1 || a.nprob > 2) return hipErrorInvalidValue;
  const bool glu = a.p[0].W2 != nullptr;
  long long blocks = 0;
  for (int i = 0; i < a.nprob; ++i) {
    const MfmaProblem& p = a.p[i];
    if ((p.W2 != nullptr) != glu || p.K % 512 || p.K <= 0) return hipErrorInvalidValue;
    // plain problems write fp32 or bf16 rows (bf16: 8-byte stores, so ldo % 4 == 0)
    if (!glu && (!p.outf == !p.outh || (p.outh && p.ldo % 4))) return hipErrorInvalidValue;
    // GLU blocks cover 128 h columns and write whole FP6 windows of h; plain blocks cover 256 columns
    if (glu ? (p.N % 512) : (p.N % 256)) return hipErrorInvalidValue;
    // 32-bit byte offsets: activations, weights of one matrix, outputs
    const long long a_row_bytes = p.fp8 ? (long long)fp8_row_bytes(p.K) : (long long)fp6_row_bytes(p.K);
    // plain (down) problems read A tiled: whole 16-row tiles
    if (p.a_rows < 0 || (!glu && p.a_rows % 16) || p.s_rows < 0 || (long long)p.a_rows * a_row_bytes >= (1ll << 31) ||
        (long long)p.N * p.K / 2 >= (1ll << 31) || (!p.routed && p.M > p.a_rows))
      return hipErrorInvalidValue;
    const long long jobs = p.routed ? p.max_jobs : (p.M + kRows - 1) / kRows;
    blocks += (jobs + 7) / 8 * (p.N / (glu ? 128 : 256));  // per grid-position class (XCD)
  }
  if (blocks == 0) return hipSuccess;
  const long long grid = blocks * 8;
  if (grid > 0x7fffffffll) return hipErrorInvalidValue;
  int fmts;
  if (a.nprob == 1 || a.p[0].fp8 == a.p[1].fp8)
    fmts = a.p[0].fp8 ? kAllFp8 : kAllFp6;
  else if (!a.p[0].fp8)
    fmts = kFp6ThenFp8;
  else
    return hipErrorInvalidValue;
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a); };
  if (glu) {
    if (fmts == kAllFp6) go(mx_mfma_kernel<true, kAllFp6>);
    else if (fmts == kAllFp8) go(mx_mfma_kernel<true, kAllFp8>);
    else go(mx_mfma_kernel<true, kFp6ThenFp8>);
  } else {
    if (fmts == kAllFp6) go(mx_mfma_kernel<false, kAllFp6>);
    else if (fmts == kAllFp8) go(mx_mfma_kernel<false, kAllFp8>);
    else go(mx_mfma_kernel<false, kFp6ThenFp8>);
  }
  return hipGetLastError();
}

}  // namespace moe
