// Internal launchers of the latent-MoE HIP kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// ---------------------------------------------------------------- dense projections
// out[m][n] = sum_k A[m][k] * W[n][k] for one or two weight segments sharing A.
enum DenseOut : int {
  kStoreBf16 = 0,       // out bf16 [M, ldo]
  kStoreF32 = 1,        // out f32  [M, ldo]
  kAddStoreBf16 = 2,    // out bf16 = bf16(acc + addend[m][n]) (addend may be null); tap f32 = acc
  kPartF32 = 3,         // out f32 planes [splits][M][ldo]: plane s = the sum over K slice s
};

struct DenseSeg {
  const void* W;        // [N, K] row-major, bf16 bits or fp32
  int N;                // rows of W
  int w_f32;            // 1: W is fp32, split exactly into three bf16 planes
  int mode;             // DenseOut
  void* out;
  int ldo;
  const float* addend;  // kAddStoreBf16 only
  int ld_add;
  float* tap;           // kAddStoreBf16 only, optional
  int ld_tap;
};

struct DenseArgs {
  const uint16_t* A;    // bf16 [M, lda]
  int lda, M, K;        // K multiple of 128
  DenseSeg seg[2];
  int nseg;
};

hipError_t launch_dense(const DenseArgs& a, hipStream_t s);

// ---------------------------------------------------------------- dense projections, large batches
// out = A . W^T per segment; A bf16 [M, lda]; W bf16 [N, K]; A's column for k is k mod kwrap
// (kwrap = K, or the width of A when W holds three split planes of fp32 weights).
struct GemmSeg {
  const uint16_t* W;
  int N, K, kwrap;      // K multiple of 256, kwrap multiple of 64
  int mode;             // DenseOut
  void* out;
  int ldo;
  const float* addend;  // kAddStoreBf16 only (may be null)
  int ld_add;
  float* tap;           // kAddStoreBf16 only, optional
  int ld_tap;
  int splits;           // kPartF32: K slices (M below the 256 x 224 tile's threshold); else 0 or 1
  int w_f32;            // 1: W is fp32 [N, K], split into three bf16 planes as it is staged (M < 2048)
  const uint16_t* addend16;  // kAddStoreBf16: a bf16 addend [m][n] (stride ld_add) instead of addend
};
struct GemmArgs {
  const uint16_t* A;
  int lda, M;
  GemmSeg seg[2];
  int nseg;
};
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s);
// K slices per segment (N[i] x K[i], nseg <= 2) for a split-K launch of M < 2048 rows that
// puts one block on each of num_cu compute units
void gemm_split_plan(int M, int nseg, const int* N, const int* K, int num_cu, int* splits);
// 2048+ rows: K slices (1 or 2) for segment 1 of a two-segment launch (the router's planes)
int gemm_large_split(int M, const int* N, const int* K, int num_cu);
// fp32 [N, K] -> bf16 [N, 3K] rows hi | mid | lo with w = hi + mid + lo exactly
hipError_t launch_split3(const float* W, int N, int K, uint16_t* out, hipStream_t s);

// ---------------------------------------------------------------- decode-size dense projections
// Split-K streaming GEMV for M <= 64 tokens: part[slice][m][n] = sum over the slice's K of A[m][k] W[n][k].
struct GemvSeg {
  const void* W;   // [N, K] row-major, bf16 bits or fp32
  int N;           // rows of W
  int w_f32;       // 1: fp32 weights, split exactly into three bf16 planes
  int splits;      // K slices (each a whole number of 256-byte row steps)
  float* part;     // [splits][M][N] fp32 partial sums
};
struct GemvArgs {
  const uint16_t* A;  // bf16 [M, lda]
  int lda, M, K;      // K * (2 or 4) bytes a multiple of 256
  GemvSeg seg[2];
  int nseg;
};
hipError_t launch_dense_gemv(const GemvArgs& a, hipStream_t s);
// y = bf16(r * sum_s part[s] + addend); tap = r * sum_s part[s] (fp32), both [M, N]; N % 4 == 0.
// r = 1, or with part_sq [M, nq] the row's 1 / sqrt(sum_i part_sq[m][i] / L + eps) (sum in i order)
struct RowScale {
  const float* part_sq;
  int nq, L;
  float eps;
};
hipError_t launch_finish_up(const float* part, int splits, int M, int N, const float* addend, uint16_t* y, float* tap,
                            RowScale rs, hipStream_t s);

// ---------------------------------------------------------------- router
struct RouteArgs {
  const float* logits;  // [T][E] router logits the selection reads
  const float* r_part;  // optional split-K logit planes [sr][T][E], summed into logits_out (== logits)
  int sr;
  const float* z_part;  // optional latent partial planes [sz][T][L], summed and rounded to bf16 into z_out
  int sz, L;
  uint16_t* z_out;
  float* logits_out;
  const float* bias;    // selection-only bias [E] or null
  int T, E, k;
  float rsf;
  int32_t* ids;         // [T][k], ascending expert id per token
  float* w;             // [T][k]
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// ---------------------------------------------------------------- align
size_t align_scratch_bytes(int T, int E);
int align_capacity(int T, int k, int E, int B);
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int B, int32_t* counts, int32_t* sorted_ids,
                        int32_t* expert_ids, int32_t* num_post, int32_t* inv_pos, void* scratch, hipStream_t s);

// ---------------------------------------------------------------- MXFP4 contractions
// Row of slot position pos of the expert-sorted layout in a routed problem's tensors:
// kRowToken = the slot's token sorted_ids[pos] / topk, kRowPos = pos itself, kRowFlat = the
// flat slot index sorted_ids[pos] = t * topk + j (tensors with one row per (token, slot)).
enum RowMode : int { kRowToken = 0, kRowPos = 1, kRowFlat = 2 };
// One grouped contraction problem: out[row] = act(A_row . W1^T, A_row . W2^T) (GLU) or A_row . W^T.
struct MxProblem {
  // activations: bf16 rows
  const uint16_t* A;
  int lda;
  int routed;                 // 1: the rows are the slots of the expert-sorted layout; 0: dense rows
  int a_row;                  // routed: A row of slot pos (kRowToken, kRowPos or kRowFlat)
  int out_row;                // routed: output row of slot pos (kRowPos or kRowFlat)
  const int32_t* sorted_ids;  // routed
  const int32_t* expert_ids;  // routed: expert of each layout block of B slots
  int tiles_per_block;        // routed: B / 16 (the kernel's 16-slot tiles per layout block)
  const int32_t* num_post;    // routed: device scalar, padded slot count
  int pairs, topk;            // routed
  int M;                      // dense: number of rows
  int max_blocks;             // 16-slot tiles to cover (upper bound; extra tiles exit)
  // weights (MXFP4): matrix of expert e at W + e*w_stride, [N, K/2] bytes; scales at S + e*s_stride, [N, K/32]
  const uint8_t* W;
  const uint8_t* S;
  const uint8_t* W2;          // GLU: the up matrix (same layout), null for a plain contraction
  const uint8_t* S2;
  size_t w_stride, s_stride;
  int N, K;                   // K multiple of 256, N multiple of the block's columns
  // output: GLU -> bf16 [rows, ldo] = act(gate) * up; plain -> f32 [rows, ldo]
  void* out;
  int ldo;
  int out_fp8;                // GLU: h rounded to its MXFP8 value per 32 columns before the bf16 store
  GluAct act;                 // GLU: the activation
};

// Up to two problems of the same kind (both GLU or both plain) in one launch;
// problem 0's blocks come first in the grid.
struct MxArgs {
  MxProblem p[2];
  int nprob;
};

hipError_t launch_mx_small(const MxArgs& a, hipStream_t s);

// ---------------------------------------------------------------- MXFP6 activations (scaled-MFMA path)
// bf16 [rows, lda] -> FP6 E2M3 hi/lo tensor of rows of K values, row after row (layout in
// mxfp6.h); K % 512 == 0
hipError_t launch_quant_fp6(const uint16_t* A, int lda, int rows, int K, uint8_t* data, uint8_t* scales,
                            hipStream_t s);

// ---------------------------------------------------------------- MXFP8 activations (mxfp8.h)
// out = the MXFP8 value of in, per 32 consecutive values of a row, stored as bf16 (exact
// down to 2^-126); rows x K with K % 32 == 0; in and out may be the same buffer.
hipError_t launch_qdq_fp8(const uint16_t* in, int ld_in, int rows, int K, uint16_t* out, int ld_out,
                          hipStream_t s);
// bf16 [rows, lda] -> MXFP8 tensor (E4M3 codes [rows, K], scales [rows, K/32], layout in mxfp8.h); K % 512 == 0
hipError_t launch_quant_fp8(const uint16_t* A, int lda, int rows, int K, uint8_t* data, uint8_t* scales,
                            hipStream_t s);

// Work list of the grouped MFMA contraction: one job per chunk of at most `slots_per_job`
// token slots of one expert, in the expert-sorted layout with block B.
// jobs[j] = {first slot, valid slots, expert, 0}; *n_jobs = number of jobs.
int mx_max_jobs(int pairs, int E, int slots_per_job);
hipError_t launch_mx_jobs(const int32_t* counts, int E, int B, int slots_per_job, int4* jobs, int32_t* n_jobs,
                          hipStream_t s);

// Grouped MXFP4 contraction on the scaled MFMA: A = FP6 hi/lo or MXFP8 activations, B = MXFP4 weights.
struct MfmaProblem {
  int fp8;                    // 0: A (and a GLU's h) in FP6 hi/lo (mxfp6.h); 1: in MXFP8 (mxfp8.h)
  const uint8_t* Aq;          // A data (1.5*K bytes per row FP6, K bytes FP8): GLU problems row after
                              // row; plain problems tiled (atile_offset), row = slot position / row
  const uint8_t* Aqs;         // A scales, row after row (K/16 bytes per row FP6, K/32 bytes FP8)
  int a_rows;                 // rows of the A data (plain: a multiple of 16); bounds its buffer resource
  int s_rows;                 // rows of the scale tensor (bounds its buffer resource)
  int routed;                 // 1: jobs from the table below; 0: dense rows 0..M-1
  int a_by_pos;               // routed: scale row = slot position; else sorted_ids[slot] / topk
  const int32_t* sorted_ids;  // routed
  int topk;
  const int4* jobs;           // routed
  const int32_t* n_jobs;      // routed, device scalar
  int max_jobs;               // routed: capacity of the job table
  int M;                      // dense rows
  const uint8_t* W;           // MXFP4 [N, K/2] of expert e at W + e*w_stride (GLU: gate)
  const uint8_t* S;           // E8M0 [N, K/32]
  const uint8_t* W2;          // GLU: up matrix; null for a plain contraction
  const uint8_t* S2;
  size_t w_stride, s_stride;
  int N, K;                   // GLU: N = h width, multiple of 512; plain: N multiple of 256; K multiple of 512
  uint8_t* outq;              // GLU: h rows in A's format, data tiled (routed: slot position, dense: row), width N
  uint8_t* outqs;
  float* outf;                // plain: fp32 [row, ldo] (routed: slot position, or with out_flat the
                              // flat slot index t * topk + j)
  uint16_t* outh;             // plain, instead of outf when set: the same rows rounded to bf16
  int out_flat;
  GluAct act;                 // GLU: the activation
  int ldo;
};
struct MfmaArgs {
  MfmaProblem p[2];
  int nprob;                  // both GLU or both plain; problem 0's blocks first
};
constexpr int kMfmaSlotsPerJob = 192;  // 12 MFMA row tiles of 16
hipError_t launch_mx_mfma(const MfmaArgs& a, hipStream_t s);

// ---------------------------------------------------------------- combine + norm
// c_t = sum_j w[t][j] * O[row of slot t * k + j] in slot order: O fp32 by flat slot index
// (inv_pos null) or by layout position (row = inv_pos[t * k + j])
hipError_t launch_combine_norm(const float* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float eps, float* c_tap, uint16_t* c_norm, hipStream_t s);
// the same with O in bf16 (the MFMA path's down output above 64 rows)
hipError_t launch_combine_norm_bf16(const uint16_t* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float eps, float* c_tap, uint16_t* c_norm, hipStream_t s);

// Decode batches: c [T, L] fp32 (required) and cg = bf16(c * g) (bf16(c) without a norm
// weight) for the up-projection, token t's columns spread over L / 256 blocks; with the norm,
// part_sq [T, L / 256] = each block's sum of c^2, from which finish_up applies 1 / rms(c) to
// the up-projection's output. L % 256 == 0, k <= 64.
hipError_t launch_combine_cols(const float* O, int L, const int32_t* inv_pos, const float* w, int T, int k,
                               const uint16_t* norm, float* c, uint16_t* cg, float* part_sq, hipStream_t s);
// out = bf16(c * s * g) per row with s = 1 / sqrt(sum(part_sq row) / L + eps) (the normalised
// aggregate, for the c_norm tap of the decode path)
hipError_t launch_norm_from_parts(const float* c, const float* part_sq, int T, int L, const uint16_t* norm, float eps,
                                  uint16_t* out, hipStream_t s);

// y = x / sqrt(mean(x^2) + eps) * g per row (g null: no weight); bf16 [rows, cols], cols % 4 == 0; y may be x
hipError_t launch_rmsnorm(const uint16_t* x, int rows, int cols, const uint16_t* g, float eps, uint16_t* y,
                          hipStream_t s);

// ---------------------------------------------------------------- Quantile Balancing
constexpr int kQbBins = 1000;
// alpha [m] = (k+1)-th largest of scores[t] + bias; hist [n, kQbBins] int32 = margin histograms.
// scores fp32 [m, n], 16-byte aligned; 2 <= n <= 4096; 1 <= k < n; m >= 0 (m = 0 stores zero histograms).
// With new_bias non-null, also new_bias [n] for the target q (the histograms' own batch).
hipError_t launch_qb_histogram(const float* scores, const float* bias, int m, int n, int k, float* alpha,
                               int32_t* hist, long long q, float* new_bias, hipStream_t s);
// new_bias [n] from hist [n, kQbBins] and the integer target q >= 1 (NaN where fewer than q margins)
hipError_t launch_qb_bias(const int32_t* hist, int n, long long q, float* new_bias, hipStream_t s);

// ---------------------------------------------------------------- streaming read (measurement)
// *checksum = XOR of all dwords of buf (bytes % 16 == 0, buf 16-byte aligned), every chunk read once.
hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* checksum, hipStream_t s);

// out[i] = src[idx[i]] for rows of `cols` floats (cols % 4 == 0), i < n
hipError_t launch_gather_rows_f32(const float* src, int cols, const int32_t* idx, int n, float* out, hipStream_t s);
hipError_t launch_gather_rows_bf16(const uint16_t* src, int cols, const int32_t* idx, int n, float* out, hipStream_t s);
hipError_t launch_widen_bf16(const uint16_t* src, size_t n, float* out, hipStream_t s);  // n % 4 == 0

// fill with a constant (a kernel, so that captured graphs hold no memset node)
hipError_t launch_fill_f32(float* p, size_t n, float v, hipStream_t s);

}  // namespace moe
