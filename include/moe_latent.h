/*
 * moe_latent.h -- C ABI of the MI355X (gfx950) Stable LatentMoE layer library.
 *
 * The layer (WASTE "Kimi K3, as released", "What is new since Kimi-Linear",
 * item 1, and the "Port status" row "latent MoE"; K3 report review, "Stable
 * LatentMoE"): the hidden state x [T, H] is projected down to a latent z [T, L]
 * (routed_expert_down_proj); a sigmoid router picks top-k of E experts per
 * token; each selected expert is a GLU MLP on the latent whose weights are
 * MXFP4; the expert outputs are combined with their router weights, optionally
 * RMS-normalised (routed_expert_norm), projected back up to H
 * (routed_expert_up_proj) and summed with the full-width shared experts.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers (HIP, one GPU) unless marked "host".
 *   - bf16 tensors are raw 16-bit bit patterns; all matrices are row-major.
 *   - MXFP4 matrix [N, K]: packed U8 [N, K/2], two E2M1 nibbles per byte, the
 *     LOW nibble holds the even element; scales U8 [N, K/32], one E8M0
 *     exponent (value 2^(e-127)) per 32 consecutive weights of a row
 *     (WASTE page, shard-header listing and "Gate 3 repeated on real K3
 *     experts").
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise the host. All argument checks run before
 *     anything is enqueued: on any error return nothing has been enqueued.
 *   - The caller owns every buffer. The library allocates no device memory in
 *     these calls and keeps no per-call state; results are bitwise identical
 *     from run to run for identical inputs.
 *   - Return value: 0 on success or a negative MOE_E* code.
 */
#ifndef MOE_LATENT_H
#define MOE_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_LATENT_ABI_VERSION 6

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null pointer, negative or inconsistent size */
#define MOE_EUNSUPPORTED (-2) /* sizes outside what the kernels handle (see moe_latent_dims) */
#define MOE_EALIAS (-3)       /* an output overlaps an input or the workspace */
#define MOE_EWORKSPACE (-4)   /* workspace too small or misaligned */
#define MOE_EHIP (-5)         /* a HIP launch failed; moe_latent_last_hip_error() has the code */
#define MOE_EABI (-6)         /* struct_size does not match this library */

/* Expert contraction kernels (moe_latent_dims.expert_path).
 *   MOE_PATH_STREAM: per 16-slot tile, weights streamed once per tile and
 *     dequantised to bf16 for bf16 MFMAs; for decode-sized batches, where the
 *     layer is bound by reading the touched experts' bytes.
 *   MOE_PATH_MFMA: grouped GEMM on the scaled MXFP4 MFMA; the activations are
 *     encoded per 32 values as two MXFP6 (E2M3) planes, hi and lo, whose sum
 *     keeps about 8 significant bits; for prefill-sized batches. Needs hidden,
 *     latent, inter and shared_inter to be multiples of 512.
 *   MOE_PATH_AUTO: MFMA when its size rule holds and the batch averages at
 *     least 12 token slots per expert (T*k >= 12*E), else STREAM. The
 *     streaming path reads an expert's weights once per 16 slots, the MFMA
 *     path once per 192; for the K3 layer on MI355X the two cross between
 *     T = 512 and T = 768 (T*k = 10.1*E .. 13.7*E). */
#define MOE_PATH_AUTO 0
#define MOE_PATH_STREAM 1
#define MOE_PATH_MFMA 2

/* Activation format of the routed experts (moe_latent_dims.act_format).
 *   MOE_ACT_BF16: the experts read the bf16 latent and the bf16-precision GLU
 *     output (the MFMA path's hi/lo MXFP6 encoding keeps about 8 significant
 *     bits of them).
 *   MOE_ACT_MXFP8: both expert inputs are MXFP8 -- E4M3 elements, one E8M0
 *     scale 2^(floor(log2 amax) - 8) per 32 consecutive values of a row,
 *     round to nearest even, saturation at 448 (OCP Microscaling v1.0) -- the
 *     deployment numerics the K3 report review describes in its
 *     quantization-aware training section (MXFP4 weights, MXFP8 activations).
 *     The shared experts, projections and router keep their precision; the
 *     z tap reports the latent before quantization. */
#define MOE_ACT_BF16 0
#define MOE_ACT_MXFP8 1

/* GLU activation of the routed and the shared experts (moe_latent_dims.glu_act).
 *   MOE_GLU_SILU: SiLU(gate) * up.
 *   MOE_GLU_SITU: SiTU, the activation K3 uses instead of SiLU in both FFN paths (WASTE
 *     "Kimi K3, as released", "What is new since Kimi-Linear" item 3: beta 4.0, linear
 *     beta 25.0). The pages do not print its formula; this library takes the reading
 *       SiTU(gate, up) = b * tanh(SiLU(gate) / b) * lb * tanh(up / lb)
 *     with b = situ_beta, lb = situ_linear_beta: the sigmoid branch and the linear branch
 *     each soft-limited by beta * tanh(z / beta), so |output| < b * lb (100 for K3) and the
 *     unit is SwiGLU up to O(z^3 / beta^2) near the origin (K3 report review, "SiTU-GLU").
 *     Agreement with K3's own implementation is not established. */
#define MOE_GLU_SILU 0
#define MOE_GLU_SITU 1

/* Layer sizes. Limits checked by every call (else MOE_EUNSUPPORTED):
 * hidden, latent, inter, shared_inter multiples of 256 (512 for MOE_PATH_MFMA);
 * 1 <= n_experts <= 65535; latent <= 8192; align_block 0 (library choice, 16) or
 * a multiple of 16; the expert-sorted intermediate (capacity x inter bf16) and
 * x (T x hidden bf16) below 2 GiB each. */
typedef struct moe_latent_dims {
  uint32_t struct_size;        /* = sizeof(moe_latent_dims) */
  int32_t T;                   /* tokens (0 is allowed: nothing is enqueued, pointers are not read) */
  int32_t hidden;              /* H, 7168 for K3 */
  int32_t latent;              /* L, 3584 */
  int32_t n_experts;           /* E, 896 */
  int32_t inter;               /* I, expert intermediate width, 3072 */
  int32_t shared_inter;        /* merged shared GLU width (6144), 0 = no shared experts */
  int32_t align_block;         /* B of the expert-sorted layout */
  float rms_eps;               /* RMSNorm epsilon (1e-6) */
  float routed_scaling_factor; /* 1.0 for K3 */
  int32_t expert_path;         /* MOE_PATH_* */
  int32_t act_format;          /* MOE_ACT_* */
  int32_t glu_act;             /* MOE_GLU_* */
  float situ_beta;             /* MOE_GLU_SITU: beta of the gate (sigmoid) branch, > 0 (4.0 for K3) */
  float situ_linear_beta;      /* MOE_GLU_SITU: beta of the linear (up) branch, > 0 (25.0 for K3) */
} moe_latent_dims;

/* Router (WASTE page, "Shape" router row and "Against the technical report"). */
typedef struct moe_router {
  const float* weight;      /* fp32 [E, H] */
  const float* select_bias; /* fp32 [E] or NULL: added to the sigmoid scores for selection only */
} moe_router;

/* Merged shared experts, one GLU H -> Is -> H (K3 report review, parameter
 * count, second step; MXFP4 as in SlimServe quants.md's K3 tensor table). */
typedef struct moe_shared {
  const uint8_t* packed; /* [gate Is x H/2 | up Is x H/2 | down H x Is/2] */
  const uint8_t* scales; /* [gate Is x H/32 | up Is x H/32 | down H x Is/32] */
} moe_shared;

/* Optional copies of intermediates (each pointer may be NULL). */
typedef struct moe_latent_taps {
  uint32_t struct_size;   /* = sizeof(moe_latent_taps) */
  uint16_t* z;            /* bf16 [T, L]  down-projection */
  float* logits;          /* fp32 [T, E]  router logits */
  int32_t* topk_ids;      /* [T, k]       selected experts, ascending id per token */
  float* topk_w;          /* fp32 [T, k]  routing weights */
  int32_t* counts;        /* [E]          pairs per expert */
  int32_t* sorted_ids;    /* [capacity]   expert-sorted flat slot indices (see moe_align_block_size) */
  int32_t* expert_ids;    /* [capacity/B] */
  int32_t* num_post;      /* [1] */
  int32_t* inv_pos;       /* [T*k]        position of slot t*k+j in sorted_ids */
  float* c;               /* fp32 [T, L]  weighted aggregate before the norm */
  uint16_t* c_norm;       /* bf16 [T, L]  the normalised aggregate RMSNorm(c) (for T > 64 the
                                           up-projection's input; for T <= 64 the
                                           up-projection reads bf16(g * c) and its output
                                           is scaled by 1 / rms(c), the same function) */
  float* y_routed;        /* fp32 [T, H]  up-projection output */
  float* y_shared;        /* fp32 [T, H]  shared experts' output (zeros if none); on the MFMA path
                             above 64 tokens whose up-projection is not split over K, the layer
                             keeps it in bf16 and the tap holds those values widened to fp32 */
  float* O;               /* fp32 [T*k, L] the routed expert's output of slot t*k+j (token t's
                             j-th selected expert), before the routing weight; on the MFMA path
                             above 64 tokens the layer keeps O in bf16, and the tap holds those
                             bf16 values widened to fp32 */
} moe_latent_taps;

int moe_latent_abi_version(void);
const char* moe_latent_strerror(int code);
/* hipError_t of the last MOE_EHIP returned on this host thread (0 if none). */
int moe_latent_last_hip_error(void);

/* Host-only. Workspace bytes needed by moe_latent_forward for these sizes. */
int moe_latent_workspace_size(const moe_latent_dims* d, int topk, size_t* bytes);

/* Host-only. Entries of the expert-sorted layout (capacity) and the block B
 * the library uses for these sizes:
 * capacity = B * floor((T*k + min(E, T*k)*(B-1)) / B). */
int moe_latent_align_layout(const moe_latent_dims* d, int topk, int32_t* capacity, int32_t* block);

/*
 * One layer forward: y = up(norm(sum_j w_tj * expert_{e_tj}(down(x_t)))) + shared(x_t).
 *
 *   x               bf16 [T, H]
 *   down            bf16 [L, H]   routed_expert_down_proj
 *   norm            bf16 [L] or NULL (no RMSNorm)
 *   router          fp32 weight [E, H], optional fp32 select_bias [E]
 *   experts_packed  U8 [E][w1 I x L/2 | w3 I x L/2 | w2 L x I/2]; w1 = gate, w3 = up, w2 = down
 *   experts_scales  U8 [E][w1 I x L/32 | w3 I x L/32 | w2 L x I/32]
 *   up              bf16 [H, L]   routed_expert_up_proj
 *   shared          merged shared GLU or NULL
 *   topk            experts per token, 1 <= topk <= min(E, 64)
 *   y               bf16 [T, H] output
 *   workspace       >= moe_latent_workspace_size bytes, 256-byte aligned
 *
 * Aliasing: y, the workspace and every tap must overlap no input (x, down, norm,
 * router weight and bias, the expert records, up, the shared record) and no other
 * of them (MOE_EALIAS); inputs may overlap one another.
 *
 * Routing: s = sigmoid(x . W_r^T), key = s + select_bias; the topk largest keys
 * win, ties to the lower expert id; weights w = s / sum(s_selected) * rsf. The
 * experts' GLU activation is d->glu_act (SiLU(gate) * up or SiTU). Near-ties of the key at the k-th place
 * can route differently from a float64 evaluation (fp32 here).
 *
 * Debugging: when the environment variable MOE_DUMP_ROUTE names a file, moe_latent_forward
 * and moe_latent_forward_ex synchronize the stream after their launches and append one record
 * per call: the 4 bytes "MOER", int32 T, k, E, then int32 topk_ids [T, k] and float topk_w
 * [T, k], little-endian. The variable is read on every call; leave it unset under graph
 * capture. A record that cannot be written does not fail the call.
 */
int moe_latent_forward(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                       const moe_router* router, const uint8_t* experts_packed, const uint8_t* experts_scales,
                       const void* up, const moe_shared* shared, int topk, void* y, void* workspace,
                       size_t ws_bytes, void* stream);

/* As moe_latent_forward, also copying the intermediates requested in `taps`
 * (device pointers, sizes as in moe_latent_taps; taps may be NULL). */
int moe_latent_forward_ex(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                          const moe_router* router, const uint8_t* experts_packed,
                          const uint8_t* experts_scales, const void* up, const moe_shared* shared, int topk,
                          void* y, void* workspace, size_t ws_bytes, void* stream, const moe_latent_taps* taps);

/*
 * moe_latent_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. The workspace is a static array of
 * MOE_LATENT_STATIC_SCRATCH_BYTES in the library's code object, one copy per GPU, held
 * until the process ends (its device address is looked up once per device). It holds
 * the workspace of a K3-shape decode batch of up to 16 tokens (13.6 MiB at T = 16);
 * layers whose moe_latent_workspace_size exceeds it return MOE_EWORKSPACE before
 * anything is enqueued. Arguments, results and errors otherwise as moe_latent_forward
 * (the current device must be the stream's); no stage events are recorded. Every call
 * on one GPU uses that GPU's one array: calls whose execution overlaps on one GPU (on
 * different streams, or from several host threads) race and give wrong results; calls
 * in one stream's order are safe. Each call writes every part of the array it later
 * reads, so nothing carries over from one call to the next.
 */
#define MOE_LATENT_STATIC_SCRATCH_BYTES (16u << 20)
int moe_latent_forward_noalloc(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                               const moe_router* router, const uint8_t* experts_packed,
                               const uint8_t* experts_scales, const void* up, const moe_shared* shared, int topk,
                               void* y, void* stream);

/*
 * Routing only: logits = x . W_r^T (fp32), then the selection of
 * moe_latent_forward. Writes topk_ids [T, topk] (ascending ids per token) and
 * topk_w [T, topk]; logits [T, E] fp32 is required scratch/output.
 */
int moe_route(const moe_latent_dims* d, const void* x, const moe_router* router, int topk, int32_t* topk_ids,
              float* topk_w, float* logits, void* stream);

/* Host-only. Device scratch bytes moe_align_block_size needs. */
int moe_align_workspace_size(int T, int topk, int n_experts, size_t* bytes);

/*
 * moe_align_block_size (SlimServe quants.md, note on the alignment fix): the
 * expert-sorted layout of the T*topk (token, slot) pairs.
 *   topk_ids   [T, topk], ids in [0, E), each token listing an expert at most
 *              once (the router's ids are distinct). Ids outside the range get no
 *              entry and inv_pos -1; an id a token repeats keeps its first slot and
 *              its later slots are handled like ids out of range.
 *   block      B >= 1: every expert segment is padded to a multiple of B; a
 *              consumer with tile height h | B expands expert_ids B/h times
 *   sorted_ids [capacity]: segments in ascending expert id, each the flat
 *              indices t*topk+j in ascending order then the sentinel T*topk;
 *              the tail past num_post also holds the sentinel
 *   expert_ids [capacity/B]: expert of each block, -1 past num_post
 *   num_post   [1]: padded entry count; inv_pos [T*topk]; counts [E]
 *   scratch    >= moe_align_workspace_size bytes
 * capacity as in moe_latent_align_layout. Integer-only and bit-exact.
 * 1 <= n_experts <= 65535; above 4096 experts topk <= 64 (else MOE_EUNSUPPORTED).
 */
int moe_align_block_size(const int32_t* topk_ids, int T, int topk, int n_experts, int block, int32_t* sorted_ids,
                         int32_t* expert_ids, int32_t* num_post, int32_t* inv_pos, int32_t* counts, void* scratch,
                         size_t scratch_bytes, void* stream);

/*
 * The MXFP8 rounding that MOE_ACT_MXFP8 applies to the routed experts' inputs
 * (K3 report review, quantization-aware training section; element and scale
 * rules of OCP Microscaling v1.0 as stated at MOE_ACT_MXFP8): y = the MXFP8
 * value of x per block of 32 consecutive values of a row, stored back in bf16.
 *   x, y   bf16 [rows, K] device, 16-byte aligned; y may equal x (in place),
 *          other overlaps are MOE_EALIAS
 *   K      multiple of 32; rows >= 0 (0 enqueues nothing)
 * Results are exact, down to magnitudes of 2^-126 (below that the bf16 store
 * rounds). Each element's rounding decision is taken on the exact quotient
 * x / 2^s, so it matches any exact evaluation bit for bit.
 */
int moe_mxfp8_round(const void* x, int rows, int K, void* y, void* stream);

/*
 * Quantile Balancing (K3 report review, section on Quantile Balancing): the
 * selection-only router bias that gives every expert the target load
 * q = max(1, floor(m*k/n)) of m tokens, n experts and k experts per token.
 * Each token's threshold alpha is the (k+1)-th largest of its biased keys
 * s + b; its margin at expert j is s_j - alpha; expert j's new bias is minus
 * the margin that q of its margins reach, estimated from a histogram of
 * MOE_QB_BINS bins of width 0.004 over [-2, 2) (margins outside are counted in
 * the end bins). Summing the histograms of several batches (integer addition,
 * the page's all-reduce) before moe_qb_bias gives the update of their union.
 * The new bias takes effect as moe_router.select_bias of later forwards.
 * Exact fp32 operations, in this order, with no contraction:
 *   key = s + b;  mu = s - alpha;  bin = min(999, max(0, floor((mu + 2) * 250)));
 *   new_bias = -(-2 + t * 0.004), t = the largest bin whose count from t up
 *   to the last bin reaches q (the lower edge of the bin that holds the q-th
 *   largest margin, so within one bin width of the exact quantile).
 */
#define MOE_QB_BINS 1000

/*
 * Thresholds and margin histograms of one batch.
 *   scores  fp32 [m, n] router scores (sigmoid of the logits), finite, 16-byte aligned
 *   bias    fp32 [n] current selection bias, or NULL (zero)
 *   m >= 0 tokens, 2 <= n <= 4096 experts, 1 <= topk < n
 *   alpha   fp32 [m] out: each token's threshold
 *   hist    int32 [n, MOE_QB_BINS] out, fully overwritten (zeros when m = 0)
 * Outputs must not overlap the inputs or each other (MOE_EALIAS). Integer
 * results: bit-exact against any exact fp32 evaluation of the rules above.
 */
int moe_qb_histogram(const float* scores, const float* bias, int m, int n, int topk, float* alpha, int32_t* hist,
                     void* stream);

/*
 * One batch's update in one call: moe_qb_histogram followed by moe_qb_bias with
 * m_total = m (m >= 1), the bias taken from the histograms in the same launch.
 * For several batches (ranks) sum their histograms and call moe_qb_bias instead.
 *   new_bias  fp32 [n] out, overlapping no other argument
 */
int moe_qb_update(const float* scores, const float* bias, int m, int n, int topk, float* alpha, int32_t* hist,
                  float* new_bias, void* stream);

/* Host-only. The integer target q = max(1, floor(m_total*topk/n)) into *q. */
int moe_qb_target(long long m_total, int n, int topk, long long* q);

/*
 * New selection bias from (summed) histograms.
 *   hist      int32 [n, MOE_QB_BINS], counts of m_total margins per expert
 *   m_total   tokens the histograms cover (over every batch summed into them)
 *   new_bias  fp32 [n] out; NaN for an expert whose histogram holds fewer than
 *             q margins (inconsistent m_total); must not overlap hist
 */
int moe_qb_bias(const int32_t* hist, int n, long long m_total, int topk, float* new_bias, void* stream);

/*
 * Measurement, not a step of the layer: the HBM read bandwidth that the
 * weight-streaming expert kernels are compared against. Reads every 16-byte
 * chunk of `buf` once with non-temporal loads (as those kernels read their
 * weights) and writes the XOR of all its dwords to *checksum, a value that does
 * not depend on the order of the reads (so it can be checked against the host).
 *   buf       device, 16-byte aligned, `bytes` a multiple of 16 (0 gives 0)
 *   checksum  device uint32, must not overlap buf
 */
int moe_hbm_read(const void* buf, size_t bytes, uint32_t* checksum, void* stream);

/*
 * RMSNorm of bf16 rows, y = x / sqrt(mean(x^2) + eps) * g, with g = 1 when weight
 * is NULL. The layer applies the same formula to the aggregated latent (K3
 * report review, "Stable LatentMoE"; WASTE "Kimi K3, as released", "Against the
 * technical report": RMSNorm before the up-projection); a decoder applies it
 * without the MoE, before each layer's input, which is what a stack of layers
 * needs between one layer's output and the next layer's input.
 *   x, y    bf16 [rows, cols] device, 8-byte aligned; y may equal x (in place),
 *           other overlaps are MOE_EALIAS
 *   weight  bf16 [cols] device or NULL; must not overlap y
 *   cols    multiple of 4; rows >= 0 (0 enqueues nothing); eps >= 0
 * Sum of squares in fp32 in a fixed order (bitwise reproducible), result rounded
 * to bf16 (nearest even).
 */
int moe_rmsnorm(const void* x, int rows, int cols, const void* weight, float eps, void* y, void* stream);

/*
 * Stage timing for measurement. While enabled, moe_latent_forward records HIP
 * events around each stage on its stream (at most 256 forwards are kept).
 * moe_latent_timing_read synchronises on the recorded events and returns, per
 * stage, the summed milliseconds and the number of forwards recorded; it then
 * clears the record. A forward that returned an error is not counted (its record
 * is incomplete and skipped). Stage names: moe_latent_stage_name(i), i < stage
 * count.
 */
int moe_latent_timing_enable(int on);
int moe_latent_stage_count(void);
const char* moe_latent_stage_name(int i);
int moe_latent_timing_read(float* ms_per_stage /* host [stage count] */, int* n_forwards /* host */);

/*
 * Releases what the library keeps between calls: the stage-timing events (timing
 * is switched off and its record cleared). Call it with no forward in flight,
 * e.g. before the process unloads the library; later calls work as before (the
 * events are created again when timing is enabled).
 */
int moe_latent_shutdown(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LATENT_H */
