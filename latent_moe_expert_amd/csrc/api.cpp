// C ABI of the latent-MoE layer library: validation, workspace plan, launches.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/moe_latent.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return MOE_EHIP;
}
#define MOE_HIP(call)                         \
  do {                                        \
    hipError_t e_ = (call);                   \
    if (e_ != hipSuccess) return hip_fail(e_); \
  } while (0)

constexpr int kMaxExperts = 65535;  // expert ids are int32 throughout; the router and align switch to
                                     // their large-E forms above 4096
constexpr int kMaxTopk = 64;
constexpr int kMaxQbExperts = 4096;  // Quantile Balancing: one wave holds a token's scores, 64 per lane
constexpr int kMaxLatent = 8192;
constexpr int kNumCu = 256;  // MI355X compute units: the split-K GEMM sizes its grid for them

// ------------------------------------------------------------------ stage timing
enum Stage { kProjRouter, kTopk, kAlign, kActEncode, kExpGateUp, kExpDown, kCombine, kUpProj, kNumStages };
// act_encode: the MXFP6 or MXFP8 encoding of the contraction inputs (MOE_PATH_MFMA), or
// the MXFP8 rounding of z (MOE_PATH_STREAM with MOE_ACT_MXFP8); ~0 otherwise.
// The shared experts' contractions run inside the expert_gate_up / expert_down launches.
const char* kStageNames[kNumStages] = {"proj_router", "topk", "align", "act_encode", "expert_gate_up",
                                       "expert_down", "combine_norm", "up_proj"};
constexpr int kMaxTimed = 256;

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;  // kMaxTimed * (kNumStages + 1)
  std::vector<char> done;      // record f complete: every stage event of that forward was recorded
  int n = 0;                   // records claimed
  // events of the next forward (claimed, not yet complete), or null when full
  hipEvent_t* claim(int* idx) {
    if (n >= kMaxTimed) return nullptr;
    const size_t need = (size_t)(n + 1) * (kNumStages + 1);
    while (ev.size() < need) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      ev.push_back(e);
    }
    done.resize((size_t)n + 1);
    done[(size_t)n] = 0;
    *idx = n++;
    return &ev[(size_t)*idx * (kNumStages + 1)];
  }
  void release() {  // caller holds mu
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    done.clear();
    n = 0;
  }
} g_timing;

// ------------------------------------------------------------------ plan
size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Plan {
  int T, H, L, E, I, Is, k, B, cap, pairs;
  bool small;      // T <= 64: split-K streaming projections
  bool mid;        // 64 < T < 2048: the 128 x 128 GEMM, split over K where its tiles leave compute units idle
  bool mfma;       // expert contractions on the scaled MFMA (MOE_PATH_MFMA)
  bool fp8;        // MXFP8 activations of the routed experts (MOE_ACT_MXFP8)
  int max_jobs;    // mfma: capacity of the job table
  int sz, sr, su;  // K slices of the down-projection, the router and the up-projection (1: none)
  size_t z, z8, logits, ids, w, counts, sorted, expert_ids, num_post, inv_pos, align_scratch, h, O, cn, hs, ys;
  size_t z_part, r_part, y_part;
  size_t cf, psq;  // small: c fp32 [T, L] and each column block's sum of c^2 [T, L/256]
  size_t zq, zqs, xq, xqs, hq, hqs, hsq, hsqs, jobs, n_jobs;  // mfma: FP6 activations and the job table
  size_t wr3;      // T > 64: router weight split into three bf16 planes [E, 3H]
  size_t total;
};

bool mfma_sizes_ok(const moe_latent_dims* d) {
  return d->hidden % 512 == 0 && d->latent % 512 == 0 && d->inter % 512 == 0 && d->shared_inter % 512 == 0;
}

// K slices of a split-K projection: about 7 row steps of 256 bytes per slice
int slices(int K, int bytes_per_weight) {
  const int steps = K * bytes_per_weight / 256;
  int sp = steps / 7;
  return sp < 1 ? 1 : (sp > 32 ? 32 : sp);
}

int check_dims(const moe_latent_dims* d, int topk) {
  if (!d) return MOE_EINVAL;
  if (d->struct_size != sizeof(moe_latent_dims)) return MOE_EABI;
  if (d->T < 0 || d->hidden <= 0 || d->latent <= 0 || d->n_experts <= 0 || d->inter <= 0 || d->shared_inter < 0 ||
      d->align_block < 0 || topk < 1 || topk > d->n_experts)
    return MOE_EINVAL;
  if (!(d->rms_eps >= 0.f) || !(d->routed_scaling_factor == d->routed_scaling_factor)) return MOE_EINVAL;
  if (d->hidden % 256 || d->latent % 256 || d->inter % 256 || d->shared_inter % 256) return MOE_EUNSUPPORTED;
  if (d->n_experts > kMaxExperts || topk > kMaxTopk || d->latent > kMaxLatent) return MOE_EUNSUPPORTED;
  if (d->align_block % 16) return MOE_EUNSUPPORTED;
  if (d->expert_path < MOE_PATH_AUTO || d->expert_path > MOE_PATH_MFMA) return MOE_EINVAL;
  if (d->act_format != MOE_ACT_BF16 && d->act_format != MOE_ACT_MXFP8) return MOE_EINVAL;
  if (d->glu_act != MOE_GLU_SILU && d->glu_act != MOE_GLU_SITU) return MOE_EINVAL;
  if (d->glu_act == MOE_GLU_SITU &&
      !(d->situ_beta > 0.f && d->situ_beta < 3.0e38f && d->situ_linear_beta > 0.f && d->situ_linear_beta < 3.0e38f))
    return MOE_EINVAL;
  if (d->expert_path == MOE_PATH_MFMA && !mfma_sizes_ok(d)) return MOE_EUNSUPPORTED;
  if ((long long)d->T * topk > (1ll << 30)) return MOE_EUNSUPPORTED;
  // activation tensors the kernels index with 32-bit byte offsets stay below 2 GiB
  {
    const long long B = d->align_block ? d->align_block : 16;
    const long long pairs = (long long)d->T * topk;
    const long long cap = B * ((pairs + (pairs < d->n_experts ? pairs : d->n_experts) * (B - 1)) / B);
    const long long lim = 1ll << 31;
    if (cap * d->inter * 2 >= lim || (long long)d->T * d->hidden * 2 >= lim ||
        (long long)d->T * d->shared_inter * 2 >= lim || (long long)d->T * d->latent * 2 >= lim)
      return MOE_EUNSUPPORTED;
    // weight matrices the kernels index with 32-bit byte offsets: the bf16 projections, the
    // fp32 router (and its three bf16 planes), one MXFP4 matrix of an expert or of the shared GLU
    const long long H = d->hidden, L = d->latent, E = d->n_experts;
    if (L * H * 2 >= lim || E * H * 6 >= lim || (long long)d->inter * L / 2 >= lim ||
        (long long)d->shared_inter * H / 2 >= lim)
      return MOE_EUNSUPPORTED;
    // the MFMA path's tiled shared h rounds T up to 16 rows
    const bool mfma = d->expert_path == MOE_PATH_MFMA ||
                      (d->expert_path == MOE_PATH_AUTO && mfma_sizes_ok(d) && pairs >= 12ll * d->n_experts);
    const long long t16 = ((long long)d->T + 15) / 16 * 16;
    if (mfma && t16 * d->shared_inter * 3 / 2 >= lim) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

Plan make_plan(const moe_latent_dims* d, int topk) {
  Plan p;
  p.T = d->T, p.H = d->hidden, p.L = d->latent, p.E = d->n_experts, p.I = d->inter, p.Is = d->shared_inter;
  p.k = topk;
  p.B = d->align_block ? d->align_block : 16;
  p.pairs = p.T * p.k;
  p.cap = moe::align_capacity(p.T, p.k, p.E, p.B);
  p.small = p.T <= 64;
  p.mfma = d->expert_path == MOE_PATH_MFMA ||
           (d->expert_path == MOE_PATH_AUTO && mfma_sizes_ok(d) && (long long)p.pairs >= 12ll * p.E);
  p.fp8 = d->act_format == MOE_ACT_MXFP8;
  p.max_jobs = p.mfma ? moe::mx_max_jobs(p.pairs, p.E, moe::kMfmaSlotsPerJob) : 0;
  p.mid = !p.small && p.T < 2048;
  if (p.small) {
    p.sz = slices(p.H, 2);
    p.sr = slices(p.H, 4);
    p.su = slices(p.L, 2);
  } else if (p.mid) {
    int sp[2];
    // the fp32 router's k-steps cost three MFMAs per fragment (its three bf16 planes): the
    // blocks are balanced on that work (weighting its bytes instead measured slower)
    const int n1[2] = {p.L, p.E}, k1[2] = {p.H, 3 * p.H};
    moe::gemm_split_plan(p.T, 2, n1, k1, kNumCu, sp);
    p.sz = sp[0], p.sr = sp[1];
    const int n2[1] = {p.H}, k2[1] = {p.L};
    moe::gemm_split_plan(p.T, 1, n2, k2, kNumCu, sp);
    p.su = sp[0];
  } else {
    p.sz = p.su = 1;
    const int n1[2] = {p.L, p.E}, k1[2] = {p.H, 3 * p.H};
    p.sr = moe::gemm_large_split(p.T, n1, k1, kNumCu);
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  p.z = take((size_t)p.T * p.L * 2);
  p.z8 = take(p.fp8 && !p.mfma ? (size_t)p.T * p.L * 2 : 0);  // stream: the MXFP8 values of z, bf16
  p.logits = take((size_t)p.T * p.E * 4);
  p.ids = take((size_t)p.pairs * 4);
  p.w = take((size_t)p.pairs * 4);
  p.counts = take((size_t)p.E * 4);
  p.sorted = take((size_t)p.cap * 4);
  p.expert_ids = take((size_t)(p.cap / p.B) * 4);
  p.num_post = take(4);
  p.inv_pos = take((size_t)p.pairs * 4);
  p.align_scratch = take(moe::align_scratch_bytes(p.T, p.E));
  p.h = take(p.mfma ? 0 : (size_t)p.pairs * p.I * 2);  // stream: one row per (token, slot)
  // stream: one row per (token, slot); MFMA: by layout position (a job's rows contiguous)
  p.O = take((size_t)(p.mfma ? p.cap : p.pairs) * p.L * 4);
  p.cn = take((size_t)p.T * p.L * 2);
  p.hs = take(p.mfma ? 0 : (size_t)p.T * p.Is * 2);
  p.ys = take((size_t)p.T * p.H * 4);
  // split-K partial planes (the GEMV always; the GEMM only for segments it splits)
  auto planes = [&](int sl) { return p.small || sl > 1 ? (size_t)sl * p.T : (size_t)0; };
  p.z_part = take(planes(p.sz) * p.L * 4);
  p.r_part = take(planes(p.sr) * p.E * 4);
  p.y_part = take(planes(p.su) * p.H * 4);
  p.cf = take(p.small ? (size_t)p.T * p.L * 4 : 0);
  p.psq = take(p.small ? (size_t)p.T * (p.L / 256) * 4 : 0);
  // FP6 sizes (MXFP8 rows are smaller); h and the shared h are tiled (a multiple of 16 rows)
  const size_t tq = p.mfma ? (size_t)p.T : 0, cq = p.mfma ? (size_t)p.cap : 0, tq16 = (tq + 15) / 16 * 16;
  p.zq = take(tq * p.L * 3 / 2);
  p.zqs = take(tq * p.L / 16);
  p.xq = take(p.Is ? tq * p.H * 3 / 2 : 0);
  p.xqs = take(p.Is ? tq * p.H / 16 : 0);
  p.hq = take(cq * p.I * 3 / 2);
  p.hqs = take(cq * p.I / 16);
  p.hsq = take(tq16 * p.Is * 3 / 2);
  p.hsqs = take(tq * p.Is / 16);
  p.jobs = take((size_t)p.max_jobs * 16);
  p.n_jobs = take(p.mfma ? 4 : 0);
  p.wr3 = take(p.small || p.mid ? 0 : (size_t)p.E * 3 * p.H * 2);  // the router's bf16 planes (T >= 2048)
  p.total = o;
  return p;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const char *x = (const char*)a, *y = (const char*)b;
  return x < y + nb && y < x + na;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// Every buffer the forward writes (y, the workspace, each tap) must overlap no buffer it
// reads and no other buffer it writes. Inputs may overlap one another (they are only read).
bool check_alias(const moe_latent_dims* d, const Plan& p, const void* x, const void* down, const void* norm,
                 const moe_router* router, const uint8_t* packed, const uint8_t* scales, const void* up,
                 const moe_shared* shared, const void* y, const void* workspace, const moe_latent_taps* taps) {
  struct Range {
    const void* p;
    size_t n;
  };
  const size_t T = p.T, H = p.H, L = p.L, E = p.E, I = p.I, Is = p.Is;
  const size_t rec = 3 * I * L / 2, srec = 3 * I * L / 32;
  const Range in[] = {
      {x, T * H * 2},
      {down, L * H * 2},
      {norm, L * 2},
      {router->weight, E * H * 4},
      {router->select_bias, E * 4},
      {packed, E * rec},
      {scales, E * srec},
      {up, H * L * 2},
      {shared ? shared->packed : nullptr, 3 * Is * H / 2},
      {shared ? shared->scales : nullptr, 3 * Is * H / 32},
  };
  std::vector<Range> out = {{y, T * H * 2}, {workspace, p.total}};
  if (taps) {
    const size_t pairs = p.pairs, cap = p.cap;
    out.push_back({taps->z, T * L * 2});
    out.push_back({taps->logits, T * E * 4});
    out.push_back({taps->topk_ids, pairs * 4});
    out.push_back({taps->topk_w, pairs * 4});
    out.push_back({taps->counts, E * 4});
    out.push_back({taps->sorted_ids, cap * 4});
    out.push_back({taps->expert_ids, cap / p.B * 4});
    out.push_back({taps->num_post, 4});
    out.push_back({taps->inv_pos, pairs * 4});
    out.push_back({taps->c, T * L * 4});
    out.push_back({taps->c_norm, T * L * 2});
    out.push_back({taps->y_routed, T * H * 4});
    out.push_back({taps->y_shared, T * H * 4});
    out.push_back({taps->O, pairs * L * 4});
  }
  (void)d;
  for (size_t i = 0; i < out.size(); ++i) {
    for (const Range& r : in)
      if (overlap(out[i].p, out[i].n, r.p, r.n)) return true;
    for (size_t j = i + 1; j < out.size(); ++j)
      if (overlap(out[i].p, out[i].n, out[j].p, out[j].n)) return true;
  }
  return false;
}

int copy_tap(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || !bytes) return MOE_OK;
  MOE_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_latent_abi_version(void) { return MOE_LATENT_ABI_VERSION; }

const char* moe_latent_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer or bad size)";
    case MOE_EUNSUPPORTED: return "sizes not supported by the kernels";
    case MOE_EALIAS: return "an output overlaps an input or the workspace";
    case MOE_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case MOE_EHIP: return "HIP launch failed (see moe_latent_last_hip_error)";
    case MOE_EABI: return "struct_size mismatch (header and library differ)";
    default: return "unknown error";
  }
}

int moe_latent_last_hip_error(void) { return g_last_hip; }

int moe_latent_workspace_size(const moe_latent_dims* d, int topk, size_t* bytes) {
  const int rc = check_dims(d, topk);
  if (rc) return rc;
  if (!bytes) return MOE_EINVAL;
  *bytes = make_plan(d, topk).total;
  return MOE_OK;
}

int moe_latent_align_layout(const moe_latent_dims* d, int topk, int32_t* capacity, int32_t* block) {
  const int rc = check_dims(d, topk);
  if (rc) return rc;
  if (!capacity || !block) return MOE_EINVAL;
  const Plan p = make_plan(d, topk);
  *capacity = p.cap;
  *block = p.B;
  return MOE_OK;
}

}  // extern "C"

namespace {

// The forward of every entry point; with record_stages false it records no stage events
// (the entry point that allocates nothing must not create events either).
// MOE_DUMP_ROUTE=path: append this call's routing to a file (debugging; synchronizes the stream)
void dump_route(const int32_t* ids, const float* w, int T, int k, int E, hipStream_t s) {
  const char* path = std::getenv("MOE_DUMP_ROUTE");
  if (!path || !*path) return;
  const size_t n = (size_t)T * k;
  std::vector<int32_t> hid(n);
  std::vector<float> hw(n);
  if (hipStreamSynchronize(s) != hipSuccess || hipMemcpy(hid.data(), ids, n * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hw.data(), w, n * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return;
  static std::mutex mu;
  std::lock_guard<std::mutex> lk(mu);
  FILE* f = std::fopen(path, "ab");
  if (!f) return;
  const int32_t head[3] = {T, k, E};
  std::fwrite("MOER", 1, 4, f);
  std::fwrite(head, 4, 3, f);
  std::fwrite(hid.data(), 4, n, f);
  std::fwrite(hw.data(), 4, n, f);
  std::fclose(f);
}

int forward_impl(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                 const moe_router* router, const uint8_t* experts_packed, const uint8_t* experts_scales,
                 const void* up, const moe_shared* shared, int topk, void* y, void* workspace, size_t ws_bytes,
                 void* stream, const moe_latent_taps* taps, bool record_stages) {
  int rc = check_dims(d, topk);
  if (rc) return rc;
  if (taps && taps->struct_size != sizeof(moe_latent_taps)) return MOE_EABI;
  if (d->T == 0) return MOE_OK;  // nothing to compute; empty tensors may have null pointers
  if (!x || !down || !router || !router->weight || !experts_packed || !experts_scales || !up || !y)
    return MOE_EINVAL;
  if ((d->shared_inter > 0) != (shared != nullptr)) return MOE_EINVAL;
  if (shared && (!shared->packed || !shared->scales)) return MOE_EINVAL;
  const Plan p = make_plan(d, topk);
  if (!workspace) return MOE_EWORKSPACE;
  if (ws_bytes < p.total || ((uintptr_t)workspace & 255)) return MOE_EWORKSPACE;
  if (check_alias(d, p, x, down, norm, router, experts_packed, experts_scales, up, shared, y, workspace, taps))
    return MOE_EALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* z = at<uint16_t>(ws, p.z);
  float* logits = at<float>(ws, p.logits);
  int32_t* ids = at<int32_t>(ws, p.ids);
  float* w = at<float>(ws, p.w);
  int32_t* counts = at<int32_t>(ws, p.counts);
  int32_t* sorted = at<int32_t>(ws, p.sorted);
  int32_t* expert_ids = at<int32_t>(ws, p.expert_ids);
  int32_t* num_post = at<int32_t>(ws, p.num_post);
  int32_t* inv_pos = at<int32_t>(ws, p.inv_pos);
  uint16_t* h = at<uint16_t>(ws, p.h);
  float* O = at<float>(ws, p.O);
  uint16_t* cn = at<uint16_t>(ws, p.cn);
  uint16_t* hs = at<uint16_t>(ws, p.hs);
  float* ys = at<float>(ws, p.ys);
  // the shared experts' output in bf16 where its one consumer is the up-projection's 256 x 224
  // tile (MFMA path, no K split of the up-projection): half the bytes written and read again
  const bool ys16 = shared && p.mfma && !p.small && p.su == 1;

  // Stage events: the record is claimed here and marked complete after the last stage
  // event; a forward that fails on the way leaves an incomplete record, which
  // moe_latent_timing_read skips.
  hipEvent_t* ev = nullptr;
  int ev_idx = -1;
  if (record_stages) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.on) ev = g_timing.claim(&ev_idx);
  }
  auto mark = [&](int i) -> int {
    if (ev) MOE_HIP(hipEventRecord(ev[i], s));
    return MOE_OK;
  };
#define STAGE_MARK(i)          \
  do {                         \
    int r_ = mark(i);          \
    if (r_) return r_;         \
  } while (0)

  STAGE_MARK(0);
  // a1: down-projection and router logits in one launch
  if (p.small) {
    moe::GemvArgs g{};
    g.A = (const uint16_t*)x;
    g.lda = p.H;
    g.M = p.T;
    g.K = p.H;
    g.nseg = 2;
    g.seg[0] = {down, p.L, 0, p.sz, at<float>(ws, p.z_part)};
    g.seg[1] = {router->weight, p.E, 1, p.sr, at<float>(ws, p.r_part)};
    MOE_HIP(moe::launch_dense_gemv(g, s));
  } else {
    moe::GemmArgs a{};
    a.A = (const uint16_t*)x;
    a.lda = p.H;
    a.M = p.T;
    a.nseg = 2;
    // segments split over K write fp32 partial planes, summed by the route launch
    a.seg[0] = {(const uint16_t*)down, p.L, p.H, p.H, p.sz > 1 ? moe::kPartF32 : moe::kStoreBf16,
                p.sz > 1 ? (void*)at<float>(ws, p.z_part) : (void*)z, p.L, nullptr, 0, nullptr, 0, p.sz, 0};
    if (p.mid) {  // the 128 x 128 tile splits the fp32 router into bf16 planes as it stages it
      a.seg[1] = {(const uint16_t*)router->weight, p.E, p.H, p.H, p.sr > 1 ? moe::kPartF32 : moe::kStoreF32,
                  p.sr > 1 ? (void*)at<float>(ws, p.r_part) : (void*)logits, p.E, nullptr, 0, nullptr, 0, p.sr, 1};
    } else {  // the 256 x 224 tile reads the router as three bf16 planes [E, 3H]
      uint16_t* wr3 = at<uint16_t>(ws, p.wr3);
      MOE_HIP(moe::launch_split3(router->weight, p.E, p.H, wr3, s));
      a.seg[1] = {wr3, p.E, 3 * p.H, p.H, p.sr > 1 ? moe::kPartF32 : moe::kStoreF32,
                  p.sr > 1 ? (void*)at<float>(ws, p.r_part) : (void*)logits, p.E, nullptr, 0, nullptr, 0, p.sr, 0};
    }
    MOE_HIP(moe::launch_gemm_bf16(a, s));
  }
  STAGE_MARK(1);
  // a2: (finish the split-K sums,) sigmoid, bias, top-k, weights
  {
    moe::RouteArgs r{};
    r.logits = logits;
    const bool rp = p.small || p.sr > 1, zp = p.small || p.sz > 1;
    r.r_part = rp ? at<float>(ws, p.r_part) : nullptr;
    r.sr = rp ? p.sr : 0;
    r.z_part = zp ? at<float>(ws, p.z_part) : nullptr;
    r.sz = p.sz;
    r.L = p.L;
    r.z_out = z;
    r.logits_out = rp ? logits : nullptr;
    r.bias = router->select_bias;
    r.T = p.T;
    r.E = p.E;
    r.k = p.k;
    r.rsf = d->routed_scaling_factor;
    r.ids = ids;
    r.w = w;
    MOE_HIP(moe::launch_route(r, s));
  }
  STAGE_MARK(2);
  // a3: moe_align_block_size
  MOE_HIP(moe::launch_align(ids, p.T, p.k, p.E, p.B, counts, sorted, expert_ids, num_post, inv_pos,
                            at<void>(ws, p.align_scratch), s));
  if (p.mfma)
    MOE_HIP(moe::launch_mx_jobs(counts, p.E, p.B, moe::kMfmaSlotsPerJob, at<int4>(ws, p.jobs),
                                at<int32_t>(ws, p.n_jobs), s));
  STAGE_MARK(3);
  // a4 + a5 (and a10's gate/up): GLU contractions. The shared experts' blocks go
  // first in the same launch, so their long K rows overlap the routed work.
  const bool situ = d->glu_act == MOE_GLU_SITU;
  const GluAct act{situ ? kGluSitu : kGluSilu, d->situ_beta, d->situ_linear_beta, situ ? 1.0f / d->situ_beta : 0.f,
                   situ ? 1.0f / d->situ_linear_beta : 0.f};
  const size_t gu_bytes = (size_t)p.I * p.L / 2, gu_scales = (size_t)p.I * p.L / 32;
  const size_t sgu = (size_t)p.Is * p.H / 2, sgs = (size_t)p.Is * p.H / 32;
  if (p.mfma) {
    // FP6 hi/lo encodings of the contraction inputs
    uint8_t* zq = at<uint8_t>(ws, p.zq);
    uint8_t* zqs = at<uint8_t>(ws, p.zqs);
    uint8_t* xq = at<uint8_t>(ws, p.xq);
    uint8_t* xqs = at<uint8_t>(ws, p.xqs);
    uint8_t* hq = at<uint8_t>(ws, p.hq);
    uint8_t* hqs = at<uint8_t>(ws, p.hqs);
    uint8_t* hsq = at<uint8_t>(ws, p.hsq);
    uint8_t* hsqs = at<uint8_t>(ws, p.hsqs);
    const int4* jobs = at<int4>(ws, p.jobs);
    const int32_t* n_jobs = at<int32_t>(ws, p.n_jobs);
    const int t16 = (p.T + 15) / 16 * 16;  // rows of the tiled shared h
    if (p.fp8)
      MOE_HIP(moe::launch_quant_fp8(z, p.L, p.T, p.L, zq, zqs, s));
    else
      MOE_HIP(moe::launch_quant_fp6(z, p.L, p.T, p.L, zq, zqs, s));
    if (shared) MOE_HIP(moe::launch_quant_fp6((const uint16_t*)x, p.H, p.T, p.H, xq, xqs, s));
    STAGE_MARK(4);
    {
      moe::MfmaArgs m{};
      int n = 0;
      if (shared) {
        moe::MfmaProblem& g = m.p[n++];
        g.Aq = xq;
        g.Aqs = xqs;
        g.a_rows = p.T;
        g.s_rows = p.T;
        g.routed = 0;
        g.M = p.T;
        g.W = shared->packed;
        g.S = shared->scales;
        g.W2 = shared->packed + sgu;
        g.S2 = shared->scales + sgs;
        g.N = p.Is;
        g.K = p.H;
        g.outq = hsq;
        g.outqs = hsqs;
      }
      moe::MfmaProblem& g = m.p[n++];
      g.fp8 = p.fp8;
      g.Aq = zq;
      g.Aqs = zqs;
      g.a_rows = p.T;
      g.s_rows = p.T;
      g.routed = 1;
      g.a_by_pos = 0;
      g.sorted_ids = sorted;
      g.topk = p.k;
      g.jobs = jobs;
      g.n_jobs = n_jobs;
      g.max_jobs = p.max_jobs;
      g.W = experts_packed;
      g.S = experts_scales;
      g.W2 = experts_packed + gu_bytes;
      g.S2 = experts_scales + gu_scales;
      g.w_stride = 3 * gu_bytes;
      g.s_stride = 3 * gu_scales;
      g.N = p.I;
      g.K = p.L;
      g.outq = hq;
      g.outqs = hqs;
      m.nprob = n;
      for (int i = 0; i < n; ++i) m.p[i].act = act;
      MOE_HIP(moe::launch_mx_mfma(m, s));
    }
    STAGE_MARK(5);
    {
      moe::MfmaArgs m{};
      int n = 0;
      if (shared) {
        moe::MfmaProblem& dn = m.p[n++];
        dn.Aq = hsq;
        dn.Aqs = hsqs;
        dn.a_rows = t16;
        dn.s_rows = p.T;
        dn.routed = 0;
        dn.M = p.T;
        dn.W = shared->packed + 2 * sgu;
        dn.S = shared->scales + 2 * sgs;
        dn.N = p.H;
        dn.K = p.Is;
        if (ys16) dn.outh = (uint16_t*)ys; else dn.outf = ys;
        dn.ldo = p.H;
      }
      moe::MfmaProblem& g = m.p[n++];
      g.fp8 = p.fp8;
      g.Aq = hq;
      g.Aqs = hqs;
      g.a_rows = p.cap;
      g.s_rows = p.cap;
      g.routed = 1;
      g.a_by_pos = 1;
      g.sorted_ids = sorted;
      g.topk = p.k;
      g.jobs = jobs;
      g.n_jobs = n_jobs;
      g.max_jobs = p.max_jobs;
      g.W = experts_packed + 2 * gu_bytes;
      g.S = experts_scales + 2 * gu_scales;
      g.w_stride = 3 * gu_bytes;
      g.s_stride = 3 * gu_scales;
      g.N = p.L;
      g.K = p.I;
      if (p.small)
        g.outf = O;
      else  // bf16 rows: the combine reads half the bytes
        g.outh = (uint16_t*)O;
      g.ldo = p.L;
      m.nprob = n;
      MOE_HIP(moe::launch_mx_mfma(m, s));
    }
    STAGE_MARK(6);
  } else {
  const uint16_t* z_in = z;
  if (p.fp8) {  // the MXFP8 values of z; the GLU epilogue rounds h the same way
    uint16_t* z8 = at<uint16_t>(ws, p.z8);
    MOE_HIP(moe::launch_qdq_fp8(z, p.L, p.T, p.L, z8, p.L, s));
    z_in = z8;
  }
  STAGE_MARK(4);
  {
    moe::MxArgs m{};
    int n = 0;
    if (shared) {
      moe::MxProblem& g = m.p[n++];
      g.A = (const uint16_t*)x;
      g.lda = p.H;
      g.routed = 0;
      g.M = p.T;
      g.max_blocks = (p.T + 15) / 16;
      g.W = shared->packed;
      g.S = shared->scales;
      g.W2 = shared->packed + sgu;
      g.S2 = shared->scales + sgs;
      g.N = p.Is;
      g.K = p.H;
      g.out = hs;
      g.ldo = p.Is;
    }
    moe::MxProblem& g = m.p[n++];
    g.A = z_in;
    g.lda = p.L;
    g.routed = 1;
    g.a_row = moe::kRowToken;
    g.out_row = moe::kRowFlat;
    g.sorted_ids = sorted;
    g.expert_ids = expert_ids;
    g.tiles_per_block = p.B / 16;
    g.num_post = num_post;
    g.pairs = p.pairs;
    g.topk = p.k;
    g.max_blocks = p.cap / 16;
    g.W = experts_packed;
    g.S = experts_scales;
    g.W2 = experts_packed + gu_bytes;
    g.S2 = experts_scales + gu_scales;
    g.w_stride = 3 * gu_bytes;
    g.s_stride = 3 * gu_scales;
    g.N = p.I;
    g.K = p.L;
    g.out = h;
    g.ldo = p.I;
    g.out_fp8 = p.fp8;
    m.nprob = n;
    for (int i = 0; i < n; ++i) m.p[i].act = act;
    MOE_HIP(moe::launch_mx_small(m, s));
  }
  STAGE_MARK(5);
  // a6 (and a10's down): plain contractions, shared blocks first
  {
    moe::MxArgs m{};
    int n = 0;
    if (shared) {
      moe::MxProblem& dn = m.p[n++];
      dn.A = hs;
      dn.lda = p.Is;
      dn.routed = 0;
      dn.M = p.T;
      dn.max_blocks = (p.T + 15) / 16;
      dn.W = shared->packed + 2 * sgu;
      dn.S = shared->scales + 2 * sgs;
      dn.N = p.H;
      dn.K = p.Is;
      dn.out = ys;
      dn.ldo = p.H;
    }
    moe::MxProblem& g = m.p[n++];
    g.A = h;
    g.lda = p.I;
    g.routed = 1;
    g.a_row = moe::kRowFlat;
    g.out_row = moe::kRowFlat;
    g.sorted_ids = sorted;
    g.expert_ids = expert_ids;
    g.tiles_per_block = p.B / 16;
    g.num_post = num_post;
    g.pairs = p.pairs;
    g.topk = p.k;
    g.max_blocks = p.cap / 16;
    g.W = experts_packed + 2 * gu_bytes;
    g.S = experts_scales + 2 * gu_scales;
    g.w_stride = 3 * gu_bytes;
    g.s_stride = 3 * gu_scales;
    g.N = p.L;
    g.K = p.I;
    g.out = O;
    g.ldo = p.L;
    m.nprob = n;
    MOE_HIP(moe::launch_mx_small(m, s));
  }
  STAGE_MARK(6);
  }
  // a7 + a8: weighted combine and RMSNorm. Decode batches spread each token over column blocks
  // and leave the norm's 1 / rms factor to the up-projection's output (finish_up).
  float* cf = taps && taps->c ? taps->c : at<float>(ws, p.cf);
  if (p.small)
    MOE_HIP(moe::launch_combine_cols(O, p.L, p.mfma ? inv_pos : nullptr, w, p.T, p.k, (const uint16_t*)norm, cf, cn,
                                     at<float>(ws, p.psq), s));
  else if (p.mfma)
    MOE_HIP(moe::launch_combine_norm_bf16((const uint16_t*)O, p.L, inv_pos, w, p.T, p.k, (const uint16_t*)norm,
                                          d->rms_eps, taps ? taps->c : nullptr, cn, s));
  else
    MOE_HIP(moe::launch_combine_norm(O, p.L, nullptr, w, p.T, p.k, (const uint16_t*)norm, d->rms_eps,
                                     taps ? taps->c : nullptr, cn, s));
  STAGE_MARK(7);
  // a9: up-projection, plus the shared output, rounded to bf16
  if (p.small) {
    moe::GemvArgs g{};
    g.A = cn;
    g.lda = p.L;
    g.M = p.T;
    g.K = p.L;
    g.nseg = 1;
    g.seg[0] = {up, p.H, 0, p.su, at<float>(ws, p.y_part)};
    MOE_HIP(moe::launch_dense_gemv(g, s));
    const moe::RowScale rs{norm ? at<float>(ws, p.psq) : nullptr, p.L / 256, p.L, d->rms_eps};
    MOE_HIP(moe::launch_finish_up(at<float>(ws, p.y_part), p.su, p.T, p.H, shared ? ys : nullptr, (uint16_t*)y,
                                  taps ? taps->y_routed : nullptr, rs, s));
  } else if (p.su > 1) {
    moe::GemmArgs a{};
    a.A = cn;
    a.lda = p.L;
    a.M = p.T;
    a.nseg = 1;
    a.seg[0] = {(const uint16_t*)up, p.H, p.L, p.L, moe::kPartF32, at<float>(ws, p.y_part), p.H, nullptr, 0, nullptr, 0,
                p.su};
    MOE_HIP(moe::launch_gemm_bf16(a, s));
    MOE_HIP(moe::launch_finish_up(at<float>(ws, p.y_part), p.su, p.T, p.H, shared ? ys : nullptr, (uint16_t*)y,
                                  taps ? taps->y_routed : nullptr, moe::RowScale{nullptr, 0, 0, 0.f}, s));
  } else {
    moe::GemmArgs a{};
    a.A = cn;
    a.lda = p.L;
    a.M = p.T;
    a.nseg = 1;
    a.seg[0] = {(const uint16_t*)up, p.H, p.L, p.L, moe::kAddStoreBf16, y, p.H, shared && !ys16 ? ys : nullptr, p.H,
                taps ? taps->y_routed : nullptr, p.H};
    if (shared && ys16) a.seg[0].addend16 = (const uint16_t*)ys;
    MOE_HIP(moe::launch_gemm_bf16(a, s));
  }
  STAGE_MARK(8);
  if (ev) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (ev_idx < (int)g_timing.done.size()) g_timing.done[(size_t)ev_idx] = 1;
  }
  if (record_stages) dump_route(ids, w, p.T, p.k, p.E, s);

  if (taps) {
    int r;
    if ((r = copy_tap(taps->z, z, (size_t)p.T * p.L * 2, s))) return r;
    if ((r = copy_tap(taps->logits, logits, (size_t)p.T * p.E * 4, s))) return r;
    if ((r = copy_tap(taps->topk_ids, ids, (size_t)p.pairs * 4, s))) return r;
    if ((r = copy_tap(taps->topk_w, w, (size_t)p.pairs * 4, s))) return r;
    if ((r = copy_tap(taps->counts, counts, (size_t)p.E * 4, s))) return r;
    if ((r = copy_tap(taps->sorted_ids, sorted, (size_t)p.cap * 4, s))) return r;
    if ((r = copy_tap(taps->expert_ids, expert_ids, (size_t)(p.cap / p.B) * 4, s))) return r;
    if ((r = copy_tap(taps->num_post, num_post, 4, s))) return r;
    if ((r = copy_tap(taps->inv_pos, inv_pos, (size_t)p.pairs * 4, s))) return r;
    if (taps->c_norm && p.small && norm) {  // the up-projection read bf16(g * c): normalise c itself
      MOE_HIP(moe::launch_norm_from_parts(cf, at<float>(ws, p.psq), p.T, p.L, (const uint16_t*)norm, d->rms_eps,
                                          (uint16_t*)taps->c_norm, s));
    } else if ((r = copy_tap(taps->c_norm, cn, (size_t)p.T * p.L * 2, s))) {
      return r;
    }
    if (taps->O) {
      if (p.mfma && !p.small)
        MOE_HIP(moe::launch_gather_rows_bf16((const uint16_t*)O, p.L, inv_pos, p.pairs, taps->O, s));
      else if (p.mfma)
        MOE_HIP(moe::launch_gather_rows_f32(O, p.L, inv_pos, p.pairs, taps->O, s));
      else if ((r = copy_tap(taps->O, O, (size_t)p.pairs * p.L * 4, s)))
        return r;
    }
    if (taps->y_shared) {
      if (shared) {
        if (ys16)
          MOE_HIP(moe::launch_widen_bf16((const uint16_t*)ys, (size_t)p.T * p.H, taps->y_shared, s));
        else if ((r = copy_tap(taps->y_shared, ys, (size_t)p.T * p.H * 4, s)))
          return r;
      } else {
        MOE_HIP(moe::launch_fill_f32(taps->y_shared, (size_t)p.T * p.H, 0.f, s));
      }
    }
  }
  return MOE_OK;
#undef STAGE_MARK
}

// ------------------------------------------------------------------ static scratch
// Workspace of moe_latent_forward_noalloc: one array per GPU in the code object. In host code
// `scratch` names a host-side stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current, and only that
// address is ever passed to kernels.
__device__ __align__(256) uint8_t scratch[MOE_LATENT_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;  // by device id; null until looked up

int static_scratch(void** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_addr.size()) g_scratch_addr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_addr[(size_t)dev]) {
    void* ptr = nullptr;
    MOE_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return MOE_EHIP;
    g_scratch_addr[(size_t)dev] = ptr;
  }
  *out = g_scratch_addr[(size_t)dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_latent_forward_ex(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                          const moe_router* router, const uint8_t* experts_packed,
                          const uint8_t* experts_scales, const void* up, const moe_shared* shared, int topk,
                          void* y, void* workspace, size_t ws_bytes, void* stream, const moe_latent_taps* taps) {
  return forward_impl(d, x, down, norm, router, experts_packed, experts_scales, up, shared, topk, y, workspace,
                      ws_bytes, stream, taps, true);
}

int moe_latent_forward(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                       const moe_router* router, const uint8_t* experts_packed, const uint8_t* experts_scales,
                       const void* up, const moe_shared* shared, int topk, void* y, void* workspace,
                       size_t ws_bytes, void* stream) {
  return forward_impl(d, x, down, norm, router, experts_packed, experts_scales, up, shared, topk, y, workspace,
                      ws_bytes, stream, nullptr, true);
}

int moe_latent_forward_noalloc(const moe_latent_dims* d, const void* x, const void* down, const void* norm,
                               const moe_router* router, const uint8_t* experts_packed,
                               const uint8_t* experts_scales, const void* up, const moe_shared* shared, int topk,
                               void* y, void* stream) {
  const int rc = check_dims(d, topk);
  if (rc) return rc;
  if (make_plan(d, topk).total > (size_t)MOE_LATENT_STATIC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  if (d->T == 0) return MOE_OK;
  void* ws = nullptr;
  const int r = static_scratch(&ws);
  if (r) return r;
  return forward_impl(d, x, down, norm, router, experts_packed, experts_scales, up, shared, topk, y, ws,
                      (size_t)MOE_LATENT_STATIC_SCRATCH_BYTES, stream, nullptr, false);
}

int moe_route(const moe_latent_dims* d, const void* x, const moe_router* router, int topk, int32_t* topk_ids,
              float* topk_w, float* logits, void* stream) {
  const int rc = check_dims(d, topk);
  if (rc) return rc;
  if (d->T == 0) return MOE_OK;
  if (!x || !router || !router->weight || !topk_ids || !topk_w || !logits) return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  moe::DenseArgs a{};
  a.A = (const uint16_t*)x;
  a.lda = d->hidden;
  a.M = d->T;
  a.K = d->hidden;
  a.nseg = 1;
  a.seg[0] = {router->weight, d->n_experts, 1, moe::kStoreF32, logits, d->n_experts, nullptr, 0, nullptr, 0};
  MOE_HIP(moe::launch_dense(a, s));
  moe::RouteArgs r{};
  r.logits = logits;
  r.sr = 0;
  r.bias = router->select_bias;
  r.T = d->T;
  r.E = d->n_experts;
  r.k = topk;
  r.rsf = d->routed_scaling_factor;
  r.ids = topk_ids;
  r.w = topk_w;
  MOE_HIP(moe::launch_route(r, s));
  return MOE_OK;
}

int moe_align_workspace_size(int T, int topk, int n_experts, size_t* bytes) {
  if (T < 0 || topk < 1 || n_experts < 1 || !bytes) return MOE_EINVAL;
  if (n_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  *bytes = moe::align_scratch_bytes(T, n_experts);
  return MOE_OK;
}

int moe_align_block_size(const int32_t* topk_ids, int T, int topk, int n_experts, int block, int32_t* sorted_ids,
                         int32_t* expert_ids, int32_t* num_post, int32_t* inv_pos, int32_t* counts, void* scratch,
                         size_t scratch_bytes, void* stream) {
  if (T < 0 || topk < 1 || n_experts < 1 || block < 1) return MOE_EINVAL;
  if (n_experts > kMaxExperts || (long long)T * topk > (1ll << 30)) return MOE_EUNSUPPORTED;
  if (n_experts > 4096 && topk > 64) return MOE_EUNSUPPORTED;
  if (!sorted_ids || !expert_ids || !num_post || !counts || (T > 0 && (!topk_ids || !inv_pos))) return MOE_EINVAL;
  if (scratch_bytes < moe::align_scratch_bytes(T, n_experts) || (!scratch && scratch_bytes)) return MOE_EWORKSPACE;
  MOE_HIP(moe::launch_align(topk_ids, T, topk, n_experts, block, counts, sorted_ids, expert_ids, num_post, inv_pos,
                            scratch, (hipStream_t)stream));
  return MOE_OK;
}

int moe_mxfp8_round(const void* x, int rows, int K, void* y, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return MOE_EINVAL;
  const size_t bytes = (size_t)rows * K * 2;
  if (x != y && overlap(x, bytes, y, bytes)) return MOE_EALIAS;
  MOE_HIP(moe::launch_qdq_fp8((const uint16_t*)x, K, rows, K, (uint16_t*)y, K, (hipStream_t)stream));
  return MOE_OK;
}

namespace {
int qb_check(const float* scores, const float* bias, int m, int n, int topk, const float* alpha, const int32_t* hist,
             const float* new_bias) {
  if (m < 0 || n < 2 || topk < 1 || topk >= n) return MOE_EINVAL;
  if (n > kMaxQbExperts) return MOE_EUNSUPPORTED;
  if (!hist || (m > 0 && (!scores || !alpha)) || ((uintptr_t)scores & 15)) return MOE_EINVAL;
  const size_t sb = (size_t)m * n * sizeof(float), hb = (size_t)n * moe::kQbBins * sizeof(int32_t);
  const size_t ab = (size_t)m * sizeof(float), bb = bias ? (size_t)n * sizeof(float) : 0;
  const size_t nb = new_bias ? (size_t)n * sizeof(float) : 0;
  if (overlap(hist, hb, scores, sb) || overlap(hist, hb, bias, bb) || overlap(hist, hb, alpha, ab) ||
      overlap(alpha, ab, scores, sb) || overlap(alpha, ab, bias, bb) || overlap(new_bias, nb, scores, sb) ||
      overlap(new_bias, nb, bias, bb) || overlap(new_bias, nb, alpha, ab) || overlap(new_bias, nb, hist, hb))
    return MOE_EALIAS;
  return MOE_OK;
}
}  // namespace

int moe_qb_histogram(const float* scores, const float* bias, int m, int n, int topk, float* alpha, int32_t* hist,
                     void* stream) {
  const int rc = qb_check(scores, bias, m, n, topk, alpha, hist, nullptr);
  if (rc != MOE_OK) return rc;
  MOE_HIP(moe::launch_qb_histogram(scores, bias, m, n, topk, alpha, hist, 0, nullptr, (hipStream_t)stream));
  return MOE_OK;
}

int moe_qb_update(const float* scores, const float* bias, int m, int n, int topk, float* alpha, int32_t* hist,
                  float* new_bias, void* stream) {
  if (m < 1 || !new_bias) return MOE_EINVAL;
  const int rc = qb_check(scores, bias, m, n, topk, alpha, hist, new_bias);
  if (rc != MOE_OK) return rc;
  const long long t = (long long)m * topk / n;
  MOE_HIP(moe::launch_qb_histogram(scores, bias, m, n, topk, alpha, hist, t < 1 ? 1 : t, new_bias,
                                   (hipStream_t)stream));
  return MOE_OK;
}

int moe_qb_target(long long m_total, int n, int topk, long long* q) {
  if (m_total < 1 || n < 2 || topk < 1 || topk >= n || !q) return MOE_EINVAL;
  if (m_total > (1ll << 40)) return MOE_EUNSUPPORTED;
  const long long t = m_total * topk / n;
  *q = t < 1 ? 1 : t;
  return MOE_OK;
}

int moe_qb_bias(const int32_t* hist, int n, long long m_total, int topk, float* new_bias, void* stream) {
  long long q = 0;
  const int rc = moe_qb_target(m_total, n, topk, &q);
  if (rc != MOE_OK) return rc;
  if (n > kMaxQbExperts) return MOE_EUNSUPPORTED;
  if (!hist || !new_bias) return MOE_EINVAL;
  if (overlap(new_bias, (size_t)n * sizeof(float), hist, (size_t)n * moe::kQbBins * sizeof(int32_t)))
    return MOE_EALIAS;
  MOE_HIP(moe::launch_qb_bias(hist, n, q, new_bias, (hipStream_t)stream));
  return MOE_OK;
}

int moe_hbm_read(const void* buf, size_t bytes, uint32_t* checksum, void* stream) {
  if (!checksum || ((uintptr_t)checksum & 3) || bytes % 16 || (bytes && (!buf || ((uintptr_t)buf & 15))))
    return MOE_EINVAL;
  if (overlap(checksum, sizeof(uint32_t), buf, bytes)) return MOE_EALIAS;
  MOE_HIP(moe::launch_hbm_read(buf, bytes, checksum, (hipStream_t)stream));
  return MOE_OK;
}

int moe_latent_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  return MOE_OK;
}

int moe_latent_stage_count(void) { return kNumStages; }

const char* moe_latent_stage_name(int i) { return (i >= 0 && i < kNumStages) ? kStageNames[i] : nullptr; }

int moe_latent_timing_read(float* ms_per_stage, int* n_forwards) {
  if (!ms_per_stage || !n_forwards) return MOE_EINVAL;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (int i = 0; i < kNumStages; ++i) ms_per_stage[i] = 0.f;
  const int n = g_timing.n;
  g_timing.n = 0;  // the record is cleared whatever happens below
  int done = 0, rc = MOE_OK;
  for (int f = 0; f < n && rc == MOE_OK; ++f) {
    if (!g_timing.done[(size_t)f]) continue;  // a forward that returned an error
    hipEvent_t* e = &g_timing.ev[(size_t)f * (kNumStages + 1)];
    hipError_t he = hipEventSynchronize(e[kNumStages]);
    for (int i = 0; i < kNumStages && he == hipSuccess; ++i) {
      float ms = 0.f;
      he = hipEventElapsedTime(&ms, e[i], e[i + 1]);
      ms_per_stage[i] += ms;
    }
    if (he != hipSuccess) rc = hip_fail(he);
    ++done;
  }
  *n_forwards = rc == MOE_OK ? done : 0;
  return rc;
}

int moe_latent_shutdown(void) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = false;
  g_timing.release();
  return MOE_OK;
}

int moe_rmsnorm(const void* x, int rows, int cols, const void* weight, float eps, void* y, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 4 || !(eps >= 0.f)) return MOE_EINVAL;
  if ((long long)rows * cols * 2 >= (1ll << 40)) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !y || ((uintptr_t)x & 7) || ((uintptr_t)y & 7) || ((uintptr_t)weight & 7)) return MOE_EINVAL;
  const size_t bytes = (size_t)rows * cols * 2;
  if (x != y && overlap(x, bytes, y, bytes)) return MOE_EALIAS;
  if (overlap(y, bytes, weight, (size_t)cols * 2)) return MOE_EALIAS;
  MOE_HIP(moe::launch_rmsnorm((const uint16_t*)x, rows, cols, (const uint16_t*)weight, eps, (uint16_t*)y,
                              (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
