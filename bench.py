"""Benchmark: one Stable LatentMoE layer forward per step on one MI355X.

A step is one pass of the whole layer (down-projection + router, top-k, align,
routed MXFP4 gate/up + GLU, routed down, combine + RMSNorm, shared experts,
up-projection) over one batch of seeded synthetic tokens with every input
already resident in HBM. Default workload: one K3 layer at decode batch 16
(hidden 7168, latent 3584, 896 MXFP4 experts with top-16, RMSNorm, 2 shared
experts merged to a 6144-wide MXFP4 GLU). Four seeded token batches rotate so
that consecutive steps touch different experts. Its roofline is HBM bandwidth
on the expert-weight bytes of the gate/up launch.

The default run also times the same layer at an 8192-token prefill (two
rotating batches) and reports it under "prefill", with the MXFP4 MFMA roofline
of its gate/up launch (algorithmic flops over the FP4/FP6 dense MFMA peak),
and at a 256-token decode batch with a uniform router ("decode256"), plus the
MXFP8 mode, the SiTU activation, Quantile Balancing and the measured HBM read ceiling.

Timing: after W warm-up steps, K steps are timed back to back (wall clock between device
synchronisations), then K steps each bracketed by HIP events on the launch stream with a
1 GiB read before each step (outside its events) that evicts the L2 and the 256 MB
last-level cache; `ms_per_step` is the median of those per-step times and `value` = T /
that median. The oracle is timed beside every measured configuration on a bounded token
sample (`cpu_baseline`). `--config stack8x4096` measures the 8-layer stack instead.

Prints one JSON line (rank 0). Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-MoE layer tokens/s; % peak HBM GB/s (decode), % MXFP4 MFMA (prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense MXFP4/MXFP6 MFMA, MI355X
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA (an MXFP8 x MXFP4 product runs at this rate)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_PROFILES = {"decode16": "mx_small_decode16_traffic.md", "prefill8192": "mx_mfma_prefill8192_traffic.md",
                    "qb8192": "qb8192_traffic.md"}


def kernel_source_hash(rel: str) -> str:
    """sha256 (first 16 hex digits) of a kernel source file followed by the library headers it
    includes, directly or through other headers, in name order: a profile record keyed by it
    goes stale when the kernel or any header it compiles with changes."""
    import hashlib
    import re
    csrc = os.path.dirname(os.path.join(ROOT, rel))
    seen, todo = set(), [os.path.basename(rel)]
    while todo:
        name = todo.pop()
        if name in seen or not os.path.exists(os.path.join(csrc, name)):
            continue
        seen.add(name)
        todo += re.findall(r'^#include "([^"]+)"', open(os.path.join(csrc, name)).read(), re.M)
    h = hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read())
    for name in sorted(seen - {os.path.basename(rel)}):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 PMC summary,
    or None when that summary was taken on a different kernel source or workload."""
    if workload not in TRAFFIC_PROFILES:
        return None
    path = os.path.join(ROOT, "profiles", TRAFFIC_PROFILES[workload])
    try:
        line = next(l for l in open(path) if l.startswith("traffic_record:"))
        rec = json.loads(line.split(":", 1)[1])
        key = kernel_source_hash(rec["source"])
    except (OSError, StopIteration, ValueError, KeyError):
        return None
    if rec.get("workload") != workload or key != rec["source_sha256_16"]:
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]


def measured_mfma(workload: str):
    """MFMA busy fraction and engine clock of the prefill gate/up launch from the committed
    rocprofv3 counter summary, or None when it was taken on a different kernel source."""
    if workload != "prefill8192":
        return None
    path = os.path.join(ROOT, "profiles", "mx_mfma_prefill8192_mfma_util.md")
    try:
        line = next(l for l in open(path) if l.startswith("mfma_record:"))
        rec = json.loads(line.split(":", 1)[1])
        key = kernel_source_hash(rec["source"])
    except (OSError, StopIteration, ValueError, KeyError):
        return None
    if key != rec["source_sha256_16"]:
        return None
    return {"mfma_busy": rec["mfma_busy"], "clock_ghz": rec["clock_ghz"]}


def _host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(c, dense, x_bits, n_tokens: int, shared=None):
    """The oracle, as it stands, on the first n_tokens of one batch of config c (host cores):
    routing over the sample, each selected expert decoded once and applied to its rows,
    combine, norm, up-projection and the shared experts. Generating the weights is not timed."""
    from oracle import layer as ol
    from workload import gen
    xs = x_bits[:n_tokens]
    r = ol.route((xs.astype(np.uint32) << 16).view(np.float32).astype(np.float64), dense["router"],
                 dense["select_bias"], c.topk, c.routed_scaling_factor)
    need = sorted(set(r["ids"].reshape(-1).tolist()))
    cache = {e: gen.make_expert(c, 0, e) for e in need}
    shared = gen.make_shared(c, 0) if shared is None else shared
    t0 = time.perf_counter()
    ol.forward(xs, dense["down"], dense["norm"], dense["router"], dense["select_bias"], lambda e: cache[e],
               dense["up"], shared, c.topk, inter=c.inter, shared_inter=c.shared_inter, rms_eps=c.rms_eps,
               rsf=c.routed_scaling_factor, align_block=16)
    dt = time.perf_counter() - t0
    blas = _blas_threads()
    return {"value": round(n_tokens / dt, 4), "unit": "tokens/s", "cores": _host_cores(), "kind": "oracle",
            "sample": f"first {n_tokens} tokens of one {c.name} batch ({len(need)} experts touched), float64 numpy "
                      f"oracle, {dt:.1f} s wall; matmuls on {blas} BLAS threads, MXFP4 decode on one thread"}


def cpu_baseline_qb(s, b, k):
    """The oracle's Quantile Balancing update, as it stands, on the same scores (host cores)."""
    from oracle import qb
    t0 = time.perf_counter()
    qb.qb_bias(s, b, k)
    dt = time.perf_counter() - t0
    return {"value": s.shape[0] / dt, "unit": "tokens/s", "cores": _host_cores(), "kind": "oracle",
            "sample": f"the whole {s.shape[0]}x{s.shape[1]} batch, numpy oracle (sort and bincount, one thread), "
                      f"{dt:.2f} s wall"}


def measure_qb(L, m=8192, n=896, k=16, iters=200, with_cpu=True):
    """Quantile Balancing bias update on the router scores of an m-token batch at the K3
    router shape, scores and bias resident in HBM. A step is one moe_qb_update (thresholds,
    histograms and the new bias); moe_qb_histogram and moe_qb_bias, the two halves used
    when histograms of several batches are summed in between, are timed on their own."""
    import torch
    from workload import gen
    s_host = gen.make_router_scores(m, n, seed=0)
    b_host = gen.make_selection_bias(n, seed=0)
    s0 = torch.from_numpy(s_host).cuda()
    b = torch.from_numpy(b_host).cuda()
    # 12 row-rotated copies (12 x 29 MB, past the 256 MB last-level cache) used in turn, so that
    # every call reads its scores from HBM
    rot = [torch.roll(s0, shifts=37 * i, dims=0).contiguous() for i in range(12)]
    it = [0]

    def nxt():
        it[0] += 1
        return rot[it[0] % len(rot)]
    alpha = torch.empty(m, dtype=torch.float32, device="cuda")
    hist = torch.empty((n, 1000), dtype=torch.int32, device="cuda")
    nb = torch.empty(n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(20):
        L.moe_qb_histogram(nxt(), b, k, alpha, hist, stream=stream)
        L.moe_qb_bias(hist, m, k, nb, stream=stream)
    torch.cuda.synchronize()
    # events on the launch stream around `iters` calls of each entry point
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    for _ in range(iters):
        L.moe_qb_histogram(nxt(), b, k, alpha, hist, stream=stream)
    ev[1].record(stream)
    for _ in range(iters):
        L.moe_qb_bias(hist, m, k, nb, stream=stream)
    ev[2].record(stream)
    for _ in range(iters):
        L.moe_qb_update(nxt(), b, k, alpha, hist, nb, stream=stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    h_ms = ev[0].elapsed_time(ev[1]) / iters
    b_ms = ev[1].elapsed_time(ev[2]) / iters
    step_ms = ev[2].elapsed_time(ev[3]) / iters
    # algorithmic bytes of moe_qb_histogram: the scores once, the bias, alpha and the histograms written once
    h_bytes = m * n * 4 + n * 4 + m * 4 + n * 1000 * 4
    achieved = h_bytes / (h_ms * 1e-3) / 1e9
    rec = {"config": {"workload": f"qb{m}: Quantile Balancing bias update over the router scores of {m} tokens, "
                                  f"{n} experts, top-{k}, 1000-bin histograms", "global_batch": m},
           "value": round(m / (step_ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(step_ms, 5),
           "roofline": {"bound": "hbm", "kernel": "moe_qb_histogram (qb_alpha_kernel + qb_hist_kernel)",
                        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(f"qb{m}") if (n, k) == (896, 16) else None,
                        "bytes_per_launch": h_bytes,
                        "avg_launch_ms": round(h_ms, 5)},
           "bias_ms": round(b_ms, 5)}
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline_qb(s_host, b_host, k)
    return rec


def measure_hbm_read(L, gib=2, iters=10):
    """HBM read bandwidth of the library's streaming-read kernel (moe_hbm_read) over a
    buffer of `gib` GiB (far past the 256 MB last-level cache), non-temporal 16-byte loads."""
    import torch
    n = gib << 30
    buf = torch.empty(n // 4, dtype=torch.int32, device="cuda").fill_(0x5a5a5a5a)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        L.moe_hbm_read(buf, out, stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(iters):
        L.moe_hbm_read(buf, out, stream=stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / iters
    del buf
    return {"gbs": round(n / (ms * 1e-3) / 1e9, 1), "bytes": n, "ms": round(ms, 4),
            "kernel": "hbm_read_kernel (moe_hbm_read)"}


def path_sweep(L, Ts=(128, 256, 512, 768, 1024, 1536, 2048, 3072, 4096), steps=10):
    """The K3 layer with each expert path forced (MOE_PATH_STREAM, MOE_PATH_MFMA) across batch
    sizes, on one resident layer: the measurement behind MOE_PATH_AUTO's threshold."""
    import torch
    from tests.gpu_harness import DeviceLayer, to_dev_bf16
    from workload import gen
    c = gen.named_config("decode16")
    dl = DeviceLayer(c)
    xb = gen.make_x(c, 0, T=2 * max(Ts))
    rows = []
    for T in Ts:
        xs = [to_dev_bf16(xb[i * T:(i + 1) * T]) for i in range(2)]
        y = torch.empty((T, c.hidden), dtype=torch.bfloat16, device="cuda")
        ms = {}
        for path in (1, 2):
            dims = dl.dims(T, expert_path=path)
            ws = torch.empty(L.moe_latent_workspace_size(dims, c.topk), dtype=torch.uint8, device="cuda")

            def step(i):
                L.moe_latent_forward(dims, xs[i % 2], dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales,
                                     dl.up, dl.sh_packed, dl.sh_scales, c.topk, y, ws)
            for i in range(3):
                step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                step(i)
            torch.cuda.synchronize()
            ms["stream" if path == 1 else "mfma"] = round((time.perf_counter() - t0) / steps * 1e3, 3)
            del ws
        auto = "mfma" if uses_mfma_path(c.with_(T=T)) else "stream"
        rows.append({"T": T, "pairs_per_expert": round(T * c.topk / c.n_experts, 2), "layer_ms": ms, "auto": auto})
        log(json.dumps(rows[-1]))
    return {"path_sweep": rows}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode16",
                    help="named workload (decode16, decode256, prefill8192, stack8x4096)")
    ap.add_argument("--cpu-tokens", type=int, default=6,
                    help="tokens of the oracle's timed sample beside each measured configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps back to back only (no cache flush between steps)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the secondary 8192-token prefill measurement of the default run")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the secondary measurements with MXFP8 routed-expert activations")
    ap.add_argument("--no-situ", action="store_true",
                    help="skip the secondary measurements with the SiTU activation")
    ap.add_argument("--no-decode256", action="store_true",
                    help="skip the secondary 256-token decode measurement of the default run")
    ap.add_argument("--no-qb", action="store_true",
                    help="skip the secondary Quantile Balancing measurement of the default run")
    ap.add_argument("--qb-only", action="store_true", help="only the Quantile Balancing measurement")
    ap.add_argument("--path-sweep", action="store_true",
                    help="only the streaming-vs-MFMA expert path sweep over batch sizes")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the steps, run 3 plain device copies of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; runs on more than one GPU are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from latent_moe_expert_amd import layer as L
    from tests.gpu_harness import DeviceLayer, to_dev_bf16
    from workload import gen

    c = gen.named_config(args.config)
    if args.copy_mb:
        src = torch.ones(args.copy_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {args.copy_mb} MiB device copies")
        del src, dst
    if args.path_sweep:
        print(json.dumps(path_sweep(L)), flush=True)
        return
    if args.qb_only:
        print(json.dumps(measure_qb(L, with_cpu=not args.no_cpu_baseline)), flush=True)
        return
    flush = None if args.no_flush else CacheFlush()
    if c.n_layers > 1:
        record = measure_stack(c, args.steps, args.warmup, L, DeviceLayer, to_dev_bf16, flush)
        print(json.dumps(record), flush=True)
        return
    t0 = time.time()
    dl = DeviceLayer(c)
    xs_bits = gen.make_x(c, 0, T=4 * c.T)
    xs = [to_dev_bf16(xs_bits[i * c.T:(i + 1) * c.T]) for i in range(4)]
    log(f"inputs resident in HBM in {time.time() - t0:.1f} s")
    cpu = not args.no_cpu_baseline
    shared_host = gen.make_shared(c, 0) if cpu else None

    record = measure(c, dl, xs, args.steps, args.warmup, L, flush=flush)
    if cpu:
        record["cpu_baseline"] = cpu_baseline(c, dl.host_dense, xs_bits[:c.T], args.cpu_tokens, shared_host)
    if c.name == "decode16":
        # the measured HBM read ceiling beside the vendor peak
        hb = measure_hbm_read(L)
        record["hbm_read_measured"] = hb
        record["roofline"]["frac_of_measured_read"] = round(record["roofline"]["achieved"] / hb["gbs"], 4)
    if c.name == "decode16" and not args.no_mxfp8:
        # the same decode with MXFP8 routed-expert activations (MOE_ACT_MXFP8)
        record["decode_mxfp8"] = measure(c, dl, xs, args.steps, args.warmup, L, summary=True, act_format=1,
                                         flush=flush)
    if c.name == "decode16" and not args.no_situ:
        # the same decode with the SiTU activation (MOE_GLU_SITU)
        record["decode_situ"] = measure(c, dl, xs, args.steps, args.warmup, L, summary=True, flush=flush,
                                        glu_act=1)
    if not args.no_decode256 and c.name == "decode16":
        # the large decode batch: T=256 with the uniform router (nearly every expert touched),
        # same resident experts and projections, its own router weight
        c2 = gen.named_config("decode256")
        router_k3 = dl.router
        dense2 = {**dl.host_dense, "router": gen.make_dense(c2, 0)["router"]}
        dl.router = torch.from_numpy(np.ascontiguousarray(dense2["router"])).cuda()
        x2_bits = gen.make_x(c2, 0, T=4 * c2.T)
        x2 = [to_dev_bf16(x2_bits[i * c2.T:(i + 1) * c2.T]) for i in range(4)]
        record["decode256"] = measure(c2, dl, x2, args.steps, 5, L, summary=True, flush=flush)
        if cpu:
            record["decode256"]["cpu_baseline"] = cpu_baseline(c2, dense2, x2_bits[:c2.T], args.cpu_tokens,
                                                               shared_host)
        dl.router = router_k3
        del x2
    if not args.no_prefill and c.name == "decode16":
        # the 8192-token prefill on the same resident layer (the scaled-MFMA expert path)
        cp = gen.named_config("prefill8192")
        xp_bits = gen.make_x(cp, 0, T=2 * cp.T)
        xp = [to_dev_bf16(xp_bits[i * cp.T:(i + 1) * cp.T]) for i in range(2)]
        record["prefill"] = measure(cp, dl, xp, max(5, args.steps // 2), 2, L, rotate=2, summary=True,
                                    flush=flush)
        if cpu:
            record["prefill"]["cpu_baseline"] = cpu_baseline(cp, dl.host_dense, xp_bits[:cp.T], args.cpu_tokens,
                                                             shared_host)
        if not args.no_situ:
            record["prefill_situ"] = measure(cp, dl, xp, max(5, args.steps // 2), 2, L, rotate=2, summary=True,
                                             flush=flush, glu_act=1)
        # the same prefill with MXFP8 routed-expert activations (MOE_ACT_MXFP8)
        if not args.no_mxfp8:
            record["prefill_mxfp8"] = measure(cp, dl, xp, max(5, args.steps // 2), 2, L, rotate=2,
                                              summary=True, act_format=1, flush=flush)
    if not args.no_qb and c.name == "decode16":
        record["qb"] = measure_qb(L, with_cpu=cpu)
    print(json.dumps(record), flush=True)


class CacheFlush:
    """Evicts the L2 and the 256 MB last-level cache before a timed step by reading a 1 GiB
    buffer with ordinary loads (a sum), outside the step's timed events. A read leaves only
    clean lines behind; a 1 GiB (or 256 MB) write instead left dirty lines whose write-back
    then ran inside the next step and slowed the decode expert launch from 0.434 to 0.57 ms,
    while a 1 GiB read, a 2 ms idle gap and no flush all gave 0.434 ms."""

    def __init__(self, gib: int = 1):
        import torch
        self.buf = torch.ones((gib << 30) // 4, dtype=torch.int32, device="cuda")
        self.acc = torch.zeros((), dtype=torch.int64, device="cuda")

    def __call__(self, stream):
        import torch
        with torch.cuda.stream(stream):
            torch.sum(self.buf, dim=0, dtype=torch.int64, out=self.acc)


def timed_steps(step, steps, stream, flush):
    """Per-step durations (ms) from HIP events recorded on the launch stream around each step,
    with the caches flushed before each one (outside the events); plus the wall time of the
    whole loop, bracketed by device synchronisations."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush(stream)
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def measure_stack(c, steps, warmup, L, DeviceLayer, to_dev_bf16, flush):
    """A stack of c.n_layers layers with distinct seeded weights, all resident in HBM. A step
    runs the T tokens through every layer in turn; layer i+1's input is the weightless
    RMSNorm of layer i's bf16 output (moe_rmsnorm, harness glue between layers)."""
    import torch
    from workload import gen
    t0 = time.time()
    layers = []
    for i in range(c.n_layers):
        layers.append(DeviceLayer(c, layer=i))
        log(f"layer {i} resident in HBM ({time.time() - t0:.1f} s)")
    x0 = to_dev_bf16(gen.make_x(c, 0))
    dims = layers[0].dims(c.T)
    ws = torch.empty(L.moe_latent_workspace_size(dims, c.topk), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((c.T, c.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    stream = torch.cuda.current_stream()

    def run(taps_fn=None):
        x = x0
        for i, dl in enumerate(layers):
            y = ys[i & 1]
            if taps_fn is None:
                L.moe_latent_forward(dims, x, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                                     dl.sh_packed, dl.sh_scales, c.topk, y, ws, stream=stream)
            else:
                L.moe_latent_forward_ex(dims, x, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                                        dl.sh_packed, dl.sh_scales, c.topk, y, ws, taps=taps_fn(i), stream=stream)
                taps_fn(i, y)
            if i + 1 < len(layers):
                L.moe_rmsnorm(y, y, None, eps=c.rms_eps, stream=stream)   # in place: the next layer's input
            x = y

    # untimed pass: every layer's output finite, and each layer's load of its hottest expert
    counts = torch.empty(c.n_experts, dtype=torch.int32, device="cuda")
    per_layer = []

    def taps_fn(i, y=None):
        if y is None:
            return {"counts": counts}
        torch.cuda.synchronize()
        cnt = counts.cpu().numpy()
        finite = bool(torch.isfinite(y.float()).all().item())
        rms = float(y.float().pow(2).mean().sqrt().item())
        per_layer.append({"layer": i, "y_finite": finite, "y_rms": round(rms, 3),
                          "hottest_expert": int(cnt.argmax()), "hottest_load": int(cnt.max()),
                          "hottest_over_mean": round(float(cnt.max()) * c.n_experts / (c.T * c.topk), 2),
                          "experts_touched": int((cnt > 0).sum())})
    run(taps_fn)
    for rec in per_layer:
        log(json.dumps(rec))
    if not all(r["y_finite"] for r in per_layer):
        raise RuntimeError(f"a layer of the stack produced non-finite outputs: {per_layer}")

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    # back to back: the wall time of `steps` whole-stack passes
    t_start = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms, _ = timed_steps(lambda i: run(), steps, stream, flush)
    med = float(np.median(step_ms))
    # stage times (library events; they add small gaps between launches)
    L.moe_latent_timing_enable(True)
    torch.cuda.synchronize()
    for _ in range(max(1, steps // 4)):
        run()
    torch.cuda.synchronize()
    L.moe_latent_timing_enable(False)
    stages, nf = L.moe_latent_timing_read()
    stage_ms = {k: v / max(nf, 1) for k, v in stages.items()}
    pairs = c.T * c.topk
    gu_ms = stage_ms["expert_gate_up"]
    gu_flops = 4.0 * pairs * c.latent * c.inter + 4.0 * c.T * c.hidden * c.shared_inter
    tf = gu_flops / (gu_ms * 1e-3) / 1e12
    # the stack's algorithmic bytes: every touched expert's record once per layer, the shared
    # experts, projections, router, norm weight, x in and y out of every layer
    rec_b = gen.expert_record_bytes(c) + gen.expert_scale_bytes(c)
    sh_b = gen.shared_record_bytes(c) + gen.shared_scale_bytes(c)
    dense_b = 2 * c.latent * c.hidden * 2 + c.n_experts * c.hidden * 4 + c.latent * 2 + 2 * c.T * c.hidden * 2
    stack_bytes = sum(r["experts_touched"] * rec_b + sh_b + dense_b for r in per_layer)
    return {
        "metric": METRIC, "value": round(c.T / (med * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(med, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{c.name}: {c.n_layers} K3 latent-MoE layers with distinct seeded weights, "
                               f"T={c.T} tokens, Zipf({c.zipf_s}) selection bias (amplitude {c.zipf_c}: hottest "
                               f"expert of layer 0 at about 10x the mean load); layer i+1's input is the "
                               f"weightless RMSNorm of layer i's output; one step runs the tokens through all "
                               f"layers; expert contractions on the scaled MFMA with MXFP6 hi/lo activations",
                   "global_batch": c.T, "parallelism": "none (1 GPU)"},
        "timing": {"ms_per_step_median_flushed": round(med, 4), "ms_per_step_mean_flushed":
                   round(float(np.mean(step_ms)), 4), "ms_per_step_back_to_back": round(wall * 1e3 / steps, 4),
                   "flush": flush is not None},
        "roofline": {"bound": "mfma", "kernel": "mx_mfma_kernel<GLU> (per layer: routed + shared gate/up + GLU)",
                     "achieved": round(tf, 1), "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_FP4_PEAK_TFLOPS, 4), "traffic": None, "flops_per_launch": gu_flops,
                     "avg_launch_ms": round(gu_ms, 5)},
        "stack_hbm_frac": round(stack_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stack_algorithmic_bytes": int(stack_bytes),
        "per_layer": per_layer,
        "layer_stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
    }


def uses_mfma_path(c) -> bool:
    """The library's automatic expert-path rule (MOE_PATH_AUTO in include/moe_latent.h)."""
    sizes = all(v % 512 == 0 for v in (c.hidden, c.latent, c.inter, c.shared_inter))
    return sizes and c.T * c.topk >= 12 * c.n_experts


def measure(c, dl, xs, steps, warmup, L, rotate=4, summary=False, act_format=0, flush=None, glu_act=0):
    """Time `steps` forwards of config c over `rotate` resident token batches; returns the
    JSON record (or, with summary, the fields of a secondary measurement). act_format 1:
    MXFP8 activations of the routed experts. The step time is the median of per-step event
    times with the caches flushed before each step; the back-to-back
    wall time of the same number of steps is reported beside it."""
    import torch
    from workload import gen
    dims = dl.dims(c.T, act_format=act_format, glu_act=glu_act)
    ws = torch.empty(L.moe_latent_workspace_size(dims, c.topk), dtype=torch.uint8, device="cuda")
    y = torch.empty((c.T, c.hidden), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        L.moe_latent_forward(dims, xs[i % rotate], dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                             dl.sh_packed, dl.sh_scales, c.topk, y, ws, stream=stream)

    # distinct experts touched by each batch (routing taps, untimed)
    D = []
    for i in range(rotate):
        ids = torch.empty((c.T, c.topk), dtype=torch.int32, device="cuda")
        L.moe_latent_forward_ex(dims, xs[i], dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                                dl.sh_packed, dl.sh_scales, c.topk, y, ws, taps={"topk_ids": ids})
        torch.cuda.synchronize()
        D.append(len(np.unique(ids.cpu().numpy())))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed steps run uninstrumented by the library: an event between two launches on the
    # stream costs a gap of several microseconds on the GPU. Back to back first, then with the
    # caches flushed before each step (events around each step only).
    t_start = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms, _ = timed_steps(step, steps, stream, flush)
    med = float(np.median(step_ms))

    # The same steps again with the library's stage events (HIP events recorded on the
    # launch stream at every stage boundary): per-stage times and the kernel durations of
    # the roofline. They include the event gaps, so they read slightly long.
    L.moe_latent_timing_enable(True)
    torch.cuda.synchronize()
    for i in range(steps):
        if flush is not None:
            flush(stream)
        step(i)
    torch.cuda.synchronize()
    L.moe_latent_timing_enable(False)
    stages, nf = L.moe_latent_timing_read()
    del ws

    ms_per_step = med
    value = c.T / (med * 1e-3)
    stage_ms = {k: v / max(nf, 1) for k, v in stages.items()}
    D_mean = float(np.mean([D[i % rotate] for i in range(steps)]))
    pairs = c.T * c.topk
    gu_ms, dn_ms = stage_ms["expert_gate_up"], stage_ms["expert_down"]
    mfma = uses_mfma_path(c)
    if act_format:
        acts = ("routed-expert activations MXFP8 (E4M3 + E8M0 per 32), shared-expert activations "
                + ("MXFP6 hi/lo" if mfma else "bf16"))
    elif mfma:
        acts = ("activations bf16, encoded for the expert contractions as MXFP6 hi/lo (two E2M3 planes with "
                "their E8M0 scales per 32 values, about 8 significant bits)")
    else:
        acts = "activations bf16"
    glu = "SiTU (beta 4, linear beta 25)" if glu_act else "SiLU(gate)*up"
    workload = (f"{c.name}: one K3 latent-MoE layer, T={c.T} tokens, hidden {c.hidden}, latent {c.latent}, "
                f"{c.n_experts} MXFP4 experts top-{c.topk}, intermediate {c.inter}, RMSNorm={c.norm}, shared GLU "
                f"{c.shared_inter}, GLU activation {glu}; weights MXFP4 (E2M1 + E8M0/32), {acts}, fp32 accumulation")
    timing = {"ms_per_step_median_flushed": round(med, 4), "ms_per_step_mean_flushed": round(float(np.mean(step_ms)), 4),
              "ms_per_step_back_to_back": round(wall * 1e3 / steps, 4), "flush": flush is not None}
    rec_b = gen.expert_record_bytes(c) + gen.expert_scale_bytes(c)
    sh_b = gen.shared_record_bytes(c) + gen.shared_scale_bytes(c) if c.shared_inter else 0
    if mfma:
        # algorithmic flops of the gate/up launch (routed pairs and shared rows, gate and up)
        gu_flops = 4.0 * pairs * c.latent * c.inter + 4.0 * c.T * c.hidden * c.shared_inter
        all_flops = 6.0 * pairs * c.latent * c.inter + 6.0 * c.T * c.hidden * c.shared_inter
        tf = gu_flops / (gu_ms * 1e-3) / 1e12
        peak = MFMA_FP8_PEAK_TFLOPS if act_format else MFMA_FP4_PEAK_TFLOPS
        fmt = ("MXFP8 routed activations (FP8 x FP4 rate), FP6 hi/lo shared" if act_format
               else "FP6 hi/lo activations")
        roofline = {"bound": "mfma", "kernel": "mx_mfma_kernel<GLU> (routed + shared MXFP4 gate/up + GLU, "
                                                f"scaled MFMA, {fmt})",
                    "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tf / peak, 4), "traffic": None if act_format else measured_traffic(c.name),
                    "flops_per_launch": gu_flops, "avg_launch_ms": round(gu_ms, 5)}
        if not act_format:
            cnt = measured_mfma(c.name)
            roofline["counters"] = cnt
            # two MFMAs (hi and lo planes) per algorithmic product: half of the nominal peak is
            # this design's ceiling; at the engine clock measured under this load, less
            roofline["design_ceiling"] = {"two_plane_frac_of_nominal": 0.5}
            if cnt:
                roofline["design_ceiling"]["at_measured_clock"] = round(0.5 * cnt["clock_ghz"] / 2.4, 4)
        # the layer as a whole against the FP4 peak: algorithmic MXFP4 flops of the routed and
        # shared experts over the whole step
        extra = {"expert_kernels_mfma_frac": round(all_flops / ((gu_ms + dn_ms) * 1e-3) / 1e12 / peak, 4),
                 "layer_mfma_frac": round(all_flops / (med * 1e-3) / 1e12 / peak, 4)}
    else:
        gu_per_expert = 2 * (c.inter * c.latent // 2 + c.inter * c.latent // 32)     # w1 + w3, packed + scales
        dn_per_expert = c.latent * c.inter // 2 + c.latent * c.inter // 32
        # algorithmic bytes of one gate/up launch (routed experts and, in the same launch, the
        # shared experts' gate/up): each touched expert's w1|w3 once, the gathered latent rows
        # once per pair, h written once per pair; the shared gate|up once, x once, hs written once
        sh_gu = 2 * (c.shared_inter * c.hidden // 2 + c.shared_inter * c.hidden // 32) if c.shared_inter else 0
        gu_bytes = (D_mean * gu_per_expert + pairs * c.latent * 2 + pairs * c.inter * 2
                    + sh_gu + (c.T * c.hidden * 2 + c.T * c.shared_inter * 2 if c.shared_inter else 0))
        achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
        exp_bytes = D_mean * (gu_per_expert + dn_per_expert) + sh_b
        roofline = {"bound": "hbm", "kernel": "mx_small_kernel<GLU> (routed + shared MXFP4 gate/up + GLU)",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None if act_format else measured_traffic(c.name),
                    "bytes_per_launch": int(gu_bytes), "avg_launch_ms": round(gu_ms, 5)}
        # strict whole-layer version: every byte the layer must move (touched expert records,
        # shared record, projections, router, norm weight, x, y) over the whole step
        layer_bytes = (D_mean * rec_b + sh_b + 2 * c.latent * c.hidden * 2 + c.n_experts * c.hidden * 4
                       + c.latent * 2 + 2 * c.T * c.hidden * 2)
        extra = {"expert_kernels_hbm_frac": round(exp_bytes / ((gu_ms + dn_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "layer_hbm_frac": round(layer_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "layer_algorithmic_bytes": int(layer_bytes)}
    if summary:
        return {"config": {"workload": workload, "global_batch": c.T}, "value": round(value, 2), "unit": "tokens/s",
                "steps": steps, "ms_per_step": round(ms_per_step, 4), "timing": timing, "roofline": roofline,
                **extra, "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()}}
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": c.T, "parallelism": "none (1 GPU)",
                   "distinct_experts_per_step": D_mean},
        "timing": timing,
        "roofline": roofline,
        **extra,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
    }


if __name__ == "__main__":
    main()
