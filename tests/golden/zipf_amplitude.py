"""Writes zipf_amplitude.json: the amplitude c of the stacked-layer workload's Zipf selection
bias b_e = c * rank_e^(-s), found by bisection so that on layer 0 the hottest expert takes
about 10x the mean load T*k/E (reading R13: the workload asks for "a few hot experts take
about 10x the mean load"). Calls the oracle's router only; the inputs come from the seeded
generators. Run: python tests/golden/zipf_amplitude.py"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.layer import route  # noqa: E402
from oracle.numerics import bf16_to_f64  # noqa: E402
from workload import gen  # noqa: E402

TARGET_RATIO = 10.0


def hottest(c, amp):
    cfg = c.with_(zipf_c=amp)
    d = gen.make_dense(cfg, 0)
    r = route(bf16_to_f64(gen.make_x(cfg, 0)), d["router"], d["select_bias"], cfg.topk, cfg.routed_scaling_factor)
    return int(np.bincount(r["ids"].reshape(-1), minlength=cfg.n_experts).max())


def main():
    c = gen.named_config("stack8x4096")
    target = TARGET_RATIO * c.T * c.topk / c.n_experts
    lo, hi = 0.0, 0.5
    assert hottest(c, hi) > target
    for _ in range(20):
        mid = (lo + hi) / 2
        if hottest(c, mid) > target:
            hi = mid
        else:
            lo = mid
    amp = round(hi, 4)
    load = hottest(c, amp)
    out = {"workload": c.name, "zipf_s": c.zipf_s, "zipf_c": amp, "hottest_load_layer0": load,
           "mean_load": c.T * c.topk / c.n_experts, "ratio": round(load * c.n_experts / (c.T * c.topk), 3),
           "target_ratio": TARGET_RATIO}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_amplitude.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
