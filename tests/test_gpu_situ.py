"""GPU parity of the SiTU GLU activation (MOE_GLU_SITU; marked gpu) against the oracle's
reading of it (oracle.layer.situ, reading R17), in the routed and the shared experts, on
both expert paths. Parity against K3's own SituAndMul is unpinned: the pages do not print
its formula. Same comparison protocol and tolerances as the SiLU layer."""
import numpy as np
import pytest

from tests import layer_inputs as li
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

K3_BETAS = (4.0, 25.0)
SITU = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()


def _H():
    from tests import gpu_harness
    return gpu_harness


CASES = [
    # (name, expert path, betas, x scaled up (saturating both branches), config)
    ("stream_k3_betas", 1, K3_BETAS, False, dict(T=37, hidden=512, latent=512, n_experts=40, topk=6, inter=256,
                                                  shared_inter=256)),
    ("stream_small_betas", 1, (0.75, 1.5), True, dict(T=23, hidden=256, latent=256, n_experts=24, topk=5,
                                                       inter=256, shared_inter=256)),
    ("mfma_k3_betas", 2, K3_BETAS, False, dict(T=96, hidden=1024, latent=1024, n_experts=8, topk=4, inter=1024,
                                                shared_inter=512)),
    ("mfma_small_betas", 2, (0.75, 1.5), True, dict(T=200, hidden=512, latent=1536, n_experts=24, topk=5,
                                                     inter=512, shared_inter=1024)),
]


@pytest.mark.parametrize("name,path,betas,scaled,kw", CASES, ids=[c[0] for c in CASES])
def test_situ_layer_parity(name, path, betas, scaled, kw):
    H = _H()
    c = li.small_config(**kw)
    d = li.build(c)
    if scaled:   # x times 4 (exact in bf16: exponent + 2), so that both limits act
        d["x"] = (d["x"].astype(np.uint32) + np.uint32(0x0100)).astype(np.uint16)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    out = dl.run(d["x"], expert_path=path, glu_act=SITU, situ_betas=betas, with_O=True)
    ref = li.oracle_forward(c, {**d, **dl.host_dense}, align_block=out["B"], activation="situ", situ_betas=betas)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    busiest = [int(e) for e in np.argsort(-out["counts"], kind="stable")[:3]]
    H.expert_outputs_check(out, c, d["x"], d["down"], lambda e: (d["exp_packed"][e], d["exp_scales"][e]), busiest,
                           c.topk, activation="situ", situ_betas=betas)
    # SiTU is not SiLU here: the SiLU oracle is clearly farther from the GPU output
    silu_ref = li.oracle_forward(c, {**d, **dl.host_dense}, align_block=out["B"])
    keep = ~ref["route"]["near_tie"]
    e_situ = np.abs(out["y_routed"][keep] - ref["y_routed"][keep]).max()
    e_silu = np.abs(out["y_routed"][keep] - silu_ref["y_routed"][keep]).max()
    assert e_silu > (4 * e_situ if scaled else e_situ)


@pytest.mark.fullsize
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,sample", [("decode16", list(range(16))), ("prefill8192", [0, 1, 4097, 8191])])
def test_full_size_situ(name, sample):
    """The K3 layer with SiTU (beta 4, linear beta 25) at decode16 (every token) and at
    prefill8192 (the MFMA path, sampled tokens), plus every slot of the two busiest experts."""
    H = _H()
    c = gen.named_config(name)
    dl = H.k3_layer()
    x = gen.make_x(c)
    out = dl.run(x, glu_act=SITU, situ_betas=K3_BETAS, with_O=True)
    ref = li.oracle_forward(c, {"x": x, **dl.host_dense, "shared": gen.make_shared(c)}, experts=dl.oracle_experts(),
                            align_block=out["B"], tokens=sample, activation="situ", situ_betas=K3_BETAS)
    H.compare_layer(out, ref, c.T, c.topk, c.n_experts)
    busiest = [int(e) for e in np.argsort(-out["counts"], kind="stable")[:2]]
    H.expert_outputs_check(out, c, x, dl.host_dense["down"], dl.oracle_experts(), busiest, c.topk,
                           activation="situ", situ_betas=K3_BETAS)
