"""moe_latent_forward_noalloc, the entry point that allocates nothing (marked gpu).

Its output must equal moe_latent_forward's on the same inputs (same kernels, different
workspace: the library's static per-GPU scratch), on two calls in a row with the second
batch smaller, for a small layer on both expert paths and for the K3 decode layer.
Sizes whose workspace exceeds the static scratch are rejected before anything is
enqueued.
"""
import numpy as np
import pytest

from tests import layer_inputs as li
from workload import gen

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()


def _both(dl, c, x_dev, expert_path=0):
    """y of moe_latent_forward (own workspace) and of moe_latent_forward_noalloc, as bf16 bits."""
    from latent_moe_expert_amd import layer as L
    from tests.gpu_harness import dev_bf16_to_bits
    T = x_dev.shape[0]
    dims = dl.dims(T, expert_path=expert_path)
    ws = torch.empty(L.moe_latent_workspace_size(dims, c.topk), dtype=torch.uint8, device="cuda")
    y_ref = torch.empty((T, c.hidden), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((T, c.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    L.moe_latent_forward(dims, x_dev, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                         dl.sh_packed, dl.sh_scales, c.topk, y_ref, ws)
    L.moe_latent_forward_noalloc(dims, x_dev, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                                 dl.sh_packed, dl.sh_scales, c.topk, y_na)
    torch.cuda.synchronize()
    return dev_bf16_to_bits(y_ref), dev_bf16_to_bits(y_na)


def _check_pair(ref, got, name):
    from tests.gpu_harness import assert_close, bf16_bits_to_f64
    assert_close(name, bf16_bits_to_f64(got), bf16_bits_to_f64(ref))
    assert np.array_equal(got, ref), f"{name}: not bitwise equal to moe_latent_forward"


@pytest.mark.parametrize("path,kw", [
    (1, dict(T=21, hidden=512, latent=256, n_experts=24, topk=4, inter=256, shared_inter=256)),
    (2, dict(T=40, hidden=512, latent=512, n_experts=8, topk=3, inter=512, shared_inter=512)),
], ids=["stream", "mfma"])
def test_noalloc_matches_forward_two_calls(path, kw):
    from tests import gpu_harness as H
    c = li.small_config(**kw)
    d = li.build(c)
    dl = H.DeviceLayer(c, dense={k: d[k] for k in ("down", "up", "norm", "router", "select_bias")},
                       experts=(d["exp_packed"], d["exp_scales"]))
    x = H.to_dev_bf16(d["x"])
    for T in (c.T, c.T // 2 - 1):        # the second call with a smaller batch
        ref, got = _both(dl, c, x[:T].contiguous(), expert_path=path)
        _check_pair(ref, got, f"T={T}")


def test_noalloc_k3_decode_two_calls():
    """The K3 layer (896 MXFP4 experts, shared experts, RMSNorm) at decode batches 16 then 5."""
    from tests import gpu_harness as H
    c = gen.named_config("decode16")
    dl = H.k3_layer()
    x = H.to_dev_bf16(gen.make_x(c, 0))
    for T in (16, 5):
        ref, got = _both(dl, c, x[:T].contiguous())
        _check_pair(ref, got, f"K3 T={T}")


def test_noalloc_rejects_workspace_beyond_scratch():
    """T = 64 at the K3 shape needs a 54 MiB workspace: MOE_EWORKSPACE, nothing written."""
    from latent_moe_expert_amd import _lib
    from latent_moe_expert_amd import layer as L
    from tests import gpu_harness as H
    c = gen.named_config("decode16")
    dl = H.k3_layer()
    dims = dl.dims(64)
    assert L.moe_latent_workspace_size(dims, c.topk) > _lib.STATIC_SCRATCH_BYTES
    x = H.to_dev_bf16(gen.make_x(c, 0, T=64))
    y = torch.zeros((64, c.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.MoeError) as err:
        L.moe_latent_forward_noalloc(dims, x, dl.down, dl.norm, dl.router, dl.bias, dl.packed, dl.scales, dl.up,
                                     dl.sh_packed, dl.sh_scales, c.topk, y)
    assert err.value.code == -4
    torch.cuda.synchronize()
    assert int((y.view(torch.int16) != 0).sum().item()) == 0
