"""GPU check of the streaming-read measurement kernel (moe_hbm_read, marked gpu): the
XOR checksum of a buffer equals the host's XOR of the same bytes, for sizes from one
16-byte chunk to past a full grid-stride sweep, so every chunk is read exactly once."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_moe_expert_amd import _lib
    _lib.load()


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 16, (1 << 20) + 48, 3 * 2048 * 256 * 16 * 8 + 160])
def test_hbm_read_checksum(nbytes):
    from latent_moe_expert_amd import layer as L
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    L.moe_hbm_read(buf, out)
    torch.cuda.synchronize()
    ref = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert np.uint32(out.cpu().numpy().view(np.uint32)[0]) == np.uint32(ref)
