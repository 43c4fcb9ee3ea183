"""The C ABI without a GPU: the library loads, exports every declared symbol, and
every argument check returns its code before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

from latent_moe_expert_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_latent.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe_latent.so is not built (run python -m latent_moe_expert_amd.build)")
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "moe_latent_forward" in names and "moe_align_block_size" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS)


def test_abi_version_and_strerror(lib):
    assert lib.moe_latent_abi_version() == 6
    for code in range(0, -7, -1):
        assert lib.moe_latent_strerror(code)
    assert lib.moe_latent_stage_count() == 8
    assert lib.moe_latent_stage_name(4) == b"expert_gate_up"


def _dims(**kw):
    base = dict(T=16, hidden=7168, latent=3584, n_experts=896, inter=3072, shared_inter=6144, align_block=0,
                rms_eps=1e-6, routed_scaling_factor=1.0, expert_path=0, act_format=0, glu_act=0, situ_beta=4.0,
                situ_linear_beta=25.0)
    base.update(kw)
    d = _lib.MoeLatentDims(ctypes.sizeof(_lib.MoeLatentDims), *[base[f] for f, _ in _lib.MoeLatentDims._fields_[1:]])
    return d


def _ws(lib, d, k=16):
    n = ctypes.c_size_t(0)
    rc = lib.moe_latent_workspace_size(ctypes.byref(d), k, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_and_layout(lib):
    rc, n = _ws(lib, _dims())
    assert rc == 0 and n > 0
    cap, blk = ctypes.c_int32(), ctypes.c_int32()
    assert lib.moe_latent_align_layout(ctypes.byref(_dims()), 16, ctypes.byref(cap), ctypes.byref(blk)) == 0
    # T*k = 256 pairs, at most 256 distinct experts, B = 16: 16 * floor((256 + 256*15) / 16) = 4096
    assert (cap.value, blk.value) == (4096, 16)


@pytest.mark.parametrize("kw,k,code", [
    (dict(hidden=100), 16, -2), (dict(latent=3600), 16, -2), (dict(inter=3200), 16, -2),
    (dict(n_experts=65536, hidden=256), 16, -2), (dict(n_experts=65535, hidden=256), 16, 0),
    (dict(n_experts=5000), 16, 0), (dict(T=200000), 16, -2),
    (dict(align_block=24), 16, -2), (dict(T=-1), 16, -1), (dict(n_experts=8), 9, -1),
    (dict(), 0, -1), (dict(), 65, -2), (dict(rms_eps=-1.0), 16, -1),
    (dict(act_format=2), 16, -1), (dict(act_format=-1), 16, -1),
    (dict(glu_act=2), 16, -1), (dict(glu_act=1), 16, 0), (dict(glu_act=1, situ_beta=0.0), 16, -1),
    (dict(glu_act=1, situ_linear_beta=-25.0), 16, -1), (dict(glu_act=1, situ_beta=float("inf")), 16, -1),
    (dict(glu_act=1, situ_beta=float("nan")), 16, -1), (dict(glu_act=0, situ_beta=0.0), 16, 0),
    # the latent z [T, L] bf16 is indexed with 32-bit byte offsets: T * L * 2 below 2 GiB
    (dict(T=131072, hidden=256, latent=8192, n_experts=1, inter=256, shared_inter=0), 1, -2),
    (dict(T=131071, hidden=256, latent=8192, n_experts=1, inter=256, shared_inter=0), 1, 0),
])
def test_dims_validation(lib, kw, k, code):
    rc, _ = _ws(lib, _dims(**kw), k)
    assert rc == code


def test_struct_size_mismatch(lib):
    d = _dims()
    d.struct_size = 12
    assert _ws(lib, d)[0] == -6


def _forward(lib, d, x=0x10000, y=0x90000000, ws=0x200000000, ws_bytes=None, shared=True, k=16, down=0x1000):
    router = _lib.MoeRouter(0x3000, None)
    sh = _lib.MoeShared(0x5000, 0x6000) if shared else None
    if ws_bytes is None:
        ws_bytes = _ws(lib, d, k)[1]
    return lib.moe_latent_forward(ctypes.byref(d), x, down, None, ctypes.byref(router), 0x7000, 0x8000, 0x9000,
                                  ctypes.byref(sh) if sh is not None else None, k, y, ws, ws_bytes, None)


def test_forward_argument_errors_before_any_launch(lib):
    d = _dims()
    assert _forward(lib, d, x=None) == -1
    assert _forward(lib, d, down=None) == -1
    assert _forward(lib, d, shared=False) == -1            # shared_inter > 0 needs shared experts
    assert _forward(lib, _dims(shared_inter=0), shared=True) == -1
    assert _forward(lib, d, ws=None) == -4
    assert _forward(lib, d, ws_bytes=1024) == -4
    assert _forward(lib, d, ws=0x200000010) == -4           # not 256-byte aligned
    assert _forward(lib, d, y=0x10000 + 64) == -3           # y overlaps x
    n = _ws(lib, d)[1]
    assert _forward(lib, d, y=0x200000000 + n // 2) == -3   # y inside the workspace
    assert _forward(lib, _dims(T=0)) == 0                  # nothing to do, nothing enqueued


# fake device addresses for the alias checks, each range far from the others
_X, _DOWN, _ROUTER, _BIAS, _UP, _SHP, _SHS = 0x10000, 0x1000000, 0x8000000, 0x9000000, 0xa000000, 0x10000000, 0x18000000
_PACKED, _SCALES, _WS, _Y, _TAPS = 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44


def _forward_ex(lib, d, taps, k=16, y=_Y, packed=_PACKED):
    router = _lib.MoeRouter(_ROUTER, _BIAS)
    sh = _lib.MoeShared(_SHP, _SHS)
    tp = _lib.MoeLatentTaps(ctypes.sizeof(_lib.MoeLatentTaps), *[taps.get(n) for n in _lib.TAP_FIELDS])
    return lib.moe_latent_forward_ex(ctypes.byref(d), _X, _DOWN, None, ctypes.byref(router), packed, _SCALES, _UP,
                                     ctypes.byref(sh), k, y, _WS, _ws(lib, d, k)[1], None, ctypes.byref(tp))


def test_forward_alias_checks_cover_weights_and_taps(lib):
    """y, the workspace and every tap may overlap no input and no other output; inputs may
    overlap one another. Without a GPU a call that passes every check fails at its first
    launch (MOE_EHIP), never with MOE_EALIAS."""
    d = _dims(T=4)
    assert _forward_ex(lib, d, {}) == -5
    assert _forward_ex(lib, d, {"z": _TAPS, "O": _TAPS + (1 << 32)}) == -5
    # y on the expert records (E x 17,547,264 bytes from _PACKED on), on the selection bias
    assert _forward_ex(lib, d, {}, y=_PACKED + 5 * 16515072) == -3
    assert _forward_ex(lib, d, {}, y=_BIAS) == -3
    # a tap on an input, on y, on the workspace, on another tap
    assert _forward_ex(lib, d, {"z": _DOWN + 64}) == -3
    assert _forward_ex(lib, d, {"c": _Y + 64}) == -3
    assert _forward_ex(lib, d, {"O": _WS + 4096}) == -3
    assert _forward_ex(lib, d, {"c": _TAPS, "y_shared": _TAPS + 8}) == -3
    # the expert records overlapping the down-projection are only read: no alias
    assert _forward_ex(lib, d, {}, packed=_DOWN) == -5


def test_shutdown_releases_timing(lib):
    assert lib.moe_latent_timing_enable(1) == 0
    assert lib.moe_latent_shutdown() == 0
    arr = (ctypes.c_float * 9)()
    nf = ctypes.c_int(-1)
    assert lib.moe_latent_timing_read(arr, ctypes.byref(nf)) == 0 and nf.value == 0
    assert lib.moe_latent_shutdown() == 0                  # idempotent


def test_rmsnorm_argument_errors(lib):
    P, Q, W = 0x100000, 0x900000, 0x2000000
    assert lib.moe_rmsnorm(P, -1, 64, None, 1e-6, Q, None) == -1
    assert lib.moe_rmsnorm(P, 4, 62, None, 1e-6, Q, None) == -1       # cols not a multiple of 4
    assert lib.moe_rmsnorm(P, 4, 64, None, -1.0, Q, None) == -1       # negative eps
    assert lib.moe_rmsnorm(None, 4, 64, None, 1e-6, Q, None) == -1
    assert lib.moe_rmsnorm(P + 4, 4, 64, None, 1e-6, Q, None) == -1   # not 8-byte aligned
    assert lib.moe_rmsnorm(P, 4, 64, None, 1e-6, P + 128, None) == -3  # partial overlap
    assert lib.moe_rmsnorm(P, 4, 64, Q + 64, 1e-6, Q, None) == -3     # weight inside y
    assert lib.moe_rmsnorm(None, 0, 64, None, 1e-6, None, None) == 0  # nothing to do, nothing enqueued
    assert lib.moe_rmsnorm(P, 4, 64, W, 1e-6, P, None) != -3          # in place is allowed


def test_align_argument_errors(lib):
    n = ctypes.c_size_t()
    assert lib.moe_align_workspace_size(16, 16, 896, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.moe_align_workspace_size(16, 16, 65536, ctypes.byref(n)) == -2
    assert lib.moe_align_workspace_size(16, 16, 65535, ctypes.byref(n)) == 0 and n.value == (65535 + 65535) * 4
    assert lib.moe_align_workspace_size(16, 16, 896, ctypes.byref(n)) == 0
    P = 0x100000
    assert lib.moe_align_block_size(P, 16, 16, 896, 0, P, P, P, P, P, P, n.value, None) == -1
    assert lib.moe_align_block_size(P, 16, 16, 896, 16, None, P, P, P, P, P, n.value, None) == -1
    assert lib.moe_align_block_size(P, 16, 16, 896, 16, P, P, P, P, P, P, 8, None) == -4


def test_timing_read_when_empty(lib):
    assert lib.moe_latent_timing_enable(0) == 0
    arr = (ctypes.c_float * 9)()
    nf = ctypes.c_int(-1)
    assert lib.moe_latent_timing_read(arr, ctypes.byref(nf)) == 0 and nf.value == 0


def test_mxfp8_round_argument_errors(lib):
    P, Q = 0x100000, 0x900000
    assert lib.moe_mxfp8_round(P, -1, 64, Q, None) == -1
    assert lib.moe_mxfp8_round(P, 4, 48, Q, None) == -1      # K not a multiple of 32
    assert lib.moe_mxfp8_round(P, 4, 0, Q, None) == -1
    assert lib.moe_mxfp8_round(None, 4, 64, Q, None) == -1
    assert lib.moe_mxfp8_round(P + 8, 4, 64, Q, None) == -1  # not 16-byte aligned
    assert lib.moe_mxfp8_round(P, 4, 64, P + 64, None) == -3  # partial overlap
    assert lib.moe_mxfp8_round(None, 0, 64, None, None) == 0  # nothing to do, nothing enqueued


def test_forward_rejects_unknown_act_format(lib):
    assert _forward(lib, _dims(act_format=7)) == -1


def test_qb_argument_errors(lib):
    P, Q, R = 0x100000, 0x900000, 0x2000000
    # m, n, topk: topk must be below n, n at least 2 and at most 4096
    assert lib.moe_qb_histogram(P, None, 16, 896, 896, Q, R, None) == -1
    assert lib.moe_qb_histogram(P, None, 16, 1, 1, Q, R, None) == -1
    assert lib.moe_qb_histogram(P, None, -1, 896, 16, Q, R, None) == -1
    assert lib.moe_qb_histogram(P, None, 16, 5000, 16, Q, R, None) == -2
    assert lib.moe_qb_histogram(None, None, 16, 896, 16, Q, R, None) == -1
    assert lib.moe_qb_histogram(P + 4, None, 16, 896, 16, Q, R, None) == -1   # scores not 16-byte aligned
    assert lib.moe_qb_histogram(P, None, 16, 896, 16, Q, None, None) == -1
    assert lib.moe_qb_histogram(P, None, 16, 896, 16, P + 64, R, None) == -3  # alpha inside the scores
    assert lib.moe_qb_histogram(P, None, 16, 896, 16, Q, P + 4096, None) == -3  # hist inside the scores
    assert lib.moe_qb_histogram(P, R + 8, 16, 896, 16, Q, R, None) == -3      # bias inside hist
    S = 0x3000000
    assert lib.moe_qb_update(P, None, 0, 896, 16, Q, R, S, None) == -1         # needs at least one token
    assert lib.moe_qb_update(P, None, 16, 896, 16, Q, R, None, None) == -1
    assert lib.moe_qb_update(P, None, 16, 896, 16, Q, R, R + 64, None) == -3   # new_bias inside hist
    assert lib.moe_qb_update(P, None, 16, 896, 16, Q, R, Q, None) == -3        # new_bias on alpha
    assert lib.moe_qb_bias(R, 896, 0, 16, Q, None) == -1
    assert lib.moe_qb_bias(R, 896, 8192, 896, Q, None) == -1
    assert lib.moe_qb_bias(None, 896, 8192, 16, Q, None) == -1
    assert lib.moe_qb_bias(R, 896, 8192, 16, R + 400, None) == -3


@pytest.mark.parametrize("m,n,k,q", [(8192, 896, 16, 146), (3, 896, 16, 1), (4, 2, 1, 2), (1 << 36, 896, 16,
                                                                                          (1 << 40) // 896)])
def test_qb_target(lib, m, n, k, q):
    out = ctypes.c_longlong(0)
    assert lib.moe_qb_target(m, n, k, ctypes.byref(out)) == 0
    assert out.value == q


def test_hbm_read_argument_errors(lib):
    P, Q = 0x100000, 0x900000
    assert lib.moe_hbm_read(P, 64, None, None) == -1
    assert lib.moe_hbm_read(P, 60, Q, None) == -1          # not a multiple of 16
    assert lib.moe_hbm_read(P + 8, 64, Q, None) == -1      # not 16-byte aligned
    assert lib.moe_hbm_read(None, 64, Q, None) == -1
    assert lib.moe_hbm_read(P, 64, Q + 2, None) == -1      # checksum not 4-byte aligned
    assert lib.moe_hbm_read(P, 64, P + 32, None) == -3     # checksum inside the buffer


def test_auto_path_threshold_at_12_slots_per_expert(lib):
    """MOE_PATH_AUTO switches to the MFMA path (whose workspace adds the MXFP6 activation
    tensors and the job table) at T*k = 12*E: T = 672 for the K3 layer (896 experts, top-16).
    Forcing either path shows which one each T took."""
    for T in (671, 672):
        auto = _ws(lib, _dims(T=T))[1]
        stream = _ws(lib, _dims(T=T, expert_path=1))[1]
        mfma = _ws(lib, _dims(T=T, expert_path=2))[1]
        assert stream != mfma
        assert auto == (stream if T < 672 else mfma), T


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_launch(lib):
    """moe_latent_forward_noalloc: a layer whose workspace exceeds the static scratch
    (16 MiB: the K3 layer at T = 64 needs 54 MiB) returns MOE_EWORKSPACE; T = 0 enqueues
    nothing; argument errors come first."""
    router = _lib.MoeRouter(_ROUTER, None)
    sh = _lib.MoeShared(_SHP, _SHS)
    call = lambda d: lib.moe_latent_forward_noalloc(ctypes.byref(d), _X, _DOWN, None, ctypes.byref(router), _PACKED,
                                                    _SCALES, _UP, ctypes.byref(sh), 16, _Y, None)
    assert _ws(lib, _dims(T=64))[1] > _lib.STATIC_SCRATCH_BYTES >= _ws(lib, _dims(T=16))[1]
    assert call(_dims(T=64)) == -4
    assert call(_dims(T=0)) == 0
    assert call(_dims(n_experts=65536)) == -2
    bad = _dims()
    bad.struct_size = 8
    assert call(bad) == -6
