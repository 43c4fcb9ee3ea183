"""Python binding of the latent-MoE layer library (argument marshalling only).

Every function has the name of the C entry point it calls; tensors are torch
tensors on the GPU (PyTorch provides device memory and streams only -- every
step of the layer runs in the library's HIP kernels).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import MoeLatentDims, MoeLatentTaps, MoeRouter, MoeShared


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        lib = _lib.load()
        msg = lib.moe_latent_strerror(code).decode()
        extra = f" (hipError {lib.moe_latent_last_hip_error()})" if code == -5 else ""
        super().__init__(f"{fn} -> {_lib.ERRORS.get(code, code)}: {msg}{extra}")
        self.code = code


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MoeError(fn, rc)


def make_dims(T: int, hidden: int, latent: int, n_experts: int, inter: int, shared_inter: int = 0,
              align_block: int = 0, rms_eps: float = 1e-6, routed_scaling_factor: float = 1.0,
              expert_path: int = 0, act_format: int = 0, glu_act: int = 0, situ_beta: float = 4.0,
              situ_linear_beta: float = 25.0) -> MoeLatentDims:
    return MoeLatentDims(ctypes.sizeof(MoeLatentDims), T, hidden, latent, n_experts, inter, shared_inter,
                         align_block, rms_eps, routed_scaling_factor, expert_path, act_format, glu_act, situ_beta,
                         situ_linear_beta)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def moe_latent_workspace_size(dims: MoeLatentDims, topk: int) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_latent_workspace_size", _lib.load().moe_latent_workspace_size(ctypes.byref(dims), topk,
                                                                              ctypes.byref(out)))
    return out.value


def moe_latent_align_layout(dims: MoeLatentDims, topk: int):
    cap, blk = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("moe_latent_align_layout", _lib.load().moe_latent_align_layout(ctypes.byref(dims), topk,
                                                                          ctypes.byref(cap), ctypes.byref(blk)))
    return cap.value, blk.value


def moe_latent_forward_ex(dims: MoeLatentDims, x, down, norm, router_weight, select_bias, experts_packed,
                          experts_scales, up, shared_packed, shared_scales, topk: int, y, workspace,
                          taps: Optional[dict] = None, stream=None) -> None:
    lib = _lib.load()
    router = MoeRouter(_ptr(router_weight, torch.float32, "router"), _ptr(select_bias, torch.float32, "select_bias"))
    shared = None
    if shared_packed is not None:
        shared = MoeShared(_ptr(shared_packed, torch.uint8, "shared_packed"),
                           _ptr(shared_scales, torch.uint8, "shared_scales"))
    tp = None
    if taps is not None:
        tp = MoeLatentTaps(ctypes.sizeof(MoeLatentTaps), *[_ptr(taps.get(n), None, n) for n in _lib.TAP_FIELDS])
    rc = lib.moe_latent_forward_ex(
        ctypes.byref(dims), _ptr(x, _BF16, "x"), _ptr(down, _BF16, "down"), _ptr(norm, _BF16, "norm"),
        ctypes.byref(router), _ptr(experts_packed, torch.uint8, "experts_packed"),
        _ptr(experts_scales, torch.uint8, "experts_scales"), _ptr(up, _BF16, "up"),
        ctypes.byref(shared) if shared is not None else None, topk, _ptr(y, _BF16, "y"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream),
        ctypes.byref(tp) if tp is not None else None)
    _check("moe_latent_forward_ex", rc)


def moe_latent_forward(dims: MoeLatentDims, x, down, norm, router_weight, select_bias, experts_packed,
                       experts_scales, up, shared_packed, shared_scales, topk: int, y, workspace,
                       stream=None) -> None:
    lib = _lib.load()
    router = MoeRouter(_ptr(router_weight, torch.float32, "router"), _ptr(select_bias, torch.float32, "select_bias"))
    shared = None
    if shared_packed is not None:
        shared = MoeShared(_ptr(shared_packed, torch.uint8, "shared_packed"),
                           _ptr(shared_scales, torch.uint8, "shared_scales"))
    rc = lib.moe_latent_forward(
        ctypes.byref(dims), _ptr(x, _BF16, "x"), _ptr(down, _BF16, "down"), _ptr(norm, _BF16, "norm"),
        ctypes.byref(router), _ptr(experts_packed, torch.uint8, "experts_packed"),
        _ptr(experts_scales, torch.uint8, "experts_scales"), _ptr(up, _BF16, "up"),
        ctypes.byref(shared) if shared is not None else None, topk, _ptr(y, _BF16, "y"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check("moe_latent_forward", rc)


def moe_latent_forward_noalloc(dims: MoeLatentDims, x, down, norm, router_weight, select_bias, experts_packed,
                               experts_scales, up, shared_packed, shared_scales, topk: int, y, stream=None) -> None:
    """moe_latent_forward with the library's static per-GPU scratch as its workspace."""
    lib = _lib.load()
    router = MoeRouter(_ptr(router_weight, torch.float32, "router"), _ptr(select_bias, torch.float32, "select_bias"))
    shared = None
    if shared_packed is not None:
        shared = MoeShared(_ptr(shared_packed, torch.uint8, "shared_packed"),
                           _ptr(shared_scales, torch.uint8, "shared_scales"))
    rc = lib.moe_latent_forward_noalloc(
        ctypes.byref(dims), _ptr(x, _BF16, "x"), _ptr(down, _BF16, "down"), _ptr(norm, _BF16, "norm"),
        ctypes.byref(router), _ptr(experts_packed, torch.uint8, "experts_packed"),
        _ptr(experts_scales, torch.uint8, "experts_scales"), _ptr(up, _BF16, "up"),
        ctypes.byref(shared) if shared is not None else None, topk, _ptr(y, _BF16, "y"), _stream(stream))
    _check("moe_latent_forward_noalloc", rc)


def moe_route(dims: MoeLatentDims, x, router_weight, select_bias, topk: int, topk_ids, topk_w, logits,
              stream=None) -> None:
    lib = _lib.load()
    router = MoeRouter(_ptr(router_weight, torch.float32, "router"), _ptr(select_bias, torch.float32, "select_bias"))
    rc = lib.moe_route(ctypes.byref(dims), _ptr(x, _BF16, "x"), ctypes.byref(router), topk,
                       _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
                       _ptr(logits, torch.float32, "logits"), _stream(stream))
    _check("moe_route", rc)


def moe_align_workspace_size(T: int, topk: int, n_experts: int) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_align_workspace_size", _lib.load().moe_align_workspace_size(T, topk, n_experts, ctypes.byref(out)))
    return out.value


def moe_align_block_size(topk_ids, T: int, topk: int, n_experts: int, block: int, sorted_ids, expert_ids, num_post,
                         inv_pos, counts, scratch, stream=None) -> None:
    lib = _lib.load()
    rc = lib.moe_align_block_size(_ptr(topk_ids, torch.int32, "topk_ids"), T, topk, n_experts, block,
                                  _ptr(sorted_ids, torch.int32, "sorted_ids"),
                                  _ptr(expert_ids, torch.int32, "expert_ids"), _ptr(num_post, torch.int32, "num_post"),
                                  _ptr(inv_pos, torch.int32, "inv_pos"), _ptr(counts, torch.int32, "counts"),
                                  _ptr(scratch, torch.uint8, "scratch"), 0 if scratch is None else scratch.numel(),
                                  _stream(stream))
    _check("moe_align_block_size", rc)


def moe_mxfp8_round(x, y, stream=None) -> None:
    """y = MXFP8 value of x (bf16 [rows, K], K % 32 == 0); y may be x."""
    if x.dim() != 2 or tuple(y.shape) != tuple(x.shape):
        raise ValueError("x and y: the same [rows, K] shape")
    rc = _lib.load().moe_mxfp8_round(_ptr(x, _BF16, "x"), x.shape[0], x.shape[1], _ptr(y, _BF16, "y"),
                                     _stream(stream))
    _check("moe_mxfp8_round", rc)


def moe_qb_histogram(scores, bias, topk: int, alpha, hist, stream=None) -> None:
    """alpha [m] and hist [n, 1000] int32 from scores fp32 [m, n] and bias fp32 [n] (or None)."""
    if scores.dim() != 2:
        raise ValueError("scores: [m, n]")
    m, n = scores.shape
    if alpha.numel() != m or tuple(hist.shape) != (n, _lib.QB_BINS):
        raise ValueError("alpha: [m], hist: [n, 1000]")
    if bias is not None and bias.numel() != n:
        raise ValueError("bias: [n]")
    rc = _lib.load().moe_qb_histogram(_ptr(scores, torch.float32, "scores"), _ptr(bias, torch.float32, "bias"), m, n,
                                      topk, _ptr(alpha, torch.float32, "alpha"), _ptr(hist, torch.int32, "hist"),
                                      _stream(stream))
    _check("moe_qb_histogram", rc)


def moe_qb_update(scores, bias, topk: int, alpha, hist, new_bias, stream=None) -> None:
    """moe_qb_histogram and moe_qb_bias of one batch (m_total = m) in one call."""
    if scores.dim() != 2:
        raise ValueError("scores: [m, n]")
    m, n = scores.shape
    if alpha.numel() != m or tuple(hist.shape) != (n, _lib.QB_BINS) or new_bias.numel() != n:
        raise ValueError("alpha: [m], hist: [n, 1000], new_bias: [n]")
    if bias is not None and bias.numel() != n:
        raise ValueError("bias: [n]")
    rc = _lib.load().moe_qb_update(_ptr(scores, torch.float32, "scores"), _ptr(bias, torch.float32, "bias"), m, n,
                                   topk, _ptr(alpha, torch.float32, "alpha"), _ptr(hist, torch.int32, "hist"),
                                   _ptr(new_bias, torch.float32, "new_bias"), _stream(stream))
    _check("moe_qb_update", rc)


def moe_qb_target(m_total: int, n: int, topk: int) -> int:
    q = ctypes.c_longlong(0)
    _check("moe_qb_target", _lib.load().moe_qb_target(m_total, n, topk, ctypes.byref(q)))
    return q.value


def moe_qb_bias(hist, m_total: int, topk: int, new_bias, stream=None) -> None:
    """new_bias [n] from hist [n, 1000] int32 covering m_total tokens."""
    n = hist.shape[0]
    if tuple(hist.shape) != (n, _lib.QB_BINS) or new_bias.numel() != n:
        raise ValueError("hist: [n, 1000], new_bias: [n]")
    rc = _lib.load().moe_qb_bias(_ptr(hist, torch.int32, "hist"), n, m_total, topk,
                                 _ptr(new_bias, torch.float32, "new_bias"), _stream(stream))
    _check("moe_qb_bias", rc)


def moe_hbm_read(buf, checksum, stream=None) -> None:
    """checksum (int32 [1], GPU) = XOR of all dwords of buf (any contiguous GPU tensor, size % 16 == 0)."""
    rc = _lib.load().moe_hbm_read(_ptr(buf, None, "buf"), buf.numel() * buf.element_size(),
                                  _ptr(checksum, torch.int32, "checksum"), _stream(stream))
    _check("moe_hbm_read", rc)


def moe_latent_timing_enable(on: bool) -> None:
    _check("moe_latent_timing_enable", _lib.load().moe_latent_timing_enable(1 if on else 0))


def moe_latent_stage_names() -> list:
    lib = _lib.load()
    return [lib.moe_latent_stage_name(i).decode() for i in range(lib.moe_latent_stage_count())]


def moe_latent_timing_read() -> tuple:
    """Returns ({stage: summed ms}, n_forwards) and clears the record."""
    lib = _lib.load()
    n = lib.moe_latent_stage_count()
    arr = (ctypes.c_float * n)()
    nf = ctypes.c_int(0)
    _check("moe_latent_timing_read", lib.moe_latent_timing_read(arr, ctypes.byref(nf)))
    return dict(zip(moe_latent_stage_names(), list(arr))), nf.value


def moe_latent_shutdown() -> None:
    _check("moe_latent_shutdown", _lib.load().moe_latent_shutdown())


def moe_rmsnorm(x, y, weight=None, eps: float = 1e-6, stream=None) -> None:
    """y = RMSNorm(x) per row (bf16 [rows, cols]); weight bf16 [cols] or None; y may be x."""
    if x.dim() != 2 or tuple(y.shape) != tuple(x.shape):
        raise ValueError("x and y: the same [rows, cols] shape")
    if weight is not None and weight.numel() != x.shape[1]:
        raise ValueError("weight: [cols]")
    rc = _lib.load().moe_rmsnorm(_ptr(x, _BF16, "x"), x.shape[0], x.shape[1], _ptr(weight, _BF16, "weight"), eps,
                                 _ptr(y, _BF16, "y"), _stream(stream))
    _check("moe_rmsnorm", rc)


def read_route_dump(path: str) -> list:
    """Records a forward appended to the file named by MOE_DUMP_ROUTE: one dict per call with
    topk_ids int32 [T, k], topk_w float32 [T, k] and n_experts."""
    import numpy as np
    data = open(path, "rb").read()
    out, o = [], 0
    while o < len(data):
        if data[o:o + 4] != b"MOER":
            raise ValueError(f"{path}: no record at byte {o}")
        T, k, E = (int(v) for v in np.frombuffer(data, dtype="<i4", count=3, offset=o + 4))
        n = T * k
        ids = np.frombuffer(data, dtype="<i4", count=n, offset=o + 16).reshape(T, k)
        w = np.frombuffer(data, dtype="<f4", count=n, offset=o + 16 + 4 * n).reshape(T, k)
        out.append({"topk_ids": ids.copy(), "topk_w": w.copy(), "n_experts": E})
        o += 16 + 8 * n
    return out
