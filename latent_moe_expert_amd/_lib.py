"""ctypes declarations of libmoe_latent.so (the C ABI in include/moe_latent.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LATENT_LIB names another build of the same library (the CPU tests load a sanitized copy)
LIB_PATH = os.environ.get("MOE_LATENT_LIB") or os.path.join(_HERE, "libmoe_latent.so")

MOE_OK = 0
QB_BINS = 1000
STATIC_SCRATCH_BYTES = 16 << 20   # MOE_LATENT_STATIC_SCRATCH_BYTES
PATH_AUTO, PATH_STREAM, PATH_MFMA = 0, 1, 2
ACT_BF16, ACT_MXFP8 = 0, 1
GLU_SILU, GLU_SITU = 0, 1
ERRORS = {-1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EALIAS", -4: "MOE_EWORKSPACE", -5: "MOE_EHIP",
          -6: "MOE_EABI"}


class MoeLatentDims(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("T", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("latent", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("align_block", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("routed_scaling_factor", ctypes.c_float), ("expert_path", ctypes.c_int32),
                ("act_format", ctypes.c_int32), ("glu_act", ctypes.c_int32), ("situ_beta", ctypes.c_float),
                ("situ_linear_beta", ctypes.c_float)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("select_bias", ctypes.c_void_p)]


class MoeShared(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


TAP_FIELDS = ["z", "logits", "topk_ids", "topk_w", "counts", "sorted_ids", "expert_ids", "num_post", "inv_pos",
              "c", "c_norm", "y_routed", "y_shared", "O"]


class MoeLatentTaps(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32)] + [(n, ctypes.c_void_p) for n in TAP_FIELDS]


EXPORTS = ["moe_latent_abi_version", "moe_latent_strerror", "moe_latent_last_hip_error",
           "moe_latent_workspace_size", "moe_latent_align_layout", "moe_latent_forward", "moe_latent_forward_ex",
           "moe_route", "moe_align_workspace_size", "moe_align_block_size", "moe_mxfp8_round",
           "moe_qb_histogram", "moe_qb_update", "moe_qb_target", "moe_qb_bias", "moe_hbm_read",
           "moe_latent_timing_enable",
           "moe_latent_stage_count", "moe_latent_stage_name", "moe_latent_timing_read", "moe_latent_shutdown",
           "moe_rmsnorm", "moe_latent_forward_noalloc"]

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m latent_moe_expert_amd.build` "
                           "(the layer has no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(MoeLatentDims)
    sig = {
        "moe_latent_abi_version": ([], I),
        "moe_latent_strerror": ([I], ctypes.c_char_p),
        "moe_latent_last_hip_error": ([], I),
        "moe_latent_workspace_size": ([D, I, ctypes.POINTER(SZ)], I),
        "moe_latent_align_layout": ([D, I, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)], I),
        "moe_latent_forward": ([D, P, P, P, ctypes.POINTER(MoeRouter), P, P, P, ctypes.POINTER(MoeShared), I, P, P,
                                SZ, P], I),
        "moe_latent_forward_ex": ([D, P, P, P, ctypes.POINTER(MoeRouter), P, P, P, ctypes.POINTER(MoeShared), I, P,
                                   P, SZ, P, ctypes.POINTER(MoeLatentTaps)], I),
        "moe_route": ([D, P, ctypes.POINTER(MoeRouter), I, P, P, P, P], I),
        "moe_align_workspace_size": ([I, I, I, ctypes.POINTER(SZ)], I),
        "moe_align_block_size": ([P, I, I, I, I, P, P, P, P, P, P, SZ, P], I),
        "moe_mxfp8_round": ([P, I, I, P, P], I),
        "moe_qb_histogram": ([P, P, I, I, I, P, P, P], I),
        "moe_qb_update": ([P, P, I, I, I, P, P, P, P], I),
        "moe_qb_target": ([ctypes.c_longlong, I, I, ctypes.POINTER(ctypes.c_longlong)], I),
        "moe_qb_bias": ([P, I, ctypes.c_longlong, I, P, P], I),
        "moe_hbm_read": ([P, SZ, P, P], I),
        "moe_latent_timing_enable": ([I], I),
        "moe_latent_stage_count": ([], I),
        "moe_latent_stage_name": ([I], ctypes.c_char_p),
        "moe_latent_timing_read": ([ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)], I),
        "moe_latent_shutdown": ([], I),
        "moe_rmsnorm": ([P, I, I, P, ctypes.c_float, P, P], I),
        "moe_latent_forward_noalloc": ([D, P, P, P, ctypes.POINTER(MoeRouter), P, P, P, ctypes.POINTER(MoeShared), I,
                                        P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib
