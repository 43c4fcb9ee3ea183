"""MI355X-native Stable LatentMoE layer: a C-ABI HIP library for gfx950 and its binding.

The layer runs entirely in the library's kernels (`libmoe_latent.so`, built
with `python -m latent_moe_expert_amd.build`); importing the binding does not
need a GPU, calling it does.
"""
from ._lib import LIB_PATH, load  # noqa: F401
