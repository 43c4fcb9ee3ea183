"""CPU oracle for one Stable LatentMoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check (`__graft_entry__.smoke`) and the benchmark's
CPU-baseline leg may import, call or run anything in this package. The product
path (the HIP library and its Python binding) never touches it, and this
package imports nothing from the product path: the two share no code.

What it computes is the plain definition of the layer, evaluated directly in
float64 from exactly upcast inputs (bf16 and MXFP4 values are exact in fp64):

  layer.route        sigmoid router, selection-only bias, top-k, renormalised
                     weights (WASTE "Kimi K3, as released", section "Against
                     the technical report": sigmoid, e_score_correction_bias
                     for selection only, renormalised over the top-k, then
                     routed_scaling_factor; section "Shape": 1 group,
                     routed_scaling_factor 1.0)
  layer.align        moe_align_block_size: per-expert padded token lists
                     (SlimServe quants.md, the note on the alignment fix)
  mxfp4.decode       E2M1 nibbles, low nibble first, times one E8M0 scale
                     2^(e-127) per 32 weights (WASTE page, section "Gate 3
                     repeated on real K3 experts")
  layer.forward      down-projection -> routed GLU experts on the latent ->
                     weighted aggregate -> optional RMSNorm -> up-projection,
                     plus the full-width shared experts (WASTE page, "Port
                     status" table row "latent MoE"; K3 report review,
                     section "Stable LatentMoE")
  mxfp8              MXFP8 activations of the routed experts (E4M3 elements,
                     one E8M0 scale per 32), the deployment numerics of the K3
                     report review (quantization-aware training section);
                     layer.forward(act="mxfp8") uses them
  qb                 Quantile Balancing: the selection bias that matches every
                     expert's target load m*k/n, exactly and from 1000-bin
                     integer histograms (K3 report review, section on Quantile
                     Balancing; readings Q1-Q6 in its docstring)
  brute              a pure-Python scalar twin of the whole layer for tiny
                     sizes, written independently (bit-field decoding, explicit
                     loops) and used only as a cross-check.

Readings where the pages are silent are listed in the module docstrings of
`layer` and `numerics`.

Parity status: every function here is pinned by the CPU tests (pages' facts,
closed forms, invariants, brute force); none is "parity unpinned".
"""
from . import numerics, mxfp4, mxfp8, layer, qb  # noqa: F401
from .layer import forward, route, align, rmsnorm, silu  # noqa: F401
