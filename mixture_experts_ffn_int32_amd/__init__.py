"""MI355X-native (gfx950) fused MoE-FFN experts.

``hyper_mega_moe(x, topk_ids, topk_weights, up_proj_weight, down_proj_weight)``
runs routing -> up-projection + SwiGLU -> down-projection -> weighted combine
on the GPU, with a fused backward, through the C ABI of ``include/hmm.h``
(libhmm.so, hand-written HIP kernels for CDNA4).  Importing the package does not
load the library; the first call does, and raises if it has not been built.
"""

from .moe import (HyperMegaMoEFunction, backward_from_saved, forward_with_saved, hyper_mega_moe,  # noqa: F401
                  quantize_cols_fp8, quantize_cols_group, quantize_cols_mx, quantize_rows_fp8,
                  quantize_rows_group, quantize_rows_mx, route, saved_views)

__all__ = ["hyper_mega_moe", "HyperMegaMoEFunction", "route", "forward_with_saved", "backward_from_saved",
           "saved_views", "quantize_rows_fp8", "quantize_cols_fp8", "quantize_rows_mx", "quantize_cols_mx",
           "quantize_rows_group", "quantize_cols_group"]
