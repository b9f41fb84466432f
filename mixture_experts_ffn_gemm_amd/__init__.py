"""MI355X (gfx950) batched routed-MoE FFN: a C-ABI HIP library (libmoe_ffn.so)
with a thin Python binding.

The library computes router + top-k + CSR bucketing + grouped int8 expert
GEMMs (gate/up + SwiGLU, down) + the ordered combine, as described in the
SharpInference issues #406, #408, #388 and #129.  See include/moe_ffn.h.
"""
from . import binding  # noqa: F401
from .binding import (moe_ffn_combine, moe_ffn_decode, moe_ffn_prefill,  # noqa: F401
                      moe_ffn_quantize, moe_ffn_residual_rmsnorm, moe_ffn_status_str,
                      moe_ffn_weights_create, moe_ffn_weights_destroy, moe_ffn_weights_dims,
                      moe_ffn_workspace_size, status_str)

__all__ = ["binding", "moe_ffn_weights_create", "moe_ffn_weights_destroy", "moe_ffn_weights_dims",
           "moe_ffn_workspace_size", "moe_ffn_prefill", "moe_ffn_decode", "moe_ffn_combine",
           "moe_ffn_quantize", "moe_ffn_residual_rmsnorm", "moe_ffn_status_str", "status_str"]
