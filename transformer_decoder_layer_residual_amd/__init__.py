"""MI355X (gfx950) fused Llama-style decoder layer: prefill and paged decode.

The compute lives in libdl_layer.so (hand-written HIP kernels behind a C ABI,
include/dl_layer.h); ``binding`` marshals torch tensors into those calls and
``inputs`` generates the seeded synthetic workloads.  Importing the package
loads nothing; the library is opened on the first call.
"""
from . import binding  # noqa: F401
from .binding import (DL_BF16, DL_F32, DL_FUSED, DL_UNFUSED, DLError,  # noqa: F401
                      dl_attn_decode_paged, dl_attn_prefill, dl_down_residual,
                      dl_ffn_swiglu, dl_gate_up_silu, dl_layer_decode, dl_layer_prefill,
                      dl_layer_workspace_size, dl_linear, dl_qkv_rope, dl_reshape_and_cache,
                      dl_rmsnorm_residual, dl_rope_table_fill, make_dims, make_weights)

__all__ = [n for n in dir() if n.startswith("dl_") or n.startswith("DL")] + [
    "make_dims", "make_weights", "binding"]
