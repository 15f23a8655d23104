"""libh3attn: packed-sequence DiT self-attention layer (per-head Q/K RMSNorm, RoPE,
valid-length non-causal softmax attention) as hand-written HIP kernels for MI355X.

The public entry points are the C ABI in ``include/h3attn.h``; ``binding`` exposes them
to Python with torch tensors supplying device memory and streams.
"""
from .binding import (H3Error, Rope, Shape, attn_layer, attn_packed, attn_varlen,  # noqa
                      kv_pack, make_rope, qk_rmsnorm_rope, workspace_size)

__all__ = ["H3Error", "Rope", "Shape", "attn_layer", "attn_packed", "attn_varlen", "kv_pack",
           "make_rope", "qk_rmsnorm_rope", "workspace_size"]
