"""dit_attn on MI355X: QK RMSNorm + interleaved RoPE prologue, flash attention
with per-row LSE, and the out/LSE merge of KV chunks, as hand-written HIP
kernels for gfx950 behind a C ABI (libdit_attn.so).

``inputs`` (seeded synthetic workloads) imports without a GPU; the kernel
wrappers (``qk_norm_rope``, ``attn_fwd``, ``attn_fwd_ws``, ``attn_merge``) load the HIP
library on first use and raise if it is missing.
"""
from __future__ import annotations

__all__ = ["qk_norm_rope", "qk_norm_rope_out", "attn_fwd", "attn_fwd_ws", "attn_fwd_workspace_bytes", "attn_merge",
           "attn_fwd_ring_overlap", "attn_fwd_gqa", "attn_fwd_ws_fused_q", "attn_fwd_ws_bsnd", "attn_fwd_ws_merge", "attn_fwd_varlen", "attn_fwd_noalloc", "attn_fwd_launch_form", "bsnd_to_bnsd", "bnsd_to_bsnd",
           "status_string", "version", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
