"""MI355X-native packed full attention for the MiniMax-H3 block.

The product is libh3attn.so (C ABI declared in include/h3attn.h): a fused Q/K
RMSNorm + MM-RoPE prologue, a flash-attention forward kernel and the backward
of both, hand-written HIP for gfx950.  This package holds the build script, the thin
ctypes binding with the same names as the C entry points, and the seeded
synthetic workloads.
"""
from ._binding import (H3AttnError, abi_version, h3attn_forward, h3attn_forward_log2,  # noqa: F401
                       h3attn_qk_prologue, h3attn_qk_prologue_scaled, h3attn_v_transpose, load_library,
                       padded_length, LIB_PATH, h3attn_forward_lse, h3attn_attention_backward,
                       h3attn_qk_prologue_backward, h3attn_k_prologue_table, h3attn_forward_log2_qprologue,
                       h3attn_forward_log2_lse, h3attn_qk_prologue_backward_scaled,
                       h3attn_attention_backward_noalloc, h3attn_kv_prologue, h3attn_kv_prologue_fp8,
                       h3attn_forward_fp8_qprologue)

__all__ = ["h3attn_qk_prologue", "h3attn_forward", "h3attn_qk_prologue_scaled", "h3attn_v_transpose",
           "h3attn_forward_log2", "h3attn_forward_lse", "h3attn_attention_backward",
           "h3attn_qk_prologue_backward", "h3attn_k_prologue_table", "h3attn_forward_log2_qprologue",
           "h3attn_forward_log2_lse", "h3attn_qk_prologue_backward_scaled", "h3attn_attention_backward_noalloc",
           "h3attn_kv_prologue", "h3attn_kv_prologue_fp8", "h3attn_forward_fp8_qprologue",
           "padded_length", "abi_version", "load_library", "H3AttnError"]
