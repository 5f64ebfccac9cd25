"""KV-cache byte counts of the hybrid model (test infrastructure).

[F16Q4] section 一: a full-attention layer stores K and V for 4 KV heads of dim 256 in
bf16 per token.  [GGUF] section 三 (KV size table) and section 四 (8-bit KV): only the
9 full layers grow with context, the 27 window layers hold a fixed amount, and the
q8_0 cache format stores 32 values in 34 bytes.
"""
from __future__ import annotations

from .attention import FULL, HEAD_DIM, N_KV_HEADS, N_LAYERS, WINDOW, layer_types


def kv_bytes_full_layer_per_token(n_kv: int = N_KV_HEADS, head_dim: int = HEAD_DIM,
                                  elem_bytes: int = 2) -> int:
    """K and V, every KV head, one token, one layer."""
    return 2 * n_kv * head_dim * elem_bytes


def kv_bytes_sliding_layer(window: int = WINDOW, **kw) -> int:
    """A sliding layer keeps exactly ``window`` tokens whatever the context length."""
    return window * kv_bytes_full_layer_per_token(**kw)


def q8_0_bytes(n_values: int) -> int:
    """q8_0 storage: blocks of 32 values, each block 32 int8 plus one fp16 scale."""
    if n_values % 32:
        raise ValueError("q8_0 stores whole blocks of 32 values")
    return (n_values // 32) * 34


def kv_bytes_model(ctx: int, n_layers: int = N_LAYERS, cache_type: str = "f16") -> int:
    """Total KV bytes of the stack at context ``ctx`` (sliding layers capped at the window)."""
    types = layer_types(n_layers)
    total_values = 0
    for t in types:
        tokens = ctx if t == FULL else min(ctx, WINDOW)
        total_values += tokens * 2 * N_KV_HEADS * HEAD_DIM
    if cache_type == "f16":
        return total_values * 2
    if cache_type == "q8_0":
        return q8_0_bytes(total_values)
    raise ValueError(f"unknown cache type {cache_type!r}")
