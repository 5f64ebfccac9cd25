"""8-bit KV cache in the q8_0 block format (test infrastructure).

[GGUF] section 四: llama.cpp's ``--cache-type-k q8_0 --cache-type-v q8_0`` keeps the K/V
cache in 8 bits, 36 -> 19 KB per token over the 9 full layers; section 三's table gives
the q8_0 sizes per context (both pinned through ``oracle.footprint``).  The page names
the format without defining it; this follows llama.cpp's published q8_0 definition:

  * a block holds 32 consecutive values x_0..x_31 and one scale d = max|x_i| / 127,
    stored as fp16;
  * each value is stored as the int8 code q_i = round(x_i / d), rounded half away from
    zero (all codes 0 when d = 0); it reads back as q_i * d.

Readings for this path (the HIP side takes the same ones):
  * blocks run along head_dim: a K or V row of 256 values is 8 blocks;
  * the decisions are taken in fp32, as the published reference does: max|x| and
    d = max|x| / 127 in fp32, the code from round(x * (1/d)) with 1/d and the product in
    fp32, then d rounded to fp16 (nearest even) for storage;
  * K is quantised after RoPE, from the rotated key in fp32 (the oracle rotates in fp64
    and rounds to fp32); V from its bf16 value, which fp32 holds exactly;
  * decode reads back q * d and attends exactly as over a bf16 cache.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import (FULL, bf16_to_f64, cache_slot, decode_rows, layer_params,
                              rope)

Q8_BLOCK = 32


def q8_quantize(x):
    """q8_0 codes and scales of ``x`` [..., n] (n a multiple of 32): returns
    (int8 [..., n], float16 [..., n/32])."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    if n % Q8_BLOCK:
        raise ValueError("q8_0 quantises whole blocks of 32 values")
    xb = x.reshape(x.shape[:-1] + (n // Q8_BLOCK, Q8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)                                   # fp32
    d = (amax / np.float32(127.0)).astype(np.float32)                    # fp32 division
    safe = np.where(d > 0, d, np.float32(1.0))
    inv = np.where(d > 0, np.float32(1.0) / safe, np.float32(0.0)).astype(np.float32)
    y = (xb * inv[..., None]).astype(np.float32)                         # fp32 product
    y64 = y.astype(np.float64)                                           # exact
    q = np.sign(y64) * np.floor(np.abs(y64) + 0.5)                       # half away from zero
    return q.astype(np.int8).reshape(x.shape), d.astype(np.float16)


def q8_dequantize(codes, scales) -> np.ndarray:
    """Values q * d in float64: codes [..., n] int8, scales [..., n/32] float16."""
    c = np.asarray(codes, dtype=np.float64)
    n = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (n // Q8_BLOCK, Q8_BLOCK))
    return (cb * np.asarray(scales, dtype=np.float64)[..., None]).reshape(c.shape)


def kv_append_q8(k_codes, k_scales, v_codes, v_scales, k, v, pos, layer_type):
    """8-bit cache after appending ``n_new`` tokens per sequence.

    Cache: codes [B, cap, 4, 256] int8 and scales [B, cap, 4, 8] float16 for K and for V.
    k/v [B, n_new, 4, 256] bf16 bits (k before RoPE); pos [B] = position of the first new
    token.  Token t of sequence b sits at position p = pos[b] + t; its rotated key and its
    value are quantised and go to ``cache_slot(p)``; tokens are written in order, so on a
    ring a later position replaces an earlier one.  Returns the four new arrays.
    """
    th, rd, _ = layer_params(layer_type)
    kc = np.array(k_codes, dtype=np.int8, copy=True)
    ks = np.array(k_scales, dtype=np.float16, copy=True)
    vc = np.array(v_codes, dtype=np.int8, copy=True)
    vs = np.array(v_scales, dtype=np.float16, copy=True)
    B, n_new = np.asarray(k).shape[:2]
    for b in range(B):
        p = int(pos[b]) + np.arange(n_new)
        kr = rope(bf16_to_f64(k[b]), p, th, rd).astype(np.float32)
        qk, dk = q8_quantize(kr)
        qv, dv = q8_quantize(bf16_to_f64(v[b]).astype(np.float32))
        for t in range(n_new):
            s = cache_slot(int(p[t]), layer_type)
            kc[b, s], ks[b, s] = qk[t], dk[t]
            vc[b, s], vs[b, s] = qv[t], dv[t]
    return kc, ks, vc, vs


def decode_q8(q, gate, k_codes, k_scales, v_codes, v_scales, seq_lens, layer_type) -> np.ndarray:
    """``decode`` against an 8-bit cache: keys and values read back as q * d.
    Returns float64 [B, 16, 256]."""
    kc, ks = np.asarray(k_codes), np.asarray(k_scales)
    vc, vs = np.asarray(v_codes), np.asarray(v_scales)
    return decode_rows(q, gate,
                       lambda b, slots, g: q8_dequantize(kc[b, slots, g], ks[b, slots, g]),
                       lambda b, slots, g: q8_dequantize(vc[b, slots, g], vs[b, slots, g]),
                       kc.shape[2], seq_lens, layer_type)


__all__ = ["Q8_BLOCK", "q8_quantize", "q8_dequantize", "kv_append_q8", "decode_q8", "FULL"]
