"""Upstream projections of the attention layer in W8A8 FP8 (test infrastructure).

[FP8] sections 二 and 三 (Spark-X2.6-4B-FP8 walkthrough, nxmr.cn/news/148448): the fused
``q_k_v_proj`` runs in W8A8 -- weights stored as FP8 E4M3 with one static symmetric scale
per output channel, input activations quantised to FP8 per token with a dynamic scale --
and ``g_proj`` (the per-head output gate) is left in BF16.  Shapes from the config table
(section 一): hidden 2560, 16 query heads and 4 KV heads of dim 256, so ``q_k_v_proj`` maps
2560 -> 4096 + 1024 + 1024 = 6144 and ``g_proj`` 2560 -> 16.

Readings (the HIP side takes the same ones):
  * FP8 E4M3 is the OCP E4M3FN encoding: 1 sign, 4 exponent (bias 7), 3 mantissa bits,
    subnormals below 2^-6, largest finite 448, no infinity;
  * the per-token scale is s = max|x| / 448 in fp32 (the symmetric range of E4M3), the
    code of x is E4M3FN(x / s) rounded to nearest even with x / s in fp32 (all codes 0
    when s = 0);
  * weights arrive already quantised (codes + per-channel scales): the MSE observer that
    chose them needs calibration data and trained weights, which this path does not have;
  * y = s_token * s_channel * sum_k dec(code_x) dec(code_w); the attention path takes y
    split as q (channels 0..4095 = head h at 256h..), k (4096..5119), v (5120..6143), and
    gate logits = x W_g^T from the bf16 x;
  * no bias terms (the pages list none).
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2560
QKV_OUT = 16 * 256 + 2 * 4 * 256      # 6144
E4M3_MAX = 448.0


def e4m3fn_decode(codes) -> np.ndarray:
    """Float64 values of E4M3FN codes (uint8); the NaN codes 0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def e4m3fn_encode(x) -> np.ndarray:
    """E4M3FN codes of float values, rounded to nearest even; magnitudes that round above
    448 are refused (the quantiser below never produces them)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("E4M3FN has no infinity")
    a = np.abs(x)
    sign = (np.signbit(x)).astype(np.int64) << 7
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    e = np.maximum(e, -6)                                  # subnormals share the 2^-6 exponent
    step = np.ldexp(1.0, e - 3)                            # spacing of codes at that exponent
    q = np.rint(a / step)                                  # nearest, ties to even (exact: a/step has few bits)
    # q in [8, 16] for normals (16 carries into the next exponent), [0, 8] below 2^-6
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q)
    normal = q >= 8
    biased = e + 7
    mant = np.where(normal, q.astype(np.int64) - 8, q.astype(np.int64))
    # the 4-bit exponent field tops out at 15, where mantissa 7 is the NaN code: beyond 448
    if np.any(normal & ((biased > 15) | ((biased == 15) & (mant == 7)))):
        raise ValueError("value rounds beyond the largest finite E4M3FN value (448)")
    code = np.where(normal, (biased << 3) | mant, mant)
    return (sign | code).astype(np.uint8)


def quantize_tokens(x_bits):
    """Per-token FP8 quantisation of bf16 activations [T, K]: returns (codes uint8 [T, K],
    scales float32 [T])."""
    from oracle.attention import bf16_to_f64
    x = bf16_to_f64(x_bits).astype(np.float32)                       # exact
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)             # fp32 division
    safe = np.where(s > 0, s, np.float32(1.0))
    y = np.where(s[:, None] > 0, x / safe[:, None], np.float32(0.0)).astype(np.float32)
    return e4m3fn_encode(y), s


def qkv_proj(x_bits, w_codes, w_scales, wg_bits):
    """Projections of bf16 hidden states x [T, 2560]: returns float64 (q [T,16,256],
    k [T,4,256], v [T,4,256], gate logits [T,16]).  w_codes [6144, 2560] E4M3FN codes,
    w_scales [6144] (float32), wg_bits [16, 2560] bf16."""
    from oracle.attention import bf16_to_f64
    xc, xs = quantize_tokens(x_bits)
    acc = e4m3fn_decode(xc) @ e4m3fn_decode(w_codes).T                # exact products, fp64 sums
    y = acc * xs.astype(np.float64)[:, None] * np.asarray(w_scales, dtype=np.float64)[None, :]
    T = y.shape[0]
    gate = bf16_to_f64(x_bits) @ bf16_to_f64(wg_bits).T
    return (y[:, :4096].reshape(T, 16, 256), y[:, 4096:5120].reshape(T, 4, 256),
            y[:, 5120:].reshape(T, 4, 256), gate)
