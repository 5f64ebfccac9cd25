"""Plain fp64 attention for the hybrid sliding/full GQA layer (test infrastructure).

Everything here is the plain definition written out: rotate, score every key against
an explicit boolean visibility matrix, softmax, weight the values, gate.  There is no
tiling, no online softmax and no reordering.  Inputs are bf16 bit patterns (uint16);
they are widened exactly to float64 and every step runs in float64.

Readings of points the pages leave open (the HIP path follows the same ones):
  * key j is visible to query i iff  i - 512 < j <= i  on sliding layers and j <= i on
    full layers (512 keys including the query itself);
  * softmax scale 1/sqrt(head_dim) = 1/16; no soft-capping, sinks or QK-norm (the pages
    mention none);
  * RoPE pairs element m with element m + r/2 inside the rotated slice of width r
    (rotate-half), with inverse frequency theta**(-2m/r); elements at index >= r are
    passed through;
  * Q head h reads KV head h // 4;
  * the gate multiplies each head's attention output by sigmoid(gate logit) before the
    output projection, which lies outside this path;
  * the cache stores post-RoPE keys and raw values, both bf16; a sliding layer stores
    position p in ring slot p mod 512.
"""
from __future__ import annotations

import math

import numpy as np

SLIDING = 0
FULL = 1

# [FP8] section 一 (config table): 16 query heads over 4 KV heads, head_dim 256, 36 layers.
# [HYB] section "配套效率设计" (GQA: 16 Q heads share 4 KV heads).
N_Q_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 256
N_LAYERS = 36
# [HYB] section "滑动窗口 512" (sliding_window 512: each token looks back over 512 tokens).
WINDOW = 512


def layer_type_of(layer: int) -> int:
    """Type of 0-based layer ``layer`` in the 36-layer stack.

    [HYB] section "36 层混合注意力排布": three sliding layers then one full layer,
    repeated 9 times, so the 36th (last) layer is full.  [CFG] section "混合注意力"
    gives the same 3:1 cycle; [F16Q4] section 一 counts 9 full and 27 sliding layers.
    """
    if layer < 0:
        raise ValueError("layer index must be >= 0")
    return FULL if layer % 4 == 3 else SLIDING


def layer_types(n_layers: int = N_LAYERS) -> list:
    return [layer_type_of(i) for i in range(n_layers)]


def layer_params(layer_type: int):
    """(rope_theta, rotary width r, window) of a layer type.

    [HYB] parameter table in section "全局注意力 5M 基频 RoPE" and section
    "滑动窗口 512"; [CFG] section "1M 上下文如何做到": sliding layers use theta 1e4
    over the whole head (partial_rotary_factor 1.0, r = 256) and a 512 window; full
    layers use theta 5e6 on the first quarter of the head (factor 0.25, r = 64) and no
    window.  ``None`` means no window.
    """
    if layer_type == SLIDING:
        return 10000.0, HEAD_DIM, WINDOW
    if layer_type == FULL:
        return 5000000.0, HEAD_DIM // 4, None
    raise ValueError(f"unknown layer type {layer_type!r}")


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head ``h``: consecutive groups of n_q/n_kv query heads.

    [HYB] section "配套效率设计": 16 query heads share 4 KV heads.  Which four share
    which KV head is not stated; contiguous groups (head h -> h // 4) are used.
    """
    return h // (n_q_heads // n_kv_heads)


def softmax_scale(head_dim: int = HEAD_DIM) -> float:
    """1/sqrt(head_dim): the pages give no scale, the standard one is used."""
    return 1.0 / math.sqrt(head_dim)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns uint16 bits.

    Written from the format's definition: 8 significant bits, the float32 exponent
    range, subnormals spaced 2**-133.  Used where the path stores bf16 (the KV cache).
    """
    x = np.asarray(x, dtype=np.float64)
    _, expo = np.frexp(x)                          # |x| = f * 2**expo with 0.5 <= f < 1
    qexp = np.maximum(expo, -125) - 8              # spacing of bf16 values around x
    q = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)  # rint: nearest, ties to even
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rope_inv_freq(theta: float, rot_dim: int) -> np.ndarray:
    """Inverse frequencies theta**(-2m/r), m = 0 .. r/2-1.

    [HYB] section "全局注意力 5M 基频 RoPE" and [CFG] section "1M 上下文如何做到"
    give theta and the rotated fraction per layer type; the exponent's denominator is
    the rotated width r (reading of a silent point).
    """
    m = np.arange(rot_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * m / float(rot_dim))


def rope(x, positions, theta: float, rot_dim: int) -> np.ndarray:
    """Rotary position embedding of ``x`` [n, heads, D] at ``positions`` [n].

    For m < r/2 and angle a = p * theta**(-2m/r):
        y[m]       = x[m] cos a - x[m + r/2] sin a
        y[m + r/2] = x[m + r/2] cos a + x[m] sin a
    and y[d] = x[d] for d >= r.  [HYB] sections "滑动窗口 512" (all 256 dims rotated on
    sliding layers) and "全局注意力 5M 基频 RoPE" (only the first 64 dims rotated on full
    layers, the rest carry no position).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.float64)
    half = rot_dim // 2
    ang = pos[:, None] * rope_inv_freq(theta, rot_dim)[None, :]      # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    y = x.copy()
    x1 = x[..., :half]
    x2 = x[..., half:rot_dim]
    y[..., :half] = x1 * c - x2 * s
    y[..., half:rot_dim] = x2 * c + x1 * s
    return y


def visibility(q_pos, k_pos, window) -> np.ndarray:
    """Explicit boolean matrix: key j visible to query i iff k_j <= q_i and q_i - k_j < W.

    [HYB] section "36 层混合注意力排布": full layers build a causal mask, sliding layers a
    sliding-window causal mask.  ``window=None`` means causal only.
    """
    q = np.asarray(q_pos, dtype=np.int64)[:, None]
    k = np.asarray(k_pos, dtype=np.int64)[None, :]
    vis = k <= q
    if window is not None:
        vis &= (q - k) < int(window)
    return vis


def _attend(qr, kr, v, vis, gate_logit, scale):
    """One head: softmax(q k^T * scale, masked) v, times sigmoid(gate).

    fp32-or-better softmax: [F16Q4] section 三 (softmax taken in fp32 over low-precision
    Q/K/V); here fp64.  Head gate: [F16Q4] section 三 and [HYB] section "配套效率设计"
    (one sigmoid gate per head scales that head's attention output).
    """
    s = (qr @ kr.T) * scale
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    p /= np.sum(p, axis=1, keepdims=True)
    o = p @ v
    g = 1.0 / (1.0 + np.exp(-np.asarray(gate_logit, dtype=np.float64)))
    return o * g[:, None]


def prefill(q, k, v, gate, layer_type, rows=None, *, theta=None, rot_dim=None,
            window="layer", row_block: int = 512) -> np.ndarray:
    """Prefill output at query rows ``rows`` (default: all), positions 0..S-1.

    q [B,S,16,256], k/v [B,S,4,256], gate [B,S,16]: bf16 bit patterns, q and k before
    RoPE.  Returns float64 [B, len(rows), 16, 256].  ``theta``, ``rot_dim`` and
    ``window`` override the layer type's values (used by the oracle's own tests).
    """
    th, rd, w = layer_params(layer_type)
    th = th if theta is None else theta
    rd = rd if rot_dim is None else rot_dim
    w = w if window == "layer" else window
    q = np.asarray(q)
    B, S, H, D = q.shape
    Hk = np.asarray(k).shape[2]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = softmax_scale(D)
    out = np.zeros((B, len(rows), H, D), dtype=np.float64)
    kpos = np.arange(S)
    for b in range(B):
        kr = rope(bf16_to_f64(k[b]), kpos, th, rd)                  # [S, Hk, D]
        vb = bf16_to_f64(v[b])
        for r0 in range(0, len(rows), row_block):
            rr = rows[r0:r0 + row_block]
            nk = int(rr.max()) + 1                                   # keys past the last row are never visible
            vis = visibility(rr, kpos[:nk], w)
            qr = rope(bf16_to_f64(q[b, rr]), rr, th, rd)             # [n, H, D]
            gb = np.asarray(gate)[b, rr]
            for h in range(H):
                g = kv_head_of(h, H, Hk)
                out[b, r0:r0 + len(rr), h] = _attend(
                    qr[:, h], kr[:nk, g], vb[:nk, g], vis, bf16_to_f64(gb[:, h]), scale)
    return out


def prefill_chunk(q, k, v, gate, cache_k, cache_v, start_pos: int, layer_type, rows=None,
                  row_block: int = 512) -> np.ndarray:
    """Prefill of a chunk that continues a cached prefix: output at chunk rows ``rows``.

    The chunk's token t sits at position P + t (P = ``start_pos``, the same for every
    sequence).  Its keys are the cached prefix, read as stored (post-RoPE bf16 keys and
    bf16 values: full layers positions 0..P-1 from slots 0..P-1, sliding layers positions
    max(0, P-511)..P-1 from ring slots p mod 512 -- older ones are outside every chunk
    query's window) followed by the chunk's own keys, rotated at their positions.  The
    visibility rule is the same as for ``prefill`` over positions.  q [B,n,16,256],
    k/v [B,n,4,256] (k before RoPE), gate [B,n,16], cache [B,cap,4,256]: bf16 bits.
    Returns float64 [B, len(rows), 16, 256].  This is the step between prefill and decode
    when a long context is fed in chunks or a prefix is reused ([F16Q4] section 一 and
    [GGUF] section 四 on long contexts held in the KV cache).
    """
    th, rd, w = layer_params(layer_type)
    q = np.asarray(q)
    B, n, H, D = q.shape
    Hk = np.asarray(k).shape[2]
    P = int(start_pos)
    if P < 0:
        raise ValueError("start_pos must be >= 0")
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = softmax_scale(D)
    h_lo = 0 if w is None else max(0, P - (w - 1))
    h_pos = np.arange(h_lo, P)                                        # cached positions in reach
    h_slot = np.array([cache_slot(int(p), layer_type) for p in h_pos], dtype=np.int64)
    new_pos = P + np.arange(n)
    kpos = np.concatenate([h_pos, new_pos])
    out = np.zeros((B, len(rows), H, D), dtype=np.float64)
    for b in range(B):
        kr = np.concatenate([bf16_to_f64(np.asarray(cache_k)[b, h_slot]),
                             rope(bf16_to_f64(k[b]), new_pos, th, rd)])    # [len(kpos), Hk, D]
        vb = np.concatenate([bf16_to_f64(np.asarray(cache_v)[b, h_slot]), bf16_to_f64(v[b])])
        for r0 in range(0, len(rows), row_block):
            rr = rows[r0:r0 + row_block]
            qpos = P + rr
            vis = visibility(qpos, kpos, w)
            qr = rope(bf16_to_f64(q[b, rr]), qpos, th, rd)
            gb = np.asarray(gate)[b, rr]
            for h in range(H):
                g = kv_head_of(h, H, Hk)
                out[b, r0:r0 + len(rr), h] = _attend(
                    qr[:, h], kr[:, g], vb[:, g], vis, bf16_to_f64(gb[:, h]), scale)
    return out


def prefill_varlen(q, k, v, gate, cu_seqlens, layer_type, rows=None) -> np.ndarray:
    """Prefill of sequences packed back to back: sequence b owns token rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1, its token t sits at position t, and it attends
    only to itself -- each sequence is the one-sequence ``prefill`` of its own rows.
    q [T,16,256], k/v [T,4,256], gate [T,16]; ``rows`` are packed row indices (default
    all).  Returns float64 [len(rows), 16, 256].
    """
    cu = [int(x) for x in cu_seqlens]
    T = np.asarray(q).shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows),) + np.asarray(q).shape[1:], dtype=np.float64)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if hi <= lo or len(sel) == 0:
            continue
        one = lambda x: np.asarray(x)[lo:hi][None]
        out[sel] = prefill(one(q), one(k), one(v), one(gate), layer_type, rows=rows[sel] - lo)[0]
    return out


def cache_slot(position: int, layer_type: int, window: int = WINDOW) -> int:
    """Cache slot of a position: itself on full layers, position mod 512 on sliding layers.

    The sliding layer keeps only its window ([CFG] section "混合注意力": a constant
    KV footprint independent of context; [GGUF] section 三: the 27 window layers take a
    fixed ~57 MB).
    """
    return position if layer_type == FULL else position % window


def kv_append(cache_k, cache_v, k, v, pos, layer_type):
    """Cache after appending ``n_new`` tokens per sequence.

    cache_k/cache_v [B, cap, 4, 256] bf16 bits; k/v [B, n_new, 4, 256] (k before RoPE);
    pos [B] = position of the first new token.  Token t of sequence b sits at position
    p = pos[b] + t: its rotated key (rounded to bf16) and its value go to
    ``cache_slot(p)``.  Tokens are written in order, so on a ring a later position
    replaces an earlier one in the same slot.  Returns new (cache_k, cache_v).
    """
    th, rd, _ = layer_params(layer_type)
    ck = np.array(cache_k, dtype=np.uint16, copy=True)
    cv = np.array(cache_v, dtype=np.uint16, copy=True)
    B, n_new = np.asarray(k).shape[:2]
    for b in range(B):
        p = int(pos[b]) + np.arange(n_new)
        kr = rope(bf16_to_f64(k[b]), p, th, rd)
        kbits = round_to_bf16_bits(kr)
        for t in range(n_new):
            s = cache_slot(int(p[t]), layer_type)
            ck[b, s] = kbits[t]
            cv[b, s] = np.asarray(v)[b, t]
    return ck, cv


def decode(q, gate, cache_k, cache_v, seq_lens, layer_type) -> np.ndarray:
    """One query token per sequence against its cache.

    q [B,16,256] (before RoPE), gate [B,16], cache [B,cap,4,256] holding post-RoPE keys,
    seq_lens [B] = tokens in the cache including the current one.  The query sits at
    position L-1; the visible keys are positions 0..L-1 (full) or max(0, L-512)..L-1
    (sliding, read from ring slots p mod 512).  Returns float64 [B,16,256].
    """
    return decode_rows(q, gate, lambda b, slots, g: bf16_to_f64(np.asarray(cache_k)[b, slots, g]),
                       lambda b, slots, g: bf16_to_f64(np.asarray(cache_v)[b, slots, g]),
                       np.asarray(cache_k).shape[2], seq_lens, layer_type)


def decode_rows(q, gate, key_rows, value_rows, n_kv_heads: int, seq_lens, layer_type) -> np.ndarray:
    """``decode`` over a cache given by accessors: key_rows(b, slots, g) and
    value_rows(b, slots, g) return the float64 rows [len(slots), 256] of KV head g of
    sequence b held in those slots."""
    th, rd, w = layer_params(layer_type)
    q = np.asarray(q)
    B, H, D = q.shape
    Hk = n_kv_heads
    scale = softmax_scale(D)
    out = np.zeros((B, H, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < 1:
            raise ValueError("a decode sequence needs at least its own token in the cache")
        qp = L - 1
        lo = 0 if w is None else max(0, L - w)
        kpos = np.arange(lo, L)
        slots = np.array([cache_slot(int(p), layer_type) for p in kpos], dtype=np.int64)
        vis = visibility([qp], kpos, w)
        qr = rope(bf16_to_f64(q[b])[None], [qp], th, rd)[0]          # [H, D]
        gb = bf16_to_f64(np.asarray(gate)[b])
        for g in range(Hk):                                          # one KV head at a time
            kr = key_rows(b, slots, g)                               # [n, D], already rotated
            vb = value_rows(b, slots, g)
            for h in range(H):
                if kv_head_of(h, H, Hk) == g:
                    out[b, h] = _attend(qr[h][None], kr, vb, vis, gb[h:h + 1], scale)[0]
    return out
