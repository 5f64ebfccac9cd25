"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws numbers and rounds them to bfloat16.  It holds none of the
attention arithmetic (no RoPE, masks, softmax or gating): both the HIP path and the
CPU oracle receive the same bf16 bit patterns from here and nothing else.

Recipe (every tensor):
  * i.i.d. N(0, 1) float32 values from numpy's PCG64 generator;
  * the tensor is cut into blocks of ``BLOCK`` elements in C order; block ``i`` is
    drawn from ``SeedSequence(seed, spawn_key=(tensor_index, i))`` so the values do
    not depend on how many threads produce them;
  * each float32 value is rounded to bfloat16 by round-to-nearest-even on its bits.

Shapes follow the model the pages describe: 16 query heads, 4 KV heads, head_dim 256
(Spark-X2.6-4B-FP8 walkthrough, nxmr.cn/news/148448, section 一, config table).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

N_Q_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 256
BLOCK = 1 << 22

# Seeds of the measured workloads (each tensor then takes its own stream below them).
SEED_SLIDING_S1024 = 20261   # one sliding layer, batch 1, S = 1024
SEED_FULL_S8192 = 20262      # one full layer, batch 1, S = 8192
SEED_DECODE_B64 = 20263      # batched decode, batch 64, lengths uniform in [1024, 32768]
SEED_STACK_S32768 = 20264    # the 36-layer prefill stack, S = 32768 (times 1000 plus the layer)
SEED_LONG_DECODE = 20265     # decode at 131072 tokens (batch 4) and 2^20 (batch 1)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tensor_index: int, shape) -> np.ndarray:
    """N(0,1) bf16 bit patterns of ``shape`` for tensor ``tensor_index`` of a seed."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(i: int) -> None:
        lo = i * BLOCK
        hi = min(n, lo + BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=(tensor_index, i))
        vals = np.random.default_rng(ss).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(vals)

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def prefill_inputs(seed: int, batch: int, seq: int) -> dict:
    """Q [B,S,16,256], K/V [B,S,4,256], gate logits [B,S,16]; bf16 bits, pre-RoPE."""
    return {
        "q": normal_bf16(seed, 0, (batch, seq, N_Q_HEADS, HEAD_DIM)),
        "k": normal_bf16(seed, 1, (batch, seq, N_KV_HEADS, HEAD_DIM)),
        "v": normal_bf16(seed, 2, (batch, seq, N_KV_HEADS, HEAD_DIM)),
        "gate": normal_bf16(seed, 3, (batch, seq, N_Q_HEADS)),
    }


def stack_layer_seed(layer: int) -> int:
    """Seed of layer ``layer`` (0-based) of the 36-layer prefill stack."""
    return SEED_STACK_S32768 * 1000 + layer


def decode_seq_lens(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence context lengths drawn uniformly from [lo, hi] (inclusive)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(99,)))
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def cache_rows(seed: int, b: int, n: int) -> tuple:
    """Cache rows (K, V) [n,4,256] of sequence ``b``: keys are treated as already rotated."""
    k = normal_bf16(seed, 2 + 2 * b, (n, N_KV_HEADS, HEAD_DIM))
    v = normal_bf16(seed, 3 + 2 * b, (n, N_KV_HEADS, HEAD_DIM))
    return k, v


def decode_inputs(seed: int, batch: int, capacity: int, fill_lens=None) -> dict:
    """Query [B,16,256], gate logits [B,16] and a K/V cache [B,capacity,4,256].

    With ``fill_lens`` only the first ``min(fill_lens[b], capacity)`` slots of sequence
    ``b`` are drawn (by ``cache_rows``); the rest stay zero and are never read.
    """
    q = normal_bf16(seed, 0, (batch, N_Q_HEADS, HEAD_DIM))
    gate = normal_bf16(seed, 1, (batch, N_Q_HEADS))
    ck = np.zeros((batch, capacity, N_KV_HEADS, HEAD_DIM), dtype=np.uint16)
    cv = np.zeros_like(ck)
    for b in range(batch):
        n = capacity if fill_lens is None else min(int(fill_lens[b]), capacity)
        ck[b, :n], cv[b, :n] = cache_rows(seed, b, n)
    return {"q": q, "gate": gate, "cache_k": ck, "cache_v": cv}


def int8_codes(seed: int, tensor_index: int, shape) -> np.ndarray:
    """Uniform int8 values in [-127, 127] of ``shape`` (blocked streams as above)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.int8)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(i: int) -> None:
        lo = i * BLOCK
        hi = min(n, lo + BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=(tensor_index, i))
        out[lo:hi] = np.random.default_rng(ss).integers(-127, 128, hi - lo, dtype=np.int16).astype(np.int8)

    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def fp16_scales(seed: int, tensor_index: int, shape, lo: float = 0.005, hi: float = 0.03) -> np.ndarray:
    """Uniform fp16 values in [lo, hi) of ``shape`` (one stream; scales are small)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_index, 0)))
    return rng.uniform(lo, hi, size=tuple(int(s) for s in shape)).astype(np.float16)


def q8_cache_rows(seed: int, b: int, n: int) -> tuple:
    """8-bit cache rows of sequence ``b``: (K codes, K scales, V codes, V scales), codes
    [n,4,256] int8 and scales [n,4,8] fp16 (a q8_0 step of 0.005-0.03 spans about the
    range of N(0,1) values)."""
    return (int8_codes(seed, 100 + 4 * b, (n, N_KV_HEADS, HEAD_DIM)),
            fp16_scales(seed, 101 + 4 * b, (n, N_KV_HEADS, HEAD_DIM // 32)),
            int8_codes(seed, 102 + 4 * b, (n, N_KV_HEADS, HEAD_DIM)),
            fp16_scales(seed, 103 + 4 * b, (n, N_KV_HEADS, HEAD_DIM // 32)))


def normal_bf16_scaled(seed: int, tensor_index: int, shape, log2_scale: int) -> np.ndarray:
    """As normal_bf16, with every value multiplied by 2**log2_scale before rounding."""
    shape = tuple(int(s) for s in shape)
    vals = bf16_bits_to_f32(normal_bf16(seed, tensor_index, shape)) * np.float32(2.0 ** log2_scale)
    return f32_to_bf16_bits(vals)


def fp8_e4m3_codes(seed: int, tensor_index: int, shape, exp_lo: int = -3, exp_hi: int = 3) -> np.ndarray:
    """Random FP8 E4M3 (OCP, bias 7) codes: uniform sign, exponent uniform in
    [exp_lo, exp_hi], uniform 3-bit mantissa -- finite normal values of magnitude
    2^exp_lo .. 2^(exp_hi+1) (synthetic quantised weights)."""
    shape = tuple(int(s) for s in shape)
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_index, 0)))
    sign = rng.integers(0, 2, size=shape) << 7
    e = rng.integers(exp_lo, exp_hi + 1, size=shape) + 7
    m = rng.integers(0, 8, size=shape)
    return (sign | (e << 3) | m).astype(np.uint8)


def uniform_f32(seed: int, tensor_index: int, shape, lo: float, hi: float) -> np.ndarray:
    """Uniform float32 values in [lo, hi) (e.g. per-channel weight scales)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_index, 0)))
    return rng.uniform(lo, hi, size=tuple(int(s) for s in shape)).astype(np.float32)


def proj_inputs(seed: int, tokens: int) -> dict:
    """Hidden states x [T, 2560] bf16 N(0,1); q_k_v_proj weights as E4M3 codes
    [6144, 2560] (rms of the code values about 4.9) with per-channel scales in
    [0.0025, 0.004), so that q, k, v come out with an rms of about 0.8, like the N(0,1)
    attention inputs elsewhere; g_proj weights [16, 2560] bf16 N(0, 2^-12) (gate logits of
    order 1)."""
    return {
        "x": normal_bf16(seed, 0, (tokens, 2560)),
        "w": fp8_e4m3_codes(seed, 1, (6144, 2560)),
        "w_scale": uniform_f32(seed, 2, (6144,), 0.0025, 0.004),
        "wg": normal_bf16_scaled(seed, 3, (16, 2560), -6),
    }
