#!/usr/bin/env python3
"""Benchmark of the hybrid GQA attention path on one MI355X.

Step = one prefill of a full-attention layer (batch 1, 8192 tokens, 16 query / 4 KV heads,
head_dim 256, RoPE theta 5e6 on the first 64 dims, sigmoid head gate): the K RoPE pass, then
the attention kernel (Q RoPE, masked QK^T, online softmax, PV and the gate epilogue); both
launches are inside the timed region.
``value`` is prefill tokens/s.  The same line carries the decode half of the metric,
measured on batched decode (batch 64, context lengths uniform in [1024, 32768], full
layer), as KV GB/s against HBM peak, and the CPU oracle timed on a bounded sample.

Inputs are seeded synthetic bf16 N(0,1) tensors already resident in HBM; timing uses HIP
events on the stream the kernels are launched on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention tokens/s (prefill, % MFMA peak) + decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_launches(fn, steps, warmup):
    """Average ms per call over ``steps`` back-to-back calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def bench_prefill(fga, synth, steps, warmup, S=8192):
    import torch
    inp = synth.prefill_inputs(synth.SEED_FULL_S8192, 1, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    out = torch.empty_like(q)
    ws = torch.empty(fga.prefill_workspace_bytes(fga.FULL, 1, S), dtype=torch.uint8, device="cuda")
    ms = time_launches(lambda: fga.prefill(fga.FULL, q, k, v, g, out=out, workspace=ws), steps, warmup)
    pairs = S * (S + 1) // 2                       # visible (query, key) pairs, causal
    flops = 4 * 256 * 16 * pairs                   # QK^T + PV, 16 query heads
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "ms": ms,
        "tokens_per_s": S / (ms * 1e-3),
        "flops": flops,
        "tflops": tflops,
    }


def bench_decode(fga, synth, steps, warmup):
    import numpy as np
    import torch
    seed = synth.SEED_DECODE_B64
    B, cap = 64, 32768
    lens = synth.decode_seq_lens(seed, B, 1024, 32768)
    q = to_dev(synth.normal_bf16(seed, 0, (B, 16, 256)))
    gate = to_dev(synth.normal_bf16(seed, 1, (B, 16)))
    cache = fga.KVCache(fga.FULL, B, cap)
    for b in range(B):
        kb, vb = synth.cache_rows(seed, b, int(lens[b]))
        cache.k[b, :lens[b]] = to_dev(kb)
        cache.v[b, :lens[b]] = to_dev(vb)
    sl = torch.as_tensor(lens).cuda()
    ws = torch.empty(fga.decode_workspace_bytes(fga.FULL, B, cap), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    ms = time_launches(lambda: fga.decode(fga.FULL, q, gate, cache, sl, cap, out=out, workspace=ws),
                       steps, warmup)
    kv_bytes = int(lens.astype(np.int64).sum()) * 4 * 256 * 2 * 2
    io_bytes = B * (16 * 256 * 2 * 2 + 16 * 2)
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    return {"ms": ms, "bytes": kv_bytes + io_bytes, "gbs": gbs, "lens_sum": int(lens.sum())}


def dev_normal(gen, shape):
    """Seeded N(0,1) bf16 tensor drawn on the device (for the large timing-only inputs)."""
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def time_each(fn, n, warmup, before=None):
    """Median ms of ``n`` single calls, each bracketed by HIP events; ``before`` runs
    (untimed) ahead of every call, e.g. to evict the caches."""
    import statistics
    import torch
    for _ in range(warmup):
        fn()
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(n):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def sliding_pairs(S):
    return sum(min(i + 1, 512) for i in range(S))


def bench_configs(fga, synth):
    """The other workloads of the hot path's scope table, each timed on its own:
    sliding prefill S=1024; a chunk of 8192 after a cached prefix of 8192 (both layer
    types); a variable-length batch of 16 sequences; the 36-layer stack at S=32768; decode
    over the 8-bit cache; one decode step of all 36 layers (bf16 and 8-bit caches); batched decode (full, cold
    caches; sliding ring, warm and cold); long decode at 128K and 1M tokens."""
    import numpy as np
    import torch
    out = {}
    gen = torch.Generator(device="cuda")

    # One sliding layer, batch 1, S = 1024 (host-drawn inputs, as in the tests).
    S = 1024
    inp = synth.prefill_inputs(synth.SEED_SLIDING_S1024, 1, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    o = torch.empty_like(q)
    ws = torch.empty(fga.prefill_workspace_bytes(fga.SLIDING, 1, S), dtype=torch.uint8, device="cuda")
    ms = time_launches(lambda: fga.prefill(fga.SLIDING, q, k, v, g, out=o, workspace=ws), 200, 50)
    tf = 16384 * sliding_pairs(S) / (ms * 1e-3) / 1e12
    out["sliding_prefill_s1024"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                    "tokens_per_s": S / (ms * 1e-3)}
    log(f"sliding prefill S=1024: {ms * 1e3:.1f} us  {tf:.0f} TFLOP/s")
    del q, k, v, g, o, ws

    # Chunked prefill: a chunk of 8192 tokens after a cached prefix of 8192, batch 1, each
    # layer type (the prefix's keys are read from the cache, device-drawn N(0,1)).
    P = n = 8192
    gen.manual_seed(synth.SEED_FULL_S8192 + 100)
    q, k, v, g = (dev_normal(gen, (1, n, 16, 256)), dev_normal(gen, (1, n, 4, 256)),
                  dev_normal(gen, (1, n, 4, 256)), dev_normal(gen, (1, n, 16)))
    o = torch.empty_like(q)
    for lt, name in ((fga.FULL, "full"), (fga.SLIDING, "sliding")):
        cap = P + n if lt == fga.FULL else 512
        cache = fga.KVCache(lt, 1, cap, k=dev_normal(gen, (1, cap, 4, 256)), v=dev_normal(gen, (1, cap, 4, 256)))
        ws = torch.empty(fga.prefill_workspace_bytes(lt, 1, n), dtype=torch.uint8, device="cuda")
        ms = time_launches(lambda: fga.prefill(lt, q, k, v, g, out=o, cache=cache, start_pos=P,
                                               workspace=ws), 100, 20)
        pairs = n * P + n * (n + 1) // 2 if lt == fga.FULL else n * 512
        tf = 16384 * pairs / (ms * 1e-3) / 1e12
        out[f"chunk_prefill_{name}_p8192_n8192"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                                    "tokens_per_s": n / (ms * 1e-3)}
        log(f"chunked prefill {name} P=8192 n=8192: {ms:.3f} ms  {tf:.0f} TFLOP/s")
        del cache, ws
    del q, k, v, g, o

    # Variable-length batch: 16 sequences of lengths uniform in [512, 8192], packed.
    lens = np.random.default_rng(synth.SEED_FULL_S8192 + 200).integers(512, 8193, size=16)
    T = int(lens.sum())
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    gen.manual_seed(synth.SEED_FULL_S8192 + 201)
    q, k, v, g = (dev_normal(gen, (T, 16, 256)), dev_normal(gen, (T, 4, 256)),
                  dev_normal(gen, (T, 4, 256)), dev_normal(gen, (T, 16)))
    o = torch.empty_like(q)
    ws = torch.empty(fga.prefill_varlen_workspace_bytes(fga.FULL, T), dtype=torch.uint8, device="cuda")
    for lt, name in ((fga.FULL, "full"), (fga.SLIDING, "sliding")):
        ms = time_launches(lambda: fga.prefill_varlen(lt, q, k, v, g, cu, int(lens.max()), out=o, workspace=ws),
                           50, 10)
        pairs = int(sum(n * (n + 1) // 2 for n in lens)) if lt == fga.FULL else int(sum(sliding_pairs(int(n)) for n in lens))
        tf = 16384 * pairs / (ms * 1e-3) / 1e12
        out[f"varlen_prefill_{name}_16seq"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                               "tokens_per_s": T / (ms * 1e-3), "tokens": T}
        log(f"varlen prefill {name}, 16 sequences (T={T}): {ms:.3f} ms  {tf:.0f} TFLOP/s")
    del q, k, v, g, o, ws, cu

    # The 36-layer stack, batch 1, S = 32768, independent inputs per layer (drawn on
    # the device: 24 GB of N(0,1) bf16); layer l is full iff l % 4 == 3.
    S = 32768
    gen.manual_seed(synth.SEED_STACK_S32768)
    layers = []
    for layer in range(36):
        layers.append(((fga.FULL if layer % 4 == 3 else fga.SLIDING),
                       dev_normal(gen, (1, S, 16, 256)), dev_normal(gen, (1, S, 4, 256)),
                       dev_normal(gen, (1, S, 4, 256)), dev_normal(gen, (1, S, 16)),
                       torch.empty(1, S, 16, 256, dtype=torch.bfloat16, device="cuda")))
    ws = torch.empty(fga.prefill_workspace_bytes(fga.FULL, 1, S), dtype=torch.uint8, device="cuda")

    def stack():
        for lt, q, k, v, g, o in layers:
            fga.prefill(lt, q, k, v, g, out=o, workspace=ws)

    ms = time_launches(stack, 5, 2)
    flops = 9 * 16384 * (S * (S + 1) // 2) + 27 * 16384 * sliding_pairs(S)
    tf = flops / (ms * 1e-3) / 1e12
    out["stack36_prefill_s32768"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                     "tokens_per_s": S / (ms * 1e-3), "tflop": flops / 1e12}
    log(f"36-layer prefill stack S=32768: {ms:.2f} ms  {tf:.0f} TFLOP/s")
    del layers, ws
    torch.cuda.empty_cache()

    # Reading a 1 GiB buffer before each cold call evicts the 256 MB MALL and the L2s.  (A
    # copy would also evict them, but leaves dirty lines whose write-back then competes
    # with the timed call.)
    flush_a = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    flush = lambda: flush_a.sum()

    def decode_case(lt, B, lens, cap, seed, cold):
        lens = np.asarray(lens, dtype=np.int32)
        gen.manual_seed(seed)
        qd = dev_normal(gen, (B, 16, 256))
        gd = dev_normal(gen, (B, 16))
        cache = fga.KVCache(lt, B, cap, k=dev_normal(gen, (B, cap, 4, 256)),
                            v=dev_normal(gen, (B, cap, 4, 256)))
        sl = torch.as_tensor(lens).cuda()
        maxlen = int(lens.max())
        wsd = torch.empty(fga.decode_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(qd)
        call = lambda: fga.decode(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)
        ms = time_each(call, 30, 5, flush if cold else None)
        vis = np.minimum(lens, 512) if lt == fga.SLIDING else lens
        nbytes = int(vis.astype(np.int64).sum()) * 4096 + B * (16 * 256 * 4 + 32)
        return {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes,
                "cache": "cold" if cold else "warm"}

    # Batched decode: batch 64, lengths uniform in [1024, 32768].
    seed = synth.SEED_DECODE_B64
    lens = synth.decode_seq_lens(seed, 64, 1024, 32768)
    r = decode_case(fga.FULL, 64, lens, 32768, seed, cold=True)
    out["decode_b64_full_cold"] = r
    log(f"decode B=64 full, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
    torch.cuda.empty_cache()
    for cold in (False, True):
        r = decode_case(fga.SLIDING, 64, lens, 512, seed + 1, cold=cold)
        out[f"decode_b64_sliding_{r['cache']}"] = r
        log(f"decode B=64 sliding ring, {r['cache']}: {r['us']:.1f} us  {r['gbs']:.0f} GB/s")

    # Long decode (B = 4 at 131072 tokens, B = 1 at 2^20), full layer (cache capacity = L) and the sliding ring.
    for B, L in ((4, 131072), (1, 1 << 20)):
        r = decode_case(fga.FULL, B, [L] * B, L, synth.SEED_LONG_DECODE + B, cold=True)
        out[f"decode_full_b{B}_l{L}_cold"] = r
        log(f"long decode full B={B} L={L}, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
        torch.cuda.empty_cache()
        r = decode_case(fga.SLIDING, B, [L] * B, 512, synth.SEED_LONG_DECODE + 10 + B, cold=True)
        out[f"decode_sliding_b{B}_l{L}_cold"] = r
        log(f"long decode sliding B={B} L={L}, cold: {r['us']:.1f} us")
    # 8-bit (q8_0) cache: 272 bytes per key row and KV head for K and for V, instead of 512.
    def decode_q8_case(lt, B, lens, cap, seed, cold):
        lens = np.asarray(lens, dtype=np.int32)
        gen.manual_seed(seed)
        qd = dev_normal(gen, (B, 16, 256))
        gd = dev_normal(gen, (B, 16))
        codes = lambda: torch.randint(-127, 128, (B, cap, 4, 256), generator=gen, device="cuda", dtype=torch.int8)
        scales = lambda: (0.005 + 0.025 * torch.rand((B, cap, 4, 8), generator=gen, device="cuda")).half()
        cache = fga.KVCacheQ8(lt, B, cap, k=codes(), k_scale=scales(), v=codes(), v_scale=scales())
        sl = torch.as_tensor(lens).cuda()
        maxlen = int(lens.max())
        wsd = torch.empty(fga.decode_q8_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(qd)
        call = lambda: fga.decode_q8(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)
        ms = time_each(call, 30, 5, flush if cold else None)
        vis = np.minimum(lens, 512) if lt == fga.SLIDING else lens
        nbytes = int(vis.astype(np.int64).sum()) * 4 * 2 * 272 + B * (16 * 256 * 4 + 32)
        return {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes,
                "cache": "cold" if cold else "warm", "kv": "q8_0"}

    seed = synth.SEED_DECODE_B64
    lens = synth.decode_seq_lens(seed, 64, 1024, 32768)
    r = decode_q8_case(fga.FULL, 64, lens, 32768, seed + 50, cold=True)
    out["decode_q8_b64_full_cold"] = r
    log(f"decode q8 B=64 full, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
    torch.cuda.empty_cache()
    r = decode_q8_case(fga.SLIDING, 64, lens, 512, seed + 51, cold=True)
    out["decode_q8_b64_sliding_cold"] = r
    log(f"decode q8 B=64 sliding ring, cold: {r['us']:.1f} us  {r['gbs']:.0f} GB/s")
    for B, L in ((4, 131072), (1, 1 << 20)):
        r = decode_q8_case(fga.FULL, B, [L] * B, L, synth.SEED_LONG_DECODE + 60 + B, cold=True)
        out[f"decode_q8_full_b{B}_l{L}_cold"] = r
        log(f"long decode q8 full B={B} L={L}, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
        torch.cuda.empty_cache()
    # One decode step of the whole 36-layer model: batch 64, lengths uniform in [1024, 32768]
    # (each layer its own cache: 9 full caches, 27 rings), bf16 and 8-bit caches.
    del flush_a
    torch.cuda.empty_cache()
    seed = synth.SEED_DECODE_B64
    lens = synth.decode_seq_lens(seed, 64, 1024, 32768)
    sl = torch.as_tensor(lens).cuda()
    maxlen = int(lens.max())
    B = 64
    for kv in ("bf16", "q8_0"):
        gen.manual_seed(seed + 300)
        layers = []
        for layer in range(36):
            lt = fga.FULL if layer % 4 == 3 else fga.SLIDING
            cap = maxlen if lt == fga.FULL else 512
            if kv == "bf16":
                cache = fga.KVCache(lt, B, cap, k=dev_normal(gen, (B, cap, 4, 256)), v=dev_normal(gen, (B, cap, 4, 256)))
                wsb = fga.decode_workspace_bytes(lt, B, maxlen)
            else:
                codes = lambda: torch.randint(-127, 128, (B, cap, 4, 256), generator=gen, device="cuda", dtype=torch.int8)
                scales = lambda: (0.005 + 0.025 * torch.rand((B, cap, 4, 8), generator=gen, device="cuda")).half()
                cache = fga.KVCacheQ8(lt, B, cap, k=codes(), k_scale=scales(), v=codes(), v_scale=scales())
                wsb = fga.decode_q8_workspace_bytes(lt, B, maxlen)
            layers.append((lt, cache, dev_normal(gen, (B, 16, 256)), dev_normal(gen, (B, 16)),
                           torch.empty(wsb, dtype=torch.uint8, device="cuda"),
                           torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")))
        dec = fga.decode if kv == "bf16" else fga.decode_q8

        def step():
            for lt, cache, qd, gd, wsd, od in layers:
                dec(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)

        ms = time_launches(step, 10, 3)
        vis = int(lens.astype(np.int64).sum()) * 9 + int(np.minimum(lens, 512).astype(np.int64).sum()) * 27
        row = 2 * 4 * (512 if kv == "bf16" else 272)
        nbytes = vis * row + 36 * B * (16 * 256 * 4 + 32)
        out[f"decode_step_36_layers_b64_{kv}"] = {"ms": ms, "tokens_per_s": B / (ms * 1e-3),
                                                  "gbs": nbytes / (ms * 1e-3) / 1e9,
                                                  "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                  "bytes": nbytes, "kv": kv}
        log(f"36-layer decode step, batch 64 ({kv} cache): {ms:.2f} ms  {B / (ms * 1e-3):.0f} tokens/s  "
            f"{nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
        del layers
        torch.cuda.empty_cache()
    # KV append: a bulk append of 32768 tokens (batch 1, full cache; the sliding ring keeps
    # the last 512), and the one-token append of a batch-64 decode step at positions
    # U[1024, 32768]; bf16 and 8-bit caches.  Bytes per written token: its K and V read
    # (2 x 2 KB) plus what the cache receives (2 x 2 KB, or 2 x 1088 B for q8_0).
    lens = synth.decode_seq_lens(synth.SEED_DECODE_B64, 64, 1024, 32768)
    for kv in ("bf16", "q8_0"):
        for lt, B, n in ((fga.FULL, 1, 32768), (fga.SLIDING, 1, 32768), (fga.FULL, 64, 1), (fga.SLIDING, 64, 1)):
            gen.manual_seed(synth.SEED_DECODE_B64 + 500 + B)
            cap = 512 if lt == fga.SLIDING else (32768 if B == 64 else n)
            k = dev_normal(gen, (B, n, 4, 256))
            v = dev_normal(gen, (B, n, 4, 256))
            pos = torch.as_tensor(lens - 1 if B == 64 else np.zeros(B, np.int32)).to(torch.int32).cuda()
            if kv == "bf16":
                cache = fga.KVCache(lt, B, cap)
                call = lambda: fga.kv_append(lt, k, v, pos, cache)
            else:
                cache = fga.KVCacheQ8(lt, B, cap)
                call = lambda: fga.kv_append_q8(lt, k, v, pos, cache)
            written = B * (min(n, 512) if lt == fga.SLIDING else n)
            row = 2 * 4 * (512 if kv == "bf16" else 272)
            nbytes = written * (2 * 4 * 512 + row)   # only the tokens it writes are read
            ms = time_each(call, 30, 5)
            name = f"kv_append_{kv}_{'full' if lt == fga.FULL else 'sliding'}_b{B}_n{n}"
            out[name] = {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                         "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes}
            log(f"kv append ({kv}) {'full' if lt == fga.FULL else 'sliding'} B={B} n={n}: {ms * 1e3:.1f} us  "
                f"{nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
            del cache, k, v
    torch.cuda.empty_cache()
    # The W8A8 FP8 q/k/v projection with the bf16 gate projection upstream of the path:
    # T tokens of hidden 2560 -> 6144 q/k/v channels (+ 16 gate logits).
    for T in (8192, 32768):
        gen.manual_seed(synth.SEED_SLIDING_S1024 + 400 + T)
        x = dev_normal(gen, (T, 2560))
        w = torch.randint(0x18, 0x50, (6144, 2560), generator=gen, device="cuda", dtype=torch.uint8)
        w = torch.where(torch.rand(w.shape, generator=gen, device="cuda") < 0.5, w, w | 0x80)
        wsc = 0.0025 + 0.0015 * torch.rand(6144, generator=gen, device="cuda")
        wg = (dev_normal(gen, (16, 2560)).float() / 64).to(torch.bfloat16)
        outs = (torch.empty(T, 16, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 4, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 4, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 16, dtype=torch.bfloat16, device="cuda"))
        wsp = torch.empty(fga.qkv_proj_fp8_workspace_bytes(T), dtype=torch.uint8, device="cuda")
        ms = time_launches(lambda: fga.qkv_proj_fp8(x, w, wsc, wg, out=outs, workspace=wsp), 20, 5)
        flops = 2 * T * 2560 * 6144
        out[f"qkv_proj_fp8_t{T}"] = {"us": ms * 1e3, "tflops_fp8": flops / (ms * 1e-3) / 1e12,
                                     "frac_fp8_mfma": flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                                     "gate_gflops_bf16": 2 * T * 2560 * 16 / 1e9}
        log(f"FP8 q/k/v + bf16 gate projection T={T}: {ms * 1e3:.0f} us  "
            f"{flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s (fp8 GEMM flops)")
        del x, w, wsc, wg, outs, wsp
        torch.cuda.empty_cache()
    return out


def copy_calibration():
    """Device-to-device copy of 4 GiB: the plain copy of known size that scales the HBM
    traffic counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = 1 << 31                                   # bf16 elements: 4 GiB
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ms = time_launches(lambda: y.copy_(x), 3, 1)
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "ms": ms,
                      "read_plus_write_gbs": 4 * n / (ms * 1e-3) / 1e9}), flush=True)


def kernel_source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "full_gqa_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of ``kernel`` recorded in profiles/traffic.json, or None when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash(rec["sources"]):
        return None
    return rec["hbm_bytes_per_launch"]


def cpu_baseline(synth, budget_s=12.0, S=8192):
    """The oracle, as it stands, on randomly sampled query rows of the prefill workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = synth.prefill_inputs(synth.SEED_FULL_S8192, 1, S)
    rng = np.random.default_rng(12345)
    rows_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        rows = rng.choice(S, size=16, replace=False)
        oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], oracle.FULL, rows=rows)
        rows_done += len(rows)
    dt = time.perf_counter() - t0
    return {
        "value": rows_done / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_done} uniformly random query rows (all 16 heads) of the full-layer "
                  f"S={S} prefill, fp64 NumPy, {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-prefill", action="store_true")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-configs", action="store_true",
                    help="skip the other workloads (sliding prefill, 36-layer stack, decode variants)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 4 GiB device copy used to scale traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import full_gqa_attention_amd as fga
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    result = {
        "metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full-attention layer causal prefill, batch 1, seq 8192, 16 Q / 4 KV "
                               "heads, head_dim 256, RoPE theta 5e6 on the first 64 dims, sigmoid "
                               "head gate, bf16 N(0,1)",
                   "batch": 1, "seq_len": 8192, "layer_type": "full"},
    }
    if not args.skip_prefill:
        log("prefill ...")
        p = bench_prefill(fga, synth, args.steps, args.warmup)
        result["value"] = p["tokens_per_s"]
        result["ms_per_step"] = p["ms"]
        result["roofline"] = {"bound": "mfma", "achieved": p["tflops"], "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": p["tflops"] / PEAK_BF16_TFLOPS,
                              "traffic": measured_traffic("prefill_full")}
        log(f"prefill {p['ms']:.3f} ms  {p['tflops']:.1f} TFLOP/s")
    if not args.skip_decode:
        log("decode ...")
        d = bench_decode(fga, synth, args.steps, args.warmup)
        result["decode"] = {
            "workload": "batched decode, batch 64, context lengths uniform in [1024, 32768], full "
                        "layer, bf16 KV [ctx, 4, 256]",
            "value": d["gbs"], "unit": "GB/s", "ms_per_step": d["ms"],
            "roofline": {"bound": "hbm", "achieved": d["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": d["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic("decode_full")},
        }
        log(f"decode {d['ms']:.3f} ms  {d['gbs']:.0f} GB/s")
    if not args.skip_configs:
        log("other workloads ...")
        result["configs"] = bench_configs(fga, synth)
    if not args.skip_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
