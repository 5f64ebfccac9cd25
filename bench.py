#!/usr/bin/env python3
"""Benchmark of the hybrid GQA attention path on one MI355X.

Step = one prefill pass of the whole 36-layer attention stack, batch 1, 32768 tokens: 27
sliding-window layers and 9 full-attention layers (layer l is full iff l mod 4 = 3), each
with its own random bf16 N(0,1) Q/K/V/gate; 16 query / 4 KV heads, head_dim 256, RoPE per
layer type, sigmoid head gate; attention only.  A step is 36 spark_attn_prefill calls
(each: the K RoPE pass, then the attention kernel).  ``value`` is the stack's prefill
tokens/s.  ``roofline`` is that of the dominant kernel, the full-layer attention (9 of the
36 calls, most of the time), from HIP events around each of its calls in the timed steps.

The same line carries the decode half of the metric (``decode``: batched decode, batch 64,
context lengths uniform in [1024, 32768], full layer, KV GB/s against HBM peak), every
other workload under ``configs`` (each with its own roofline figures), and the CPU oracle
(``cpu_baseline``): timed on the host's cores on a row sample of the headline stack, and
over every output of the single-layer and decode workloads, with the GPU result's error
against it.  ``configs`` also holds a square bf16 GEMM of the vendor library timed on the
same box (context for the fractions of the published MFMA peak; not part of the path).

Inputs are synthetic and resident in HBM before timing starts; timing uses HIP events on
the stream the kernels are launched on.  Every timed loop is preceded by at least
``--preheat`` seconds of back-to-back calls (clocks ramp up under load), then ``--warmup``
calls.  ``--only`` runs a subset of the workloads (for profiling one at a time).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention tokens/s (prefill, % MFMA peak) + decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
FLOP_PER_PAIR = 4 * 256 * 16   # QK^T + PV over the 16 query heads, per visible (query, key) pair
WORKLOADS = ("stack", "full_s8192", "sliding_s1024", "chunk", "varlen", "decode_b64", "decode_long",
             "decode_q8", "decode_step", "append", "proj", "gemm_ref")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    """bf16 tensor -> uint16 bit patterns on the host."""
    import numpy as np
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t):
    import numpy as np
    return (host_bits(t).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def full_pairs(S):
    return S * (S + 1) // 2


def sliding_pairs(S):
    return sum(min(i + 1, 512) for i in range(S))


def dev_normal(gen, shape):
    """Seeded N(0,1) bf16 tensor drawn on the device (for the large timing-only inputs)."""
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


# ---------------------------------------------------------------------------------- timing
def preheat(fn, seconds):
    """Back-to-back calls until ``seconds`` have passed (at least one round)."""
    import torch
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return time.perf_counter() - t0


def time_launches(fn, steps, warmup, preheat_s):
    """Mean ms per call over ``steps`` back-to-back calls, HIP events on the current stream,
    after ``preheat_s`` seconds of calls and ``warmup`` more."""
    import torch
    pre = preheat(fn, preheat_s)
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
    return start.elapsed_time(end) / steps, pre


SLEEP_CYCLES = 400_000


def time_each(fn, n, warmup, preheat_s, before):
    """Median ms of ``n`` single calls, each bracketed by HIP events.  ``before`` enqueues
    device work ahead of every call (a cache flush, or a spin that evicts nothing); the
    call and its events are enqueued while that work still runs, so the events time the
    call on the device and not the host's launch of it."""
    import torch
    preheat(fn, preheat_s)
    for _ in range(warmup):
        fn()
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(n):
        before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def spin():
    import torch
    torch.cuda._sleep(SLEEP_CYCLES)


# ---------------------------------------------------------------------------------- oracle
def host_info():
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    aff = len(os.sched_getaffinity(0))
    return {"affinity_cores": aff, "blas_threads": blas, "cpu_model": model,
            "threads_used": min(aff, blas) if blas else aff}


def parity(got, want):
    import numpy as np
    d = np.abs(got - want)
    max_abs = float(d.max())
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    return {"max_abs": max_abs, "rel_l2": rel, "within_bar": bool(max_abs <= 1e-2 and rel <= 5e-3)}


class Ctx:
    def __init__(self, fga, synth, args):
        self.fga, self.synth, self.args = fga, synth, args
        self.cpu = not args.skip_cpu_baseline
        self.oracle_runs = {}          # workload -> oracle timing and GPU error
        self.configs = {}
        import torch
        self.gen = torch.Generator(device="cuda")
        self._flush = None

    def flush(self):
        """Read a 1 GiB buffer: evicts the 256 MB MALL and the L2s (a copy would leave dirty
        lines whose write-back then lands in the timed call)."""
        import torch
        if self._flush is None:
            self._flush = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        self._flush.sum()

    def drop_flush(self):
        self._flush = None

    def oracle_check(self, name, what, run, got, n_out, unit):
        """Time ``run()`` (the oracle) and compare its result with the GPU's ``got``."""
        t0 = time.perf_counter()
        want = run()
        dt = time.perf_counter() - t0
        rec = {"what": what, "oracle_s": dt, unit: n_out, f"{unit}_per_s": n_out / dt}
        rec.update(parity(got, want))
        self.oracle_runs[name] = rec
        log(f"  oracle {name}: {dt:.1f} s, max_abs {rec['max_abs']:.2e}, rel_l2 {rec['rel_l2']:.2e}")


# ------------------------------------------------------------------------------- workloads
def w_stack(ctx, steps, warmup, preheat_s):
    """The 36-layer prefill stack at S = 32768 (inputs drawn on the device, 24 GB)."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    S = 32768
    ctx.gen.manual_seed(synth.SEED_STACK_S32768)
    layers = []
    for layer in range(36):
        layers.append((fga.layer_type_of(layer), dev_normal(ctx.gen, (1, S, 16, 256)),
                       dev_normal(ctx.gen, (1, S, 4, 256)), dev_normal(ctx.gen, (1, S, 4, 256)),
                       dev_normal(ctx.gen, (1, S, 16)),
                       torch.empty(1, S, 16, 256, dtype=torch.bfloat16, device="cuda")))
    ws = torch.empty(fga.prefill_workspace_bytes(fga.FULL, 1, S), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run(evs=None):
        for i, (lt, q, k, v, g, o) in enumerate(layers):
            if evs is not None:
                evs[i][0].record(stream)
            fga.prefill(lt, q, k, v, g, out=o, workspace=ws)
            if evs is not None:
                evs[i][1].record(stream)

    pre = preheat(run, preheat_s)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(36)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(steps):
        run(ev[s])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    per = {fga.FULL: [], fga.SLIDING: []}
    for s in range(steps):
        for i, (lt, *_rest) in enumerate(layers):
            per[lt].append(ev[s][i][0].elapsed_time(ev[s][i][1]))
    full_ms = float(np.mean(per[fga.FULL]))
    sl_ms = float(np.mean(per[fga.SLIDING]))
    flops = 9 * FLOP_PER_PAIR * full_pairs(S) + 27 * FLOP_PER_PAIR * sliding_pairs(S)
    f_full = FLOP_PER_PAIR * full_pairs(S)
    f_sl = FLOP_PER_PAIR * sliding_pairs(S)
    res = {"ms": ms, "tokens_per_s": S / (ms * 1e-3), "tflop": flops / 1e12,
           "tflops": flops / (ms * 1e-3) / 1e12, "preheat_s": pre,
           "full_call_ms": full_ms, "full_call_tflops": f_full / (full_ms * 1e-3) / 1e12,
           "sliding_call_ms": sl_ms, "sliding_call_tflops": f_sl / (sl_ms * 1e-3) / 1e12,
           "full_flop_per_call": f_full, "sliding_flop_per_call": f_sl}
    res["frac_mfma"] = res["tflops"] / PEAK_BF16_TFLOPS
    log(f"36-layer prefill stack S=32768: {ms:.2f} ms/step  {res['tflops']:.0f} TFLOP/s; full call "
        f"{full_ms:.3f} ms ({res['full_call_tflops']:.0f} TFLOP/s), sliding call {sl_ms * 1e3:.0f} us "
        f"({res['sliding_call_tflops']:.0f} TFLOP/s); preheat {pre:.2f} s")
    if ctx.cpu:
        cpu_stack_sample(ctx, layers, S)
    del layers, ws
    torch.cuda.empty_cache()
    return res


def cpu_stack_sample(ctx, layers, S):
    """The oracle on 192 rows of one full layer (3) and one sliding layer (0) of the timed
    stack -- the edge rows 0, 1, 511, 512, 513, S/2, S-1 and uniformly random others -- on the
    same inputs, against the GPU's outputs of those rows."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(ctx.synth.SEED_STACK_S32768 + 1)
    rec = {}
    fixed = np.array([0, 1, 511, 512, 513, S // 2, S - 1])
    for layer, n_rows in ((3, 192), (0, 192)):
        lt, q, k, v, g, o = layers[layer]
        others = np.setdiff1d(np.arange(S), fixed)
        rows = np.sort(np.concatenate([fixed, rng.choice(others, size=n_rows - len(fixed), replace=False)]))
        inp = [host_bits(t) for t in (q, k, v, g)]
        got = f64_of(o[:, rows])
        t0 = time.perf_counter()
        want = oracle.prefill(*inp, lt, rows=rows)
        dt = time.perf_counter() - t0
        r = {"rows": n_rows, "oracle_s": dt, "rows_per_s": n_rows / dt}
        r.update(parity(got, want))
        rec["full" if lt == ctx.fga.FULL else "sliding"] = r
        log(f"  oracle stack layer {layer}: {n_rows} rows in {dt:.1f} s, max_abs {r['max_abs']:.2e}")
    t_tok = 9 / rec["full"]["rows_per_s"] + 27 / rec["sliding"]["rows_per_s"]
    ctx.stack_cpu = {"value": 1.0 / t_tok, "layers": rec}


def w_full_s8192(ctx, steps, warmup, preheat_s):
    """One full layer, S = 8192 (host-drawn inputs, as in the parity tests); the oracle over
    every output."""
    import torch
    fga, synth = ctx.fga, ctx.synth
    S = 8192
    inp = synth.prefill_inputs(synth.SEED_FULL_S8192, 1, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    out = torch.empty_like(q)
    ws = torch.empty(fga.prefill_workspace_bytes(fga.FULL, 1, S), dtype=torch.uint8, device="cuda")
    ms, pre = time_launches(lambda: fga.prefill(fga.FULL, q, k, v, g, out=out, workspace=ws), max(steps, 200),
                            warmup, preheat_s)
    flops = FLOP_PER_PAIR * full_pairs(S)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"full prefill S=8192: {ms * 1e3:.1f} us  {tf:.0f} TFLOP/s")
    if ctx.cpu:
        import oracle
        ctx.oracle_check("full_prefill_s8192", "every output (8192 rows x 16 heads)",
                         lambda: oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], oracle.FULL),
                         f64_of(out), S, "rows")
    return {"ms": ms, "tokens_per_s": S / (ms * 1e-3), "flop": flops, "tflops": tf, "preheat_s": pre,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill_full_s8192")}}


def w_sliding_s1024(ctx, steps, warmup, preheat_s):
    """One sliding layer, S = 1024 (host-drawn inputs); the oracle over every output."""
    import torch
    fga, synth = ctx.fga, ctx.synth
    S = 1024
    inp = synth.prefill_inputs(synth.SEED_SLIDING_S1024, 1, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    o = torch.empty_like(q)
    ws = torch.empty(fga.prefill_workspace_bytes(fga.SLIDING, 1, S), dtype=torch.uint8, device="cuda")
    ms, pre = time_launches(lambda: fga.prefill(fga.SLIDING, q, k, v, g, out=o, workspace=ws), max(steps, 200),
                            warmup, preheat_s)
    flops = FLOP_PER_PAIR * sliding_pairs(S)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"sliding prefill S=1024: {ms * 1e3:.1f} us  {tf:.0f} TFLOP/s")
    if ctx.cpu:
        import oracle
        ctx.oracle_check("sliding_prefill_s1024", "every output (1024 rows x 16 heads)",
                         lambda: oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], oracle.SLIDING),
                         f64_of(o), S, "rows")
    return {"ms": ms, "tokens_per_s": S / (ms * 1e-3), "flop": flops, "tflops": tf, "preheat_s": pre,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16_TFLOPS, "traffic": measured_traffic("prefill_sliding_s1024")}}


def w_chunk(ctx, steps, warmup, preheat_s):
    """A chunk of 8192 tokens after a cached prefix of 8192, batch 1, each layer type."""
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
    P = n = 8192
    ctx.gen.manual_seed(synth.SEED_FULL_S8192 + 100)
    q, k, v, g = (dev_normal(ctx.gen, (1, n, 16, 256)), dev_normal(ctx.gen, (1, n, 4, 256)),
                  dev_normal(ctx.gen, (1, n, 4, 256)), dev_normal(ctx.gen, (1, n, 16)))
    o = torch.empty_like(q)
    for lt, name in ((fga.FULL, "full"), (fga.SLIDING, "sliding")):
        cap = P + n if lt == fga.FULL else 512
        cache = fga.KVCache(lt, 1, cap, k=dev_normal(ctx.gen, (1, cap, 4, 256)), v=dev_normal(ctx.gen, (1, cap, 4, 256)))
        ws = torch.empty(fga.prefill_workspace_bytes(lt, 1, n), dtype=torch.uint8, device="cuda")
        ms, pre = time_launches(lambda: fga.prefill(lt, q, k, v, g, out=o, cache=cache, start_pos=P, workspace=ws),
                                100, 20, preheat_s)
        pairs = n * P + full_pairs(n) if lt == fga.FULL else n * 512
        tf = FLOP_PER_PAIR * pairs / (ms * 1e-3) / 1e12
        out[f"chunk_prefill_{name}_p8192_n8192"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                                    "tokens_per_s": n / (ms * 1e-3)}
        log(f"chunked prefill {name} P=8192 n=8192: {ms:.3f} ms  {tf:.0f} TFLOP/s")
        del cache, ws
    return out


def w_varlen(ctx, steps, warmup, preheat_s):
    """16 sequences of lengths uniform in [512, 8192], packed."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
    lens = np.random.default_rng(synth.SEED_FULL_S8192 + 200).integers(512, 8193, size=16)
    T = int(lens.sum())
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    ctx.gen.manual_seed(synth.SEED_FULL_S8192 + 201)
    q, k, v, g = (dev_normal(ctx.gen, (T, 16, 256)), dev_normal(ctx.gen, (T, 4, 256)),
                  dev_normal(ctx.gen, (T, 4, 256)), dev_normal(ctx.gen, (T, 16)))
    o = torch.empty_like(q)
    ws = torch.empty(fga.prefill_varlen_workspace_bytes(fga.FULL, T), dtype=torch.uint8, device="cuda")
    for lt, name in ((fga.FULL, "full"), (fga.SLIDING, "sliding")):
        ms, pre = time_launches(lambda: fga.prefill_varlen(lt, q, k, v, g, cu, int(lens.max()), out=o, workspace=ws),
                                50, 10, preheat_s)
        pairs = int(sum(full_pairs(int(x)) for x in lens)) if lt == fga.FULL else int(sum(sliding_pairs(int(x)) for x in lens))
        tf = FLOP_PER_PAIR * pairs / (ms * 1e-3) / 1e12
        out[f"varlen_prefill_{name}_16seq"] = {"ms": ms, "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                               "tokens_per_s": T / (ms * 1e-3), "tokens": T}
        log(f"varlen prefill {name}, 16 sequences (T={T}): {ms:.3f} ms  {tf:.0f} TFLOP/s")
    return out


def _decode_bytes(lt, lens, fga, row_bytes=4096):
    import numpy as np
    vis = np.minimum(lens, 512) if lt == fga.SLIDING else lens
    B = len(lens)
    return int(vis.astype(np.int64).sum()) * row_bytes + B * (16 * 256 * 4 + 32)


def decode_case(ctx, lt, B, lens, cap, seed, modes, preheat_s, check=None):
    """bf16 decode timed per call (median of 30): ``modes`` among "cold" (caches evicted
    before each call) and "warm"; ``check`` names the oracle run over every output."""
    import numpy as np
    import torch
    fga = ctx.fga
    lens = np.asarray(lens, dtype=np.int32)
    ctx.gen.manual_seed(seed)
    qd = dev_normal(ctx.gen, (B, 16, 256))
    gd = dev_normal(ctx.gen, (B, 16))
    cache = fga.KVCache(lt, B, cap, k=dev_normal(ctx.gen, (B, cap, 4, 256)), v=dev_normal(ctx.gen, (B, cap, 4, 256)))
    sl = torch.as_tensor(lens).cuda()
    maxlen = int(lens.max())
    wsd = torch.empty(fga.decode_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
    od = torch.empty_like(qd)
    call = lambda: fga.decode(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)
    nbytes = _decode_bytes(lt, lens, fga)
    res = {}
    for mode in modes:
        ms = time_each(call, 30, 5, preheat_s, ctx.flush if mode == "cold" else spin)
        res[mode] = {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes, "cache": mode}
    if ctx.cpu and check:
        import oracle
        call()
        torch.cuda.synchronize()
        got = f64_of(od)
        hq, hg = host_bits(qd), host_bits(gd)
        hk, hv = host_bits(cache.k), host_bits(cache.v)
        ctx.oracle_check(check, "every output (batch x 16 heads)",
                         lambda: oracle.decode(hq, hg, hk, hv, lens, lt), got, B * 16, "outputs")
        del hk, hv
    del cache
    torch.cuda.empty_cache()
    return res


def w_decode_b64(ctx, steps, warmup, preheat_s):
    """Batched decode, batch 64, lengths uniform in [1024, 32768]: the full layer back to
    back (the decode half of the headline) and per call cold; the sliding ring warm and cold."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
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
    od = torch.empty_like(q)
    ms, pre = time_launches(lambda: fga.decode(fga.FULL, q, gate, cache, sl, cap, out=od, workspace=ws),
                            max(steps, 100), warmup, preheat_s)
    nbytes = _decode_bytes(fga.FULL, lens, fga)
    gbs = nbytes / (ms * 1e-3) / 1e9
    ctx.decode_headline = {
        "workload": "batched decode, batch 64, context lengths uniform in [1024, 32768], full layer, bf16 KV "
                    "[ctx, 4, 256] (4.3 GB per call, far above the 256 MB MALL)",
        "value": gbs, "unit": "GB/s", "ms_per_step": ms, "bytes": nbytes, "preheat_s": pre,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("decode_full_b64")}}
    log(f"decode B=64 full (back to back): {ms * 1e3:.0f} us  {gbs:.0f} GB/s")
    del cache, ws
    torch.cuda.empty_cache()
    r = decode_case(ctx, fga.FULL, B, lens, cap, seed + 5, ("cold",), preheat_s, check="decode_b64_full")
    out["decode_b64_full_cold"] = r["cold"]
    log(f"decode B=64 full, cold: {r['cold']['us']:.0f} us  {r['cold']['gbs']:.0f} GB/s")
    r = decode_case(ctx, fga.SLIDING, B, lens, 512, seed + 1, ("warm", "cold"), preheat_s,
                    check="decode_b64_sliding")
    for mode in ("warm", "cold"):
        out[f"decode_b64_sliding_{mode}"] = r[mode]
        out[f"decode_b64_sliding_{mode}"]["traffic"] = measured_traffic("decode_sliding_b64")
        log(f"decode B=64 sliding ring, {mode}: {r[mode]['us']:.1f} us  {r[mode]['gbs']:.0f} GB/s")
    return out


def w_decode_long(ctx, steps, warmup, preheat_s):
    """Long decode: batch 4 at 131072 tokens and batch 1 at 2^20, full layer (capacity = L)
    and the sliding ring, cold."""
    out = {}
    fga, synth = ctx.fga, ctx.synth
    for B, L in ((4, 131072), (1, 1 << 20)):
        r = decode_case(ctx, fga.FULL, B, [L] * B, L, synth.SEED_LONG_DECODE + B, ("cold",), preheat_s,
                        check=f"decode_full_b{B}_l{L}")
        out[f"decode_full_b{B}_l{L}_cold"] = r["cold"]
        log(f"long decode full B={B} L={L}, cold: {r['cold']['us']:.0f} us  {r['cold']['gbs']:.0f} GB/s")
        r = decode_case(ctx, fga.SLIDING, B, [L] * B, 512, synth.SEED_LONG_DECODE + 10 + B, ("cold",), preheat_s,
                        check=f"decode_sliding_b{B}_l{L}")
        out[f"decode_sliding_b{B}_l{L}_cold"] = r["cold"]
        log(f"long decode sliding B={B} L={L}, cold: {r['cold']['us']:.1f} us")
    return out


def q8_cache(ctx, lt, B, cap):
    import torch
    fga = ctx.fga
    codes = lambda: torch.randint(-127, 128, (B, cap, 4, 256), generator=ctx.gen, device="cuda", dtype=torch.int8)
    scales = lambda: (0.005 + 0.025 * torch.rand((B, cap, 4, 8), generator=ctx.gen, device="cuda")).half()
    return fga.KVCacheQ8(lt, B, cap, k=codes(), k_scale=scales(), v=codes(), v_scale=scales())


def w_decode_q8(ctx, steps, warmup, preheat_s):
    """Decode over the 8-bit (q8_0) cache: 272 bytes per key row and KV head for K and V."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}

    def case(lt, B, lens, cap, seed):
        lens = np.asarray(lens, dtype=np.int32)
        ctx.gen.manual_seed(seed)
        qd = dev_normal(ctx.gen, (B, 16, 256))
        gd = dev_normal(ctx.gen, (B, 16))
        cache = q8_cache(ctx, lt, B, cap)
        sl = torch.as_tensor(lens).cuda()
        maxlen = int(lens.max())
        wsd = torch.empty(fga.decode_q8_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
        od = torch.empty_like(qd)
        call = lambda: fga.decode_q8(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)
        ms = time_each(call, 30, 5, preheat_s, ctx.flush)
        nbytes = _decode_bytes(lt, lens, fga, row_bytes=4 * 2 * 272)
        del cache
        torch.cuda.empty_cache()
        return {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes, "cache": "cold", "kv": "q8_0"}

    seed = synth.SEED_DECODE_B64
    lens = synth.decode_seq_lens(seed, 64, 1024, 32768)
    r = case(fga.FULL, 64, lens, 32768, seed + 50)
    out["decode_q8_b64_full_cold"] = r
    log(f"decode q8 B=64 full, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
    r = case(fga.SLIDING, 64, lens, 512, seed + 51)
    out["decode_q8_b64_sliding_cold"] = r
    log(f"decode q8 B=64 sliding ring, cold: {r['us']:.1f} us  {r['gbs']:.0f} GB/s")
    for B, L in ((4, 131072), (1, 1 << 20)):
        r = case(fga.FULL, B, [L] * B, L, synth.SEED_LONG_DECODE + 60 + B)
        out[f"decode_q8_full_b{B}_l{L}_cold"] = r
        log(f"long decode q8 full B={B} L={L}, cold: {r['us']:.0f} us  {r['gbs']:.0f} GB/s")
    return out


def w_decode_step(ctx, steps, warmup, preheat_s):
    """One decode step of all 36 layers: batch 64, lengths uniform in [1024, 32768] (9 full
    caches, 27 rings), bf16 and 8-bit caches."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
    ctx.drop_flush()
    torch.cuda.empty_cache()
    seed = synth.SEED_DECODE_B64
    lens = synth.decode_seq_lens(seed, 64, 1024, 32768)
    sl = torch.as_tensor(lens).cuda()
    maxlen = int(lens.max())
    B = 64
    for kv in ("bf16", "q8_0"):
        ctx.gen.manual_seed(seed + 300)
        layers = []
        for layer in range(36):
            lt = fga.layer_type_of(layer)
            cap = maxlen if lt == fga.FULL else 512
            if kv == "bf16":
                cache = fga.KVCache(lt, B, cap, k=dev_normal(ctx.gen, (B, cap, 4, 256)),
                                    v=dev_normal(ctx.gen, (B, cap, 4, 256)))
                wsb = fga.decode_workspace_bytes(lt, B, maxlen)
            else:
                cache = q8_cache(ctx, lt, B, cap)
                wsb = fga.decode_q8_workspace_bytes(lt, B, maxlen)
            layers.append((lt, cache, dev_normal(ctx.gen, (B, 16, 256)), dev_normal(ctx.gen, (B, 16)),
                           torch.empty(wsb, dtype=torch.uint8, device="cuda"),
                           torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")))
        dec = fga.decode if kv == "bf16" else fga.decode_q8

        def step():
            for lt, cache, qd, gd, wsd, od in layers:
                dec(lt, qd, gd, cache, sl, maxlen, out=od, workspace=wsd)

        ms, pre = time_launches(step, 10, 3, preheat_s)
        # The same step captured once in a HIP graph and replayed, as a serving loop would
        # (tests/test_gpu_graph.py checks that replays reproduce the eager calls bit for bit).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        ms_graph, _ = time_launches(graph.replay, 10, 3, preheat_s)
        vis = int(lens.astype(np.int64).sum()) * 9 + int(np.minimum(lens, 512).astype(np.int64).sum()) * 27
        row = 2 * 4 * (512 if kv == "bf16" else 272)
        nbytes = vis * row + 36 * B * (16 * 256 * 4 + 32)
        out[f"decode_step_36_layers_b64_{kv}"] = {"ms": ms, "tokens_per_s": B / (ms * 1e-3),
                                                  "gbs": nbytes / (ms * 1e-3) / 1e9,
                                                  "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                  "ms_graph": ms_graph, "tokens_per_s_graph": B / (ms_graph * 1e-3),
                                                  "frac_hbm_graph": nbytes / (ms_graph * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                  "bytes": nbytes, "kv": kv}
        log(f"36-layer decode step, batch 64 ({kv} cache): {ms:.2f} ms  {B / (ms * 1e-3):.0f} tokens/s  "
            f"{nbytes / (ms * 1e-3) / 1e9:.0f} GB/s; as a graph replay {ms_graph:.2f} ms")
        del graph, layers
        torch.cuda.empty_cache()
    return out


def w_append(ctx, steps, warmup, preheat_s):
    """KV append: 32768 tokens in bulk (batch 1; the ring keeps the last 512) and the one-token
    append of a batch-64 decode step at positions U[1024, 32768]; bf16 and 8-bit caches.
    Bytes per written token: its K and V read (2 x 2 KB) plus what the cache receives."""
    import numpy as np
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
    lens = synth.decode_seq_lens(synth.SEED_DECODE_B64, 64, 1024, 32768)
    for kv in ("bf16", "q8_0"):
        for lt, B, n in ((fga.FULL, 1, 32768), (fga.SLIDING, 1, 32768), (fga.FULL, 64, 1), (fga.SLIDING, 64, 1)):
            ctx.gen.manual_seed(synth.SEED_DECODE_B64 + 500 + B)
            cap = 512 if lt == fga.SLIDING else (32768 if B == 64 else n)
            k = dev_normal(ctx.gen, (B, n, 4, 256))
            v = dev_normal(ctx.gen, (B, n, 4, 256))
            pos = torch.as_tensor(lens - 1 if B == 64 else np.zeros(B, np.int32)).to(torch.int32).cuda()
            if kv == "bf16":
                cache = fga.KVCache(lt, B, cap)
                call = lambda: fga.kv_append(lt, k, v, pos, cache)
            else:
                cache = fga.KVCacheQ8(lt, B, cap)
                call = lambda: fga.kv_append_q8(lt, k, v, pos, cache)
            written = B * (min(n, 512) if lt == fga.SLIDING else n)
            row = 2 * 4 * (512 if kv == "bf16" else 272)
            nbytes = written * (2 * 4 * 512 + row)
            ms = time_each(call, 30, 5, preheat_s, spin)
            name = f"kv_append_{kv}_{'full' if lt == fga.FULL else 'sliding'}_b{B}_n{n}"
            out[name] = {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                         "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes}
            log(f"kv append ({kv}) {'full' if lt == fga.FULL else 'sliding'} B={B} n={n}: {ms * 1e3:.1f} us  "
                f"{nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
            del cache, k, v
    torch.cuda.empty_cache()
    return out


def w_proj(ctx, steps, warmup, preheat_s):
    """The W8A8 FP8 q/k/v projection with the bf16 gate projection upstream of the path:
    T tokens of hidden 2560 -> 6144 q/k/v channels (+ 16 gate logits)."""
    import torch
    fga, synth = ctx.fga, ctx.synth
    out = {}
    for T in (8192, 32768):
        ctx.gen.manual_seed(synth.SEED_SLIDING_S1024 + 400 + T)
        x = dev_normal(ctx.gen, (T, 2560))
        w = torch.randint(0x18, 0x50, (6144, 2560), generator=ctx.gen, device="cuda", dtype=torch.uint8)
        w = torch.where(torch.rand(w.shape, generator=ctx.gen, device="cuda") < 0.5, w, w | 0x80)
        wsc = 0.0025 + 0.0015 * torch.rand(6144, generator=ctx.gen, device="cuda")
        wg = (dev_normal(ctx.gen, (16, 2560)).float() / 64).to(torch.bfloat16)
        outs = (torch.empty(T, 16, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 4, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 4, 256, dtype=torch.bfloat16, device="cuda"),
                torch.empty(T, 16, dtype=torch.bfloat16, device="cuda"))
        wsp = torch.empty(fga.qkv_proj_fp8_workspace_bytes(T), dtype=torch.uint8, device="cuda")
        ms, pre = time_launches(lambda: fga.qkv_proj_fp8(x, w, wsc, wg, out=outs, workspace=wsp), 20, 5, preheat_s)
        flops = 2 * T * 2560 * 6144
        out[f"qkv_proj_fp8_t{T}"] = {"us": ms * 1e3, "tflops_fp8": flops / (ms * 1e-3) / 1e12,
                                     "frac_fp8_mfma": flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                                     "gate_gflops_bf16": 2 * T * 2560 * 16 / 1e9,
                                     "traffic": measured_traffic(f"qkv_proj_fp8_t{T}")}
        log(f"FP8 q/k/v + bf16 gate projection T={T}: {ms * 1e3:.0f} us  "
            f"{flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s (fp8 GEMM flops)")
        del x, w, wsc, wg, outs, wsp
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------ counters
def copy_calibration():
    """Device-to-device copy of 4 GiB: the plain copy of known size that scales the HBM
    traffic counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = 1 << 31                                   # bf16 elements: 4 GiB
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ms, _ = time_launches(lambda: y.copy_(x), 3, 1, 0.0)
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "ms": ms,
                      "read_plus_write_gbs": 4 * n / (ms * 1e-3) / 1e9}), flush=True)


def gemm_reference(preheat_s=1.0):
    """A square bf16 GEMM from the vendor library (torch.matmul, hipBLASLt) on the same box:
    what a dense bf16 MFMA workload reaches there, as context for the attention kernels'
    fraction of the published peak.  Not part of the path."""
    import torch
    out = {}
    for n in (8192, 16384):
        a = torch.randn(n, n, device="cuda").bfloat16()
        b = torch.randn(n, n, device="cuda").bfloat16()
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        ms, pre = time_launches(lambda: torch.matmul(a, b, out=c), 20, 5, preheat_s)
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        out[f"vendor_bf16_gemm_n{n}"] = {"ms": ms, "tflops": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS,
                                         "preheat_s": pre, "what": "torch.matmul (hipBLASLt), context only"}
        del a, b, c
    torch.cuda.empty_cache()
    return out


def w_gemm_ref(ctx, steps, warmup, preheat_s):
    r = gemm_reference(max(preheat_s, 0.5))
    log("vendor bf16 GEMM: " + ", ".join(f"{k} {v['tflops']:.0f} TFLOP/s" for k, v in r.items()))
    return r


def kernel_source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "full_gqa_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per launch recorded in profiles/traffic.json for ``key``, or None when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key)
    if not rec or rec.get("source_hash") != kernel_source_hash(rec["sources"]):
        return None
    return rec["hbm_bytes_per_launch"]


# ---------------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the headline stack")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--preheat", type=float, default=0.5,
                    help="seconds of back-to-back calls before every timed loop")
    ap.add_argument("--only", default=",".join(WORKLOADS),
                    help="comma-separated subset of: " + ", ".join(WORKLOADS))
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time a square bf16 GEMM of the vendor library (context for the MFMA fractions)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 4 GiB device copy used to scale traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is single-GPU; "
              "a multi-GPU run has nothing to launch", file=sys.stderr)
        sys.exit(2)
    only = [w for w in args.only.split(",") if w]
    bad = [w for w in only if w not in WORKLOADS]
    if bad:
        ap.error(f"unknown workloads {bad}")

    import torch
    import full_gqa_attention_amd as fga
    import synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_reference:
        print(json.dumps(gemm_reference()), flush=True)
        return
    ctx = Ctx(fga, synth, args)
    result = {
        "metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "36-layer attention stack prefill (27 sliding-window + 9 full layers, last "
                               "full), batch 1, seq 32768, 16 Q / 4 KV heads, head_dim 256, per-type RoPE, "
                               "sigmoid head gate, independent bf16 N(0,1) Q/K/V/gate per layer; attention only",
                   "batch": 1, "seq_len": 32768, "layers": 36},
    }
    fns = {"stack": w_stack, "full_s8192": w_full_s8192, "sliding_s1024": w_sliding_s1024, "chunk": w_chunk,
           "varlen": w_varlen, "decode_b64": w_decode_b64, "decode_long": w_decode_long,
           "decode_q8": w_decode_q8, "decode_step": w_decode_step, "append": w_append, "proj": w_proj,
           "gemm_ref": w_gemm_ref}
    configs = {}
    for name in WORKLOADS:
        if name not in only:
            continue
        log(f"{name} ...")
        r = fns[name](ctx, args.steps, args.warmup, args.preheat)
        if name == "stack":
            result["value"] = r["tokens_per_s"]
            result["ms_per_step"] = r["ms"]
            result["preheat_s"] = r["preheat_s"]
            result["roofline"] = {
                "bound": "mfma", "achieved": r["full_call_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": r["full_call_tflops"] / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic("prefill_full_s32768"),
                "kernel": "full-layer attention call at S=32768 (prefill_rope_kernel<1, true> + prefill_kernel<1, false>)",
                "flop_per_launch": r["full_flop_per_call"], "ms_per_launch": r["full_call_ms"]}
            configs["stack36_prefill_s32768"] = r
        elif name in ("full_s8192", "sliding_s1024"):
            configs[{"full_s8192": "full_prefill_s8192", "sliding_s1024": "sliding_prefill_s1024"}[name]] = r
        else:
            configs.update(r)
    if getattr(ctx, "decode_headline", None):
        result["decode"] = ctx.decode_headline
    result["configs"] = configs
    if ctx.cpu:
        info = host_info()
        cb = {"value": None, "unit": "tokens/s", "cores": info["threads_used"], "kind": "oracle"}
        if getattr(ctx, "stack_cpu", None):
            cb["value"] = ctx.stack_cpu["value"]
            cb["sample"] = ("fp64 NumPy oracle on 192 query rows (all 16 heads; rows 0, 1, 511, 512, 513, S/2, "
                            "S-1 and 185 uniformly random others) of layer 3 (full) and of layer 0 (sliding) of "
                            "the timed S=32768 stack, on the same inputs; stack tokens/s extrapolated as "
                            "1 / (9 t_full_row + 27 t_sliding_row)")
            cb["stack_layers"] = ctx.stack_cpu["layers"]
        cb.update({k: info[k] for k in ("affinity_cores", "blas_threads", "cpu_model")})
        cb["per_workload"] = ctx.oracle_runs
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
