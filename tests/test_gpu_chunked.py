"""Chunked prefill parity: a chunk that continues a cached prefix (start_pos > 0), the HIP
path through the C ABI against the fp64 oracle, plus the cache it leaves behind."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_cached_keys_close, assert_parity, bits_of, f64_of, note, to_dev

pytestmark = pytest.mark.gpu


def _capacity(lt, P, n):
    return oracle.WINDOW if lt == oracle.SLIDING else P + n + 3


def _case(seed, lt, B, P, n):
    """Chunk inputs and a cache whose every slot holds seeded finite bf16 values (the
    slots out of the chunk's reach too: they must not change the result)."""
    inp = synth.prefill_inputs(seed, B, n)
    cap = _capacity(lt, P, n)
    ck = synth.normal_bf16(seed + 1, 0, (B, cap, 4, 256))
    cv = synth.normal_bf16(seed + 1, 1, (B, cap, 4, 256))
    return inp, ck, cv


def _run(fga, lt, inp, ck, cv, P):
    import torch
    B, cap = ck.shape[0], ck.shape[1]
    cache = fga.KVCache(lt, B, cap, k=to_dev(ck), v=to_dev(cv))
    q, k, v, g = (to_dev(inp[x]) for x in ("q", "k", "v", "gate"))
    out = fga.prefill(lt, q, k, v, g, cache=cache, start_pos=P)
    torch.cuda.synchronize()
    return out, cache


def _check_cache(cache, ck, cv, inp, P, lt, what):
    B = ck.shape[0]
    wk, wv = oracle.kv_append(ck, cv, inp["k"], inp["v"], np.full(B, P, np.int32), lt)
    gv = bits_of(cache.v)
    assert np.array_equal(gv, wv), f"{what}: cached values differ at {np.argwhere(gv != wv)[:5].tolist()}"
    assert_cached_keys_close(bits_of(cache.k), wk, what)


CASES = [
    # (B, P, n): prefix length P, chunk length n
    (1, 1, 1), (1, 1, 64), (2, 37, 100), (1, 64, 65), (1, 300, 1), (2, 500, 300),
    (1, 511, 2), (1, 512, 33), (1, 600, 100), (2, 777, 512), (1, 1000, 1300), (1, 2049, 700),
]


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
@pytest.mark.parametrize("B,P,n", CASES, ids=[f"B{b}P{p}n{n}" for b, p, n in CASES])
def test_chunk_all_rows(fga, lt, B, P, n):
    what = f"chunk lt={lt} B={B} P={P} n={n}"
    note(what)
    seed = 5000 + 13 * P + 7 * n + B
    inp, ck, cv = _case(seed, lt, B, P, n)
    out, cache = _run(fga, lt, inp, ck, cv, P)
    want = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"], inp["gate"], ck, cv, P, lt)
    assert_parity(f64_of(out), want, what)
    _check_cache(cache, ck, cv, inp, P, lt, what)


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_chunk_8192_after_prefix_8192_sampled_rows(fga, lt):
    """Chunk of 8192 tokens after a cached prefix of 8192, batch 1: 128 sampled rows (the
    shape the benchmark times)."""
    P = n = 8192
    what = f"chunk lt={lt} P={P} n={n}"
    note(what)
    inp, ck, cv = _case(7100 + lt, lt, 1, P, n)
    out, cache = _run(fga, lt, inp, ck, cv, P)
    fixed = [0, 1, 31, 32, 510, 511, 512, 4096, n - 1]
    rows = np.unique(np.concatenate([fixed, np.random.default_rng(7101).choice(n, 119, replace=False)]))
    want = oracle.prefill_chunk(inp["q"], inp["k"], inp["v"], inp["gate"], ck, cv, P, lt, rows=rows)
    assert_parity(f64_of(out[:, rows]), want, what)
    _check_cache(cache, ck, cv, inp, P, lt, what)


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_chunks_equal_one_shot(fga, lt):
    """A context fed in chunks (through the cache) gives the one-shot prefill's output to
    the parity bar, and leaves the same cache bit for bit: the keys are rounded to bf16
    once, by the same rotation at the same position, either way.  (The outputs need not
    match bit for bit: a row's running softmax maximum moves whenever any row of its wave
    needs it to, and the chunks group rows into waves differently.)"""
    import torch
    B, S, cuts = 2, 2000, [0, 700, 701, 1500, 2000]
    inp = synth.prefill_inputs(7200 + lt, B, S)
    cap = _capacity(lt, 0, S)
    whole = fga.KVCache(lt, B, cap)
    q, k, v, g = (to_dev(inp[x]) for x in ("q", "k", "v", "gate"))
    ref = fga.prefill(lt, q, k, v, g, cache=whole)
    parts = fga.KVCache(lt, B, cap)
    got = torch.empty_like(ref)
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = slice(a, b)
        got[:, sl] = fga.prefill(lt, q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                 g[:, sl].contiguous(), cache=parts, start_pos=a)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(parts.k), bits_of(whole.k)), "cached keys differ"
    assert np.array_equal(bits_of(parts.v), bits_of(whole.v)), "cached values differ"
    ndiff = int((got.view(torch.int16) != ref.view(torch.int16)).sum())
    note(f"[chunked] lt={lt}: {ndiff} of {ref.numel()} outputs differ from one-shot in their bits")
    assert_parity(f64_of(got), f64_of(ref), f"chunked vs one-shot lt={lt}")
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=np.array([0, 699, 700, 701, 1999]))
    assert_parity(f64_of(got[:, [0, 699, 700, 701, 1999]]), want, f"chunked lt={lt} vs oracle")


def test_chunk_then_decode(fga):
    """Prefill in two chunks, then decode the next token from the cache they left; checked
    against the oracle's decode over the same context."""
    import torch
    B, S = 1, 900
    for lt in (oracle.SLIDING, oracle.FULL):
        note(f"chunk then decode lt={lt}")
        inp = synth.prefill_inputs(7300 + lt, B, S + 1)
        cap = _capacity(lt, 0, S + 1)
        cache = fga.KVCache(lt, B, cap)
        q, k, v, g = (to_dev(inp[x]) for x in ("q", "k", "v", "gate"))
        fga.prefill(lt, q[:, :600].contiguous(), k[:, :600].contiguous(), v[:, :600].contiguous(),
                    g[:, :600].contiguous(), cache=cache)
        fga.prefill(lt, q[:, 600:S].contiguous(), k[:, 600:S].contiguous(), v[:, 600:S].contiguous(),
                    g[:, 600:S].contiguous(), cache=cache, start_pos=600)
        pos = torch.full((B,), S, dtype=torch.int32, device="cuda")
        fga.kv_append(lt, k[:, S:].contiguous(), v[:, S:].contiguous(), pos, cache)
        lens = torch.full((B,), S + 1, dtype=torch.int32, device="cuda")
        out = fga.decode(lt, q[:, S].contiguous(), g[:, S].contiguous(), cache, lens, S + 1)
        torch.cuda.synchronize()
        want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=np.array([S]))
        assert_parity(f64_of(out), want[:, 0], f"chunk+decode lt={lt}")
