"""Variable-length batched prefill: the HIP path through the C ABI against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_cached_keys_close, assert_parity, bits_of, f64_of, i32_dev, note, to_dev

pytestmark = pytest.mark.gpu


def _packed(seed, lens):
    T = int(sum(lens))
    inp = synth.prefill_inputs(seed, 1, T)
    return {n: a[0] for n, a in inp.items()}, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _run(fga, lt, x, cu, max_len, cache=None):
    import torch
    out = fga.prefill_varlen(lt, to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["gate"]),
                             i32_dev(cu), max_len, cache=cache)
    torch.cuda.synchronize()
    return out


MIXES = [[1], [63, 64, 65], [700, 0, 1, 1100, 33], [513, 2, 512, 1000]]


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
@pytest.mark.parametrize("lens", MIXES, ids=["L" + "-".join(map(str, m)) for m in MIXES])
def test_varlen_all_rows(fga, lt, lens):
    what = f"varlen lt={lt} lens={lens}"
    note(what)
    x, cu = _packed(8000 + sum(lens) + lt, lens)
    got = f64_of(_run(fga, lt, x, cu, max(lens)))
    want = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["gate"], cu, lt)
    assert_parity(got, want, what)


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_varlen_equals_single_sequence_calls(fga, lt):
    """Each sequence's rows are those of a batch-1 prefill of that sequence.  Full layers:
    bit for bit (the same tiles in the same order, only the row offsets differ).  Sliding
    layers: a batch-1 call this short splits each key band over two wave groups and merges
    them, so the rounding differs; the rows must agree to the parity bar."""
    import torch
    lens = [700, 0, 1, 1100, 33, 64]
    x, cu = _packed(8100 + lt, lens)
    got = bits_of(_run(fga, lt, x, cu, max(lens), ))
    for b, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(int(cu[b]), int(cu[b + 1]))
        one = fga.prefill(lt, *(to_dev(x[k][sl][None]) for k in ("q", "k", "v", "gate")))
        torch.cuda.synchronize()
        ref = bits_of(one)[0]
        if lt == oracle.FULL:
            nd = int((got[sl] != ref).sum())
            assert nd == 0, f"sequence {b}: {nd} output elements differ from its batch-1 call"
        else:
            f = lambda u: (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
            assert_parity(f(got[sl]), f(ref), f"sequence {b} against its batch-1 call")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_varlen_writes_cache(fga, lt):
    """With a cache, row b receives sequence b's rotated keys and values (the last 512 on
    a ring); rows of empty sequences are left alone."""
    lens = [37, 0, 700, 512]
    x, cu = _packed(8200 + lt, lens)
    B = len(lens)
    cap = 512 if lt == oracle.SLIDING else max(lens) + 3
    cache = fga.KVCache(lt, B, cap)
    out = _run(fga, lt, x, cu, max(lens), cache=cache)
    ck = np.zeros((B, cap, 4, 256), np.uint16)
    cv = np.zeros_like(ck)
    for b, n in enumerate(lens):
        if n:
            sl = slice(int(cu[b]), int(cu[b + 1]))
            kb, vb = oracle.kv_append(ck[b:b + 1], cv[b:b + 1], x["k"][sl][None], x["v"][sl][None],
                                      np.zeros(1, np.int32), lt)
            ck[b], cv[b] = kb[0], vb[0]
    gv = bits_of(cache.v)
    assert np.array_equal(gv, cv), f"cached values differ at {np.argwhere(gv != cv)[:5].tolist()}"
    assert_cached_keys_close(bits_of(cache.k), ck, f"varlen cache lt={lt}")
    want = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["gate"], cu, lt)
    assert_parity(f64_of(out), want, f"varlen+cache lt={lt}")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_varlen_length_mix_sampled_rows(fga, lt):
    """Sixteen sequences of lengths uniform in [1, 8192]: 24 sampled rows per sequence
    (its first and last rows, and rows 511, 512 where present)."""
    rng = np.random.default_rng(8300 + lt)
    lens = rng.integers(1, 8193, size=16).tolist()
    x, cu = _packed(8301 + lt, lens)
    note(f"varlen mix lt={lt} T={int(cu[-1])}")
    got = _run(fga, lt, x, cu, max(lens))
    rows = []
    for b, n in enumerate(lens):
        pick = {0, n - 1} | {r for r in (511, 512) if r < n}
        pick |= set(rng.choice(n, size=min(n, 20), replace=False).tolist())
        rows += [int(cu[b]) + r for r in sorted(pick)]
    rows = np.array(rows)
    want = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["gate"], cu, lt, rows=rows)
    assert_parity(f64_of(got[rows]), want, f"varlen mix lt={lt}")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_varlen_benchmark_mix_sampled_rows(fga, lt):
    """The benchmark's batch: sixteen sequences of lengths uniform in [512, 8192] (the same
    draw), 12 sampled rows per sequence, first and last included."""
    lens = np.random.default_rng(synth.SEED_FULL_S8192 + 200).integers(512, 8193, size=16).tolist()
    x, cu = _packed(8400 + lt, lens)
    note(f"varlen benchmark mix lt={lt} T={int(cu[-1])}")
    got = _run(fga, lt, x, cu, max(lens))
    rng = np.random.default_rng(8401 + lt)
    rows = []
    for b, n in enumerate(lens):
        pick = {0, n - 1} | set(rng.choice(n, size=10, replace=False).tolist())
        rows += [int(cu[b]) + r for r in sorted(pick)]
    rows = np.array(rows)
    want = oracle.prefill_varlen(x["q"], x["k"], x["v"], x["gate"], cu, lt, rows=rows)
    assert_parity(f64_of(got[rows]), want, f"varlen benchmark mix lt={lt}")
