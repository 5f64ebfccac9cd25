"""Prefill parity: the HIP path through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, f64_of, note, to_dev

pytestmark = pytest.mark.gpu


def _run(fga, inp, lt, cache=None):
    import torch
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    out = fga.prefill(lt, q, k, v, g, cache=cache)
    torch.cuda.synchronize()
    return out


# Sliding layers without a prefix take the split-band kernel while batch x ceil(S/64) x 4 < 256
# (B3 S1300: 252 blocks; B1 S4032: 252) and the 64-row kernel from 256 on (B4 S1000, B1 S4033).
# The split kernel's workgroups take 2 query heads up to B1 S1024 and at B2 S1100 (280
# four-head workgroups: 2 rounds of 256 CUs against 3 for the 2-head form), 4 at B3 S1300
# and B1 S4032 (492 and 504: 2 rounds against 4).
SMALL = [(1, 1), (1, 2), (2, 63), (1, 64), (1, 65), (2, 100), (1, 511), (1, 512), (1, 513),
         (1, 700), (2, 1100), (3, 1300), (4, 1000), (1, 4032), (1, 4033)]


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
@pytest.mark.parametrize("B,S", SMALL, ids=[f"B{b}S{s}" for b, s in SMALL])
def test_prefill_small_all_rows(fga, lt, B, S):
    note(f"prefill lt={lt} B={B} S={S}")
    inp = synth.prefill_inputs(1000 + 7 * S + B, B, S)
    got = f64_of(_run(fga, inp, lt))
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt)
    assert_parity(got, want, f"prefill lt={lt} B={B} S={S}")


def test_sliding_s1024_all_rows(fga):
    """Single sliding-window layer, batch 1, S=1024, theta 1e4 over all 256 dims."""
    inp = synth.prefill_inputs(synth.SEED_SLIDING_S1024, 1, 1024)
    got = f64_of(_run(fga, inp, oracle.SLIDING))
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], oracle.SLIDING)
    assert_parity(got, want, "sliding S=1024")


def _sample_rows(S, seed, n_random):
    fixed = [0, 1, 63, 64, 511, 512, 513, S // 2, S - 1]
    rnd = np.random.default_rng(seed).choice(S, size=n_random, replace=False)
    return np.unique(np.concatenate([fixed, rnd]))


@pytest.mark.timeout(900)
def test_full_s8192_all_rows(fga):
    """Single full layer, batch 1, S=8192, theta 5e6 on the first 64 dims: every row."""
    S = 8192
    inp = synth.prefill_inputs(synth.SEED_FULL_S8192, 1, S)
    got = f64_of(_run(fga, inp, oracle.FULL))
    note("full S=8192: oracle over all 8192 rows")
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], oracle.FULL)
    assert_parity(got, want, "full S=8192 all rows")


@pytest.mark.parametrize("layer", list(range(36)))
def test_stack_layer_s32768_sampled_rows(fga, layer):
    """36-layer stack, batch 1, S=32768, independent inputs per layer: 64 sampled rows each."""
    S = 32768
    lt = oracle.layer_type_of(layer)
    note(f"stack layer {layer} lt={lt}")
    inp = synth.prefill_inputs(synth.stack_layer_seed(layer), 1, S)
    got = _run(fga, inp, lt)
    rows = _sample_rows(S, synth.stack_layer_seed(layer) + 1, 55)
    got = f64_of(got[:, rows])
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=rows)
    assert_parity(got, want, f"stack S=32768 layer {layer} lt={lt}")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
@pytest.mark.parametrize("S", [37, 512, 700])
def test_prefill_writes_cache(fga, lt, S):
    """With a cache the prefill stores the rotated keys and the values like kv_append."""
    B = 2
    inp = synth.prefill_inputs(3000 + S, B, S)
    cap = 512 if lt == oracle.SLIDING else S + 5
    cache = fga.KVCache(lt, B, cap)
    out = _run(fga, inp, lt, cache=cache)
    ck0 = np.zeros((B, cap, 4, 256), np.uint16)
    ck, cv = oracle.kv_append(ck0, ck0.copy(), inp["k"], inp["v"], np.zeros(B, np.int32), lt)
    from gpu_util import assert_cached_keys_close, bits_of
    gv = bits_of(cache.v)
    assert np.array_equal(gv, cv), f"cached values differ at {np.argwhere(gv != cv)[:5].tolist()}"
    assert_cached_keys_close(bits_of(cache.k), ck, f"prefill cache lt={lt} S={S}")
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt)
    assert_parity(f64_of(out), want, f"prefill+cache lt={lt} S={S}")


@pytest.mark.parametrize("B,S", [(1, 1024), (2, 1100), (1, 4032)], ids=["B1S1024", "B2S1100", "B1S4032"])
def test_short_sliding_prefill_is_deterministic(fga, B, S):
    """Short sliding layers run with the key band split over two wave groups whose states
    meet in LDS, in workgroups of 2 query heads (B1S1024, B2S1100) or 4 (B1S4032):
    repeated calls are bit-identical (fresh NaN-filled buffers each call)."""
    import torch
    inp = synth.prefill_inputs(4343 + S, B, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    ref = fga.prefill(oracle.SLIDING, q, k, v, g).view(torch.int16).clone()
    for rep in range(8):
        out = fga.prefill(oracle.SLIDING, q, k, v, g).view(torch.int16)
        ndiff = int((out != ref).sum())
        assert ndiff == 0, f"call {rep + 1}: {ndiff} output elements differ from the first call"


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_prefill_is_deterministic(fga, lt):
    """Repeated calls on the same inputs give bit-identical outputs (no race between the
    waves of a workgroup or between an MFMA and the instructions that read its result).
    Every call writes a fresh NaN-filled output through a fresh NaN-filled workspace, so
    a skipped element cannot pass as an earlier call's result."""
    import torch
    S = 8192
    inp = synth.prefill_inputs(4242 + lt, 1, S)
    q, k, v, g = (to_dev(inp[n]) for n in ("q", "k", "v", "gate"))
    ref = fga.prefill(lt, q, k, v, g).view(torch.int16).clone()
    for rep in range(8):
        out = fga.prefill(lt, q, k, v, g).view(torch.int16)
        ndiff = int((out != ref).sum())
        assert ndiff == 0, f"call {rep + 1}: {ndiff} output elements differ from the first call"


def test_prefill_rejects_bad_arguments(fga):
    import torch
    q = torch.zeros(1, 8, 16, 256, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 8, 4, 256, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 8, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fga.SparkError) as e:      # a prefix is read from a cache
        fga.prefill(oracle.FULL, q, k, k, g, start_pos=3)
    assert e.value.status == 1
    with pytest.raises(fga.SparkError) as e:      # capacity < start_pos + seq_len
        fga.prefill(oracle.FULL, q, k, k, g, cache=fga.KVCache(oracle.FULL, 1, 10), start_pos=3)
    assert e.value.status == 1
    cache = fga.KVCache(oracle.FULL, 1, 4)
    with pytest.raises(fga.SparkError) as e:
        fga.prefill(oracle.FULL, q, k, k, g, cache=cache)
    assert e.value.status == 1
