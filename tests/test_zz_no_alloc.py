"""spark_attn_decode_noalloc: the decode entry point that allocates nothing (its partial
results in the library's static device scratch), through the C ABI, against
spark_attn_decode on the same inputs and against the oracle; two calls in a row, the
second smaller, so that the second reads a scratch the first left full."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, bits_of, f64_of, i32_dev, note, to_dev
from guarded import Framed

pytestmark = pytest.mark.gpu


def _case(fga, lt, seed, lens):
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    d = synth.decode_inputs(seed, B, int(lens.max()), fill_lens=lens)
    if lt == oracle.SLIDING:     # the ring: positions max(0, L-512)..L-1 in slot p mod 512
        ck = np.zeros((B, 512, 4, 256), np.uint16)
        cv = np.zeros_like(ck)
        for b in range(B):
            p = np.arange(max(0, int(lens[b]) - 512), int(lens[b]))
            ck[b, p % 512] = d["cache_k"][b, p]
            cv[b, p % 512] = d["cache_v"][b, p]
        d["cache_k"], d["cache_v"] = ck, cv
    cache = fga.KVCache(lt, B, d["cache_k"].shape[1], k=to_dev(d["cache_k"]), v=to_dev(d["cache_v"]))
    return d, cache, lens


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_noalloc_matches_decode_twice(fga, lt):
    import torch
    first = ([3000, 1500, 33, 4000, 512, 9000, 1, 700], 0)    # (lengths, num_parts)
    second = ([1200, 17, 600], 5)
    for i, (lens, parts) in enumerate((first, second)):
        d, cache, lens = _case(fga, lt, 7100 + 10 * i + lt, lens)
        q, g, L = to_dev(d["q"]), to_dev(d["gate"]), i32_dev(lens)
        want_dev = fga.decode(lt, q, g, cache, L, int(lens.max()), num_parts=parts)
        out = Framed(q.shape, torch.bfloat16)
        note(f"decode_noalloc lt={lt} call {i + 1}: B={len(lens)} parts={parts}")
        got = fga.decode_noalloc(lt, q, g, cache, L, int(lens.max()), out=out.t, num_parts=parts)
        torch.cuda.synchronize()
        out.check_guards("decode_noalloc out")
        out.check_written("decode_noalloc out")
        assert np.array_equal(bits_of(got), bits_of(want_dev)), "differs from spark_attn_decode"
        want = oracle.decode(d["q"], d["gate"], d["cache_k"], d["cache_v"], lens, lt)
        assert_parity(f64_of(got), want, f"decode_noalloc lt={lt} call {i + 1}")


def test_noalloc_batch_64_full(fga):
    """Batch 64 at lengths uniform in [1024, 32768] (about 5 MiB of scratch), cache drawn on
    the device: bit for bit the output of spark_attn_decode, on two calls in a row."""
    import torch
    seed = synth.SEED_DECODE_B64 + 21
    B, cap = 64, 32768
    lens = synth.decode_seq_lens(seed, B, 1024, cap)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
    cache = fga.KVCache(oracle.FULL, B, cap, k=rnd(B, cap, 4, 256), v=rnd(B, cap, 4, 256))
    q, g, L = rnd(B, 16, 256), rnd(B, 16), i32_dev(lens)
    ref = fga.decode(oracle.FULL, q, g, cache, L, cap)
    for rep in range(2):
        got = fga.decode_noalloc(oracle.FULL, q, g, cache, L, cap)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(got), bits_of(ref)), f"call {rep + 1} differs from spark_attn_decode"


def test_noalloc_rejects_beyond_scratch(fga):
    import torch
    B, cap = 1000, 64           # (256 + 1000) partial results of 16.5 KB: over 16 MiB
    assert fga.decode_workspace_bytes(oracle.FULL, B, cap, 0) > fga.NOALLOC_SCRATCH_BYTES
    cache = fga.KVCache(oracle.FULL, B, cap)
    q = torch.zeros(B, 16, 256, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(B, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fga.SparkError) as e:
        fga.decode_noalloc(oracle.FULL, q, g, cache, i32_dev(np.full(B, cap)), cap)
    assert e.value.status == 3
