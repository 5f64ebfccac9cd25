"""Decode and KV-append parity: the HIP path through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_cached_keys_close, assert_parity, bits_of, f64_of, i32_dev, note, to_dev

pytestmark = pytest.mark.gpu


def _ring_from_contiguous(ck, cv, lens):
    """Ring caches holding positions max(0, L-512)..L-1 of contiguous caches, in slot p mod 512."""
    B = ck.shape[0]
    rk = np.zeros((B, 512, 4, 256), np.uint16)
    rv = np.zeros_like(rk)
    for b in range(B):
        L = int(lens[b])
        p = np.arange(max(0, L - 512), L)
        rk[b, p % 512] = ck[b, p]
        rv[b, p % 512] = cv[b, p]
    return rk, rv


def _decode_dev(fga, lt, d, ck, cv, lens, num_parts=0, max_len=None):
    import torch
    B = len(lens)
    cap = ck.shape[1]
    cache = fga.KVCache(lt, B, cap, k=to_dev(ck), v=to_dev(cv))
    out = fga.decode(lt, to_dev(d["q"]), to_dev(d["gate"]), cache, i32_dev(lens),
                     max(1, int(max(lens))) if max_len is None else max_len, num_parts=num_parts)
    torch.cuda.synchronize()
    return f64_of(out)


EDGE = [[1], [5], [511], [512], [513], [1, 37, 600, 1025], [4097, 64, 2000]]


@pytest.mark.parametrize("lens", EDGE, ids=["L" + "-".join(map(str, x)) for x in EDGE])
@pytest.mark.parametrize("num_parts", [0, 1, 3, 64, 5000])
def test_decode_edges_both_types(fga, lens, num_parts):
    """Partition counts from one workgroup for the whole batch to far more workgroups than
    32-key chunks (most then hold no chunk), so partitions start and end mid-sequence, at
    sequence boundaries and inside ragged last chunks."""
    lens = np.array(lens, np.int32)
    B, cap = len(lens), int(lens.max())
    d = synth.decode_inputs(4000 + int(lens.sum()), B, cap, fill_lens=lens)
    note(f"decode edges lens={lens.tolist()} parts={num_parts}")
    got = _decode_dev(fga, oracle.FULL, d, d["cache_k"], d["cache_v"], lens, num_parts)
    want = oracle.decode(d["q"], d["gate"], d["cache_k"], d["cache_v"], lens, oracle.FULL)
    assert_parity(got, want, f"decode full lens={lens.tolist()} parts={num_parts}")
    rk, rv = _ring_from_contiguous(d["cache_k"], d["cache_v"], lens)
    got = _decode_dev(fga, oracle.SLIDING, d, rk, rv, lens, num_parts)
    want = oracle.decode(d["q"], d["gate"], rk, rv, lens, oracle.SLIDING)
    assert_parity(got, want, f"decode sliding lens={lens.tolist()} parts={num_parts}")


def test_partition_count_does_not_change_result(fga):
    lens = np.array([3000, 1500, 33, 4000], np.int32)
    d = synth.decode_inputs(4100, 4, 4000, fill_lens=lens)
    outs = [_decode_dev(fga, oracle.FULL, d, d["cache_k"], d["cache_v"], lens, p)
            for p in (1, 7, 256, 2048)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 4e-3


@pytest.mark.parametrize("num_parts", [0, 2, 40])
def test_decode_zero_length_sequences(fga, num_parts):
    """A sequence with L = 0 sees no key and gets a zero output; its neighbours are unaffected."""
    lens = np.array([0, 70, 0, 0, 33, 0], np.int32)
    B, cap = len(lens), 128
    d = synth.decode_inputs(4200, B, cap, fill_lens=lens)
    got = _decode_dev(fga, oracle.FULL, d, d["cache_k"], d["cache_v"], lens, num_parts, max_len=cap)
    live = lens > 0
    assert np.all(got[~live] == 0.0)
    want = oracle.decode(d["q"][live], d["gate"][live], d["cache_k"][live], d["cache_v"][live],
                         lens[live], oracle.FULL)
    assert_parity(got[live], want, f"decode with empty sequences parts={num_parts}")


def test_batched_decode_b64(fga):
    """Batch 64, context lengths uniform in [1024, 32768]; full cache and 512-slot ring."""
    import torch
    seed = synth.SEED_DECODE_B64
    B, cap = 64, 32768
    lens = synth.decode_seq_lens(seed, B, 1024, 32768)
    note(f"decode B=64 lens sum={int(lens.sum())}")
    q = synth.normal_bf16(seed, 0, (B, 16, 256))
    gate = synth.normal_bf16(seed, 1, (B, 16))
    cache = fga.KVCache(oracle.FULL, B, cap)
    host_k = np.zeros((B, cap, 4, 256), np.uint16)
    host_v = np.zeros_like(host_k)
    for b in range(B):
        kb, vb = synth.cache_rows(seed, b, int(lens[b]))
        host_k[b, :lens[b]], host_v[b, :lens[b]] = kb, vb
        cache.k[b, :lens[b]] = to_dev(kb)
        cache.v[b, :lens[b]] = to_dev(vb)
    out = fga.decode(oracle.FULL, to_dev(q), to_dev(gate), cache, i32_dev(lens), cap)
    torch.cuda.synchronize()
    want = oracle.decode(q, gate, host_k, host_v, lens, oracle.FULL)
    assert_parity(f64_of(out), want, "decode B=64 full")
    rk, rv = _ring_from_contiguous(host_k, host_v, lens)
    del cache
    ring = fga.KVCache(oracle.SLIDING, B, 512, k=to_dev(rk), v=to_dev(rv))
    out = fga.decode(oracle.SLIDING, to_dev(q), to_dev(gate), ring, i32_dev(lens), cap)
    torch.cuda.synchronize()
    want = oracle.decode(q, gate, rk, rv, lens, oracle.SLIDING)
    assert_parity(f64_of(out), want, "decode B=64 sliding")


@pytest.mark.parametrize("B,L", [(4, 131072), (1, 1048576)], ids=["B4_L131072", "B1_L1048576"])
def test_long_decode(fga, B, L):
    """Long-context decode on a full layer (cache capacity = L) and on the sliding ring."""
    import torch
    seed = synth.SEED_LONG_DECODE + B
    lens = np.full(B, L, np.int32)
    q = synth.normal_bf16(seed, 0, (B, 16, 256))
    gate = synth.normal_bf16(seed, 1, (B, 16))
    cache = fga.KVCache(oracle.FULL, B, L)
    host_k = np.zeros((B, L, 4, 256), np.uint16)
    host_v = np.zeros_like(host_k)
    for b in range(B):
        host_k[b], host_v[b] = synth.cache_rows(seed, b, L)
        cache.k[b] = to_dev(host_k[b])
        cache.v[b] = to_dev(host_v[b])
    note(f"long decode B={B} L={L} uploaded")
    out = fga.decode(oracle.FULL, to_dev(q), to_dev(gate), cache, i32_dev(lens), L)
    torch.cuda.synchronize()
    want = oracle.decode(q, gate, host_k, host_v, lens, oracle.FULL)
    assert_parity(f64_of(out), want, f"long decode full B={B} L={L}")
    rk, rv = _ring_from_contiguous(host_k, host_v, lens)
    del cache
    ring = fga.KVCache(oracle.SLIDING, B, 512, k=to_dev(rk), v=to_dev(rv))
    out = fga.decode(oracle.SLIDING, to_dev(q), to_dev(gate), ring, i32_dev(lens), L)
    torch.cuda.synchronize()
    want = oracle.decode(q, gate, rk, rv, lens, oracle.SLIDING)
    assert_parity(f64_of(out), want, f"long decode sliding B={B} L={L}")


APPEND = [(oracle.FULL, 1, [0, 7]), (oracle.FULL, 33, [0, 100]), (oracle.SLIDING, 5, [0, 1000]),
          (oracle.SLIDING, 600, [100, 0]), (oracle.SLIDING, 512, [3, 512])]


@pytest.mark.parametrize("lt,n_new,pos", APPEND, ids=[f"lt{a}_n{b}_p{c[0]}" for a, b, c in APPEND])
def test_kv_append(fga, lt, n_new, pos):
    import torch
    B = len(pos)
    cap = 512 if lt == oracle.SLIDING else max(pos) + n_new + 3
    ck0 = synth.normal_bf16(4200 + n_new, 0, (B, cap, 4, 256))
    cv0 = synth.normal_bf16(4200 + n_new, 1, (B, cap, 4, 256))
    k = synth.normal_bf16(4200 + n_new, 2, (B, n_new, 4, 256))
    v = synth.normal_bf16(4200 + n_new, 3, (B, n_new, 4, 256))
    cache = fga.KVCache(lt, B, cap, k=to_dev(ck0), v=to_dev(cv0))
    fga.kv_append(lt, to_dev(k), to_dev(v), i32_dev(pos), cache)
    torch.cuda.synchronize()
    ck, cv = oracle.kv_append(ck0, cv0, k, v, np.array(pos), lt)
    gv = bits_of(cache.v)
    assert np.array_equal(gv, cv), f"values/untouched slots differ at {np.argwhere(gv != cv)[:5].tolist()}"
    assert_cached_keys_close(bits_of(cache.k), ck, f"append lt={lt} n={n_new} pos={pos}")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_prefill_then_decode_consistency(fga, lt):
    """Prefill S tokens into the cache, append token S, decode it: equals oracle prefill row S."""
    import torch
    S = 777
    inp = synth.prefill_inputs(4300, 1, S + 1)
    cap = 512 if lt == oracle.SLIDING else S + 1
    cache = fga.KVCache(lt, 1, cap)
    pre = {n: inp[n][:, :S] for n in inp}
    fga.prefill(lt, to_dev(pre["q"]), to_dev(pre["k"]), to_dev(pre["v"]), to_dev(pre["gate"]), cache=cache)
    fga.kv_append(lt, to_dev(inp["k"][:, S:]), to_dev(inp["v"][:, S:]), i32_dev([S]), cache)
    out = fga.decode(lt, to_dev(inp["q"][:, S]), to_dev(inp["gate"][:, S]), cache, i32_dev([S + 1]), S + 1)
    torch.cuda.synchronize()
    want = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=[S])[:, 0]
    assert_parity(f64_of(out), want, f"prefill->append->decode lt={lt}")


@pytest.mark.parametrize("num_parts", [0, 7, 4000])
def test_decode_batch_beyond_plan_threads(fga, num_parts):
    """A batch of 1500 sequences (more than the plan's 1024 threads, so each thread owns two)
    with lengths 0..64, some empty: every partition must find its first sequence."""
    B, cap = 1500, 64
    lens = np.random.default_rng(77).integers(0, cap + 1, size=B).astype(np.int32)
    lens[::97] = 0
    d = synth.decode_inputs(6060, B, cap, fill_lens=lens)
    note(f"decode B={B} parts={num_parts}")
    got = _decode_dev(fga, oracle.FULL, d, d["cache_k"], d["cache_v"], lens, num_parts, max_len=cap)
    live = lens > 0
    want = oracle.decode(d["q"][live], d["gate"][live], d["cache_k"][live], d["cache_v"][live],
                         lens[live], oracle.FULL)
    assert_parity(got[live], want, f"decode B={B} parts={num_parts}")
    assert np.all(got[~live] == 0.0)


RING_LENS = [0, 1, 5, 31, 32, 33, 255, 256, 257, 480, 511, 512, 513, 700, 1000, 2049, 17, 300, 64, 96]


@pytest.mark.parametrize("B", [15, 16, 20])
def test_sliding_ring_batch_edges(fga, B):
    """Batches of 15, 16 and 20 on a sliding layer (split + merge below batch 16, the
    one-launch ring kernel from 16 on): an empty sequence, ragged chunks, waves whose second
    chunk is empty, partly filled and full, and rings holding more positions than the window."""
    lens = np.array(RING_LENS[:B], np.int32)
    d = synth.decode_inputs(4400, B, int(lens.max()), fill_lens=lens)
    rk, rv = _ring_from_contiguous(d["cache_k"], d["cache_v"], lens)
    got = _decode_dev(fga, oracle.SLIDING, d, rk, rv, lens)
    live = lens > 0
    assert np.all(got[~live] == 0.0)
    want = oracle.decode(d["q"][live], d["gate"][live], rk[live], rv[live], lens[live], oracle.SLIDING)
    assert_parity(got[live], want, f"decode sliding ring, batch {B} of edge lengths")


def test_sliding_ring_is_deterministic(fga):
    """Repeated ring-kernel calls at batch 64 give bit-identical outputs (fresh NaN-filled
    outputs each call): the 8 waves' states meet in LDS behind one barrier."""
    import torch
    B = 64
    lens = synth.decode_seq_lens(4500, B, 1024, 32768)
    rk = synth.normal_bf16(4500, 0, (B, 512, 4, 256))
    rv = synth.normal_bf16(4500, 1, (B, 512, 4, 256))
    cache = fga.KVCache(oracle.SLIDING, B, 512, k=to_dev(rk), v=to_dev(rv))
    q = to_dev(synth.normal_bf16(4500, 2, (B, 16, 256)))
    g = to_dev(synth.normal_bf16(4500, 3, (B, 16)))
    L = i32_dev(lens)
    ref = fga.decode(oracle.SLIDING, q, g, cache, L, int(lens.max())).view(torch.int16).clone()
    for rep in range(8):
        out = fga.decode(oracle.SLIDING, q, g, cache, L, int(lens.max())).view(torch.int16)
        ndiff = int((out != ref).sum())
        assert ndiff == 0, f"call {rep + 1}: {ndiff} output elements differ from the first call"


def test_decode_is_deterministic(fga):
    """Repeated decode calls on the same cache give bit-identical outputs."""
    import torch
    lens = np.array([3000, 1500, 33, 4000, 512, 9000], np.int32)
    B, cap = len(lens), int(lens.max())
    d = synth.decode_inputs(5151, B, cap, fill_lens=lens)
    cache = fga.KVCache(oracle.FULL, B, cap, k=to_dev(d["cache_k"]), v=to_dev(d["cache_v"]))
    q, g, L = to_dev(d["q"]), to_dev(d["gate"]), i32_dev(lens)
    ref = fga.decode(oracle.FULL, q, g, cache, L, cap).view(torch.int16).clone()
    for rep in range(8):
        out = fga.decode(oracle.FULL, q, g, cache, L, cap).view(torch.int16)
        ndiff = int((out != ref).sum())
        assert ndiff == 0, f"call {rep + 1}: {ndiff} output elements differ from the first call"


def test_decode_rejects_small_workspace(fga):
    import torch
    cache = fga.KVCache(oracle.FULL, 1, 64)
    q = torch.zeros(1, 16, 256, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 16, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(fga.SparkError) as e:
        fga.decode(oracle.FULL, q, g, cache, i32_dev([64]), 64, workspace=ws, num_parts=2)
    assert e.value.status == 3
