"""8-bit (q8_0) KV cache parity: append and decode through the C ABI against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, f64_of, i32_dev, note, to_dev

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    return t.detach().cpu().numpy()


def _cache_arrays(seed, B, cap, fill_lens=None):
    """Seeded codes and scales for every slot (or the first fill_lens[b] slots of b)."""
    kc = np.zeros((B, cap, 4, 256), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((B, cap, 4, 8), np.float16)
    vs = np.zeros_like(ks)
    for b in range(B):
        n = cap if fill_lens is None else min(int(fill_lens[b]), cap)
        kc[b, :n], ks[b, :n], vc[b, :n], vs[b, :n] = synth.q8_cache_rows(seed, b, n)
    return kc, ks, vc, vs


def _gpu_cache(fga, lt, arrays):
    kc, ks, vc, vs = arrays
    return fga.KVCacheQ8(lt, kc.shape[0], kc.shape[1], k=_dev(kc), k_scale=_dev(ks), v=_dev(vc), v_scale=_dev(vs))


def _assert_cache(cache, want, what):
    """V codes and scales bit for bit; K (rotated on the GPU in fp32 with hardware sin/cos,
    in the oracle in fp64) codes within one step and scales within one fp16 step, both
    rarely off."""
    kc, ks, vc, vs = (_host(cache.k), _host(cache.k_scale), _host(cache.v), _host(cache.v_scale))
    wkc, wks, wvc, wvs = want
    assert np.array_equal(vc, wvc), f"{what}: V codes differ at {np.argwhere(vc != wvc)[:5].tolist()}"
    assert np.array_equal(vs.view(np.uint16), wvs.view(np.uint16)), f"{what}: V scales differ"
    dk = np.abs(kc.astype(np.int32) - wkc.astype(np.int32))
    ds = np.abs(ks.astype(np.float64) - wks.astype(np.float64))
    ulp = np.ldexp(1.0, np.frexp(np.maximum(wks.astype(np.float64), 2.0 ** -14))[1] - 11)
    frac_c = float(np.mean(dk != 0))
    frac_s = float(np.mean(ks.view(np.uint16) != wks.view(np.uint16)))
    note(f"[q8 cache] {what}: K codes differing {frac_c:.2e} (max {int(dk.max())}), "
         f"K scales differing {frac_s:.2e}")
    assert dk.max() <= 1, f"{what}: a K code differs by {int(dk.max())}"
    assert (ds <= ulp).all(), f"{what}: a K scale differs by more than one fp16 step"
    assert frac_c < 1e-3 and frac_s < 1e-3, f"{what}: too many K differences"


APPEND = [(oracle.FULL, 1, [0, 7], 64), (oracle.FULL, 33, [0, 100], 200), (oracle.SLIDING, 5, [0, 1000], 512),
          (oracle.SLIDING, 600, [100, 0], 512), (oracle.SLIDING, 512, [3, 512], 512),
          (oracle.FULL, 1000, [2, 5000], 6100)]


@pytest.mark.parametrize("lt,n_new,pos,cap", APPEND, ids=[f"lt{a}_n{b}_p{c[1]}" for a, b, c, _ in APPEND])
def test_kv_append_q8(fga, lt, n_new, pos, cap):
    """Quantised append into a cache already holding other codes: written slots match the
    oracle's q8_0 append, untouched slots keep their contents (ring wrap included)."""
    import torch
    B = len(pos)
    note(f"append q8 lt={lt} n={n_new} pos={pos}")
    inp = synth.prefill_inputs(6100 + n_new + lt, B, n_new)
    before = _cache_arrays(6200 + n_new, B, cap)
    cache = _gpu_cache(fga, lt, before)
    fga.kv_append_q8(lt, to_dev(inp["k"]), to_dev(inp["v"]), i32_dev(pos), cache)
    torch.cuda.synchronize()
    want = oracle.kv_append_q8(*before, inp["k"], inp["v"], np.array(pos, np.int32), lt)
    _assert_cache(cache, want, f"append lt={lt} n={n_new} pos={pos}")


def _decode_q8(fga, lt, q, gate, arrays, lens, num_parts=0, max_len=None):
    import torch
    cache = _gpu_cache(fga, lt, arrays)
    out = fga.decode_q8(lt, to_dev(q), to_dev(gate), cache, i32_dev(lens),
                        max(1, int(max(lens))) if max_len is None else max_len, num_parts=num_parts)
    torch.cuda.synchronize()
    return f64_of(out)


def _ring_of(arrays, lens):
    """Ring arrays holding positions max(0, L-512)..L-1 of contiguous arrays, in slot p mod 512."""
    out = []
    for a in arrays:
        r = np.zeros((a.shape[0], 512) + a.shape[2:], a.dtype)
        for b in range(a.shape[0]):
            p = np.arange(max(0, int(lens[b]) - 512), int(lens[b]))
            r[b, p % 512] = a[b, p]
        out.append(r)
    return tuple(out)


EDGE = [[1], [31], [512], [513], [1, 37, 600, 1025], [4097, 64, 2000]]


@pytest.mark.parametrize("lens", EDGE, ids=["L" + "-".join(map(str, x)) for x in EDGE])
@pytest.mark.parametrize("num_parts", [0, 1, 3, 5000])
def test_decode_q8_edges(fga, lens, num_parts):
    """Ragged chunks, partitions across sequence boundaries, empty partitions; full cache
    and ring."""
    lens = np.array(lens, np.int32)
    B, cap = len(lens), int(lens.max())
    seed = 6300 + int(lens.sum())
    q = synth.normal_bf16(seed, 0, (B, 16, 256))
    gate = synth.normal_bf16(seed, 1, (B, 16))
    arrays = _cache_arrays(seed, B, cap, fill_lens=lens)
    note(f"decode q8 lens={lens.tolist()} parts={num_parts}")
    got = _decode_q8(fga, oracle.FULL, q, gate, arrays, lens, num_parts)
    want = oracle.decode_q8(q, gate, *arrays, lens, oracle.FULL)
    assert_parity(got, want, f"decode q8 full lens={lens.tolist()} parts={num_parts}")
    ring = _ring_of(arrays, lens)
    got = _decode_q8(fga, oracle.SLIDING, q, gate, ring, lens, num_parts)
    want = oracle.decode_q8(q, gate, *ring, lens, oracle.SLIDING)
    assert_parity(got, want, f"decode q8 sliding lens={lens.tolist()} parts={num_parts}")


def test_decode_q8_b64(fga):
    """Batch 64, context lengths uniform in [1024, 32768]: full cache and 512-slot ring."""
    seed = synth.SEED_DECODE_B64
    B, cap = 64, 32768
    lens = synth.decode_seq_lens(seed, B, 1024, 32768)
    q = synth.normal_bf16(seed, 0, (B, 16, 256))
    gate = synth.normal_bf16(seed, 1, (B, 16))
    arrays = _cache_arrays(seed + 7, B, cap, fill_lens=lens)
    note("decode q8 B=64 full")
    got = _decode_q8(fga, oracle.FULL, q, gate, arrays, lens, max_len=cap)
    assert_parity(got, oracle.decode_q8(q, gate, *arrays, lens, oracle.FULL), "decode q8 B=64 full")
    ring = _ring_of(arrays, lens)
    del arrays
    got = _decode_q8(fga, oracle.SLIDING, q, gate, ring, lens, max_len=cap)
    assert_parity(got, oracle.decode_q8(q, gate, *ring, lens, oracle.SLIDING), "decode q8 B=64 sliding")


def test_decode_q8_long(fga):
    """Batch 4 at 131072 tokens on a full layer, and their 512-slot rings."""
    seed = synth.SEED_LONG_DECODE + 40
    B, L = 4, 131072
    lens = np.full(B, L, np.int32)
    q = synth.normal_bf16(seed, 0, (B, 16, 256))
    gate = synth.normal_bf16(seed, 1, (B, 16))
    arrays = _cache_arrays(seed, B, L)
    note("decode q8 long full")
    got = _decode_q8(fga, oracle.FULL, q, gate, arrays, lens)
    assert_parity(got, oracle.decode_q8(q, gate, *arrays, lens, oracle.FULL), "decode q8 B=4 L=131072 full")
    ring = _ring_of(arrays, lens)
    got = _decode_q8(fga, oracle.SLIDING, q, gate, ring, lens)
    assert_parity(got, oracle.decode_q8(q, gate, *ring, lens, oracle.SLIDING), "decode q8 B=4 L=131072 sliding")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
@pytest.mark.parametrize("num_parts", [0, 7, 300])
def test_decode_q8_is_deterministic(fga, lt, num_parts):
    """Repeated 8-bit decode calls at batch 64 (lengths uniform in [1024, 32768]) give
    bit-identical outputs, with the library's partition count and with uneven ones; each
    call gets a fresh NaN-filled output and workspace.  The K codes pass between the
    lanes of a wave through LDS, which this would expose if a read overtook a write."""
    import torch
    seed = synth.SEED_DECODE_B64 + 11
    B = 64
    lens = synth.decode_seq_lens(seed, B, 1024, 32768)
    cap = 512 if lt == oracle.SLIDING else int(lens.max())
    arrays = _cache_arrays(seed, B, cap, fill_lens=None if lt == oracle.SLIDING else lens)
    cache = _gpu_cache(fga, lt, arrays)
    del arrays
    q = to_dev(synth.normal_bf16(seed, 0, (B, 16, 256)))
    g = to_dev(synth.normal_bf16(seed, 1, (B, 16)))
    L = i32_dev(lens)
    note(f"decode q8 determinism lt={lt} parts={num_parts}")
    ref = fga.decode_q8(lt, q, g, cache, L, int(lens.max()), num_parts=num_parts).view(torch.int16).clone()
    for rep in range(6):
        out = fga.decode_q8(lt, q, g, cache, L, int(lens.max()), num_parts=num_parts).view(torch.int16)
        ndiff = int((out != ref).sum())
        assert ndiff == 0, f"call {rep + 1}: {ndiff} output elements differ from the first call"


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_append_then_decode_q8(fga, lt):
    """A context appended in two pieces to an 8-bit cache, then decoded: against the
    oracle's own append and decode of the same context."""
    import torch
    B, S = 2, 900
    cap = 512 if lt == oracle.SLIDING else S
    inp = synth.prefill_inputs(6400 + lt, B, S)
    cache = fga.KVCacheQ8(lt, B, cap)
    k, v = to_dev(inp["k"]), to_dev(inp["v"])
    fga.kv_append_q8(lt, k[:, :700].contiguous(), v[:, :700].contiguous(), i32_dev([0, 0]), cache)
    fga.kv_append_q8(lt, k[:, 700:].contiguous(), v[:, 700:].contiguous(), i32_dev([700, 700]), cache)
    lens = np.array([S, S], np.int32)
    qd, gd = inp["q"][:, S - 1], inp["gate"][:, S - 1]
    out = fga.decode_q8(lt, to_dev(qd), to_dev(gd), cache, i32_dev(lens), S)
    torch.cuda.synchronize()
    z = (np.zeros((B, cap, 4, 256), np.int8), np.zeros((B, cap, 4, 8), np.float16),
         np.zeros((B, cap, 4, 256), np.int8), np.zeros((B, cap, 4, 8), np.float16))
    w = oracle.kv_append_q8(*z, inp["k"][:, :700], inp["v"][:, :700], np.array([0, 0]), lt)
    w = oracle.kv_append_q8(*w, inp["k"][:, 700:], inp["v"][:, 700:], np.array([700, 700]), lt)
    _assert_cache(cache, w, f"append+decode cache lt={lt}")
    want = oracle.decode_q8(qd, gd, *w, lens, lt)
    assert_parity(f64_of(out), want, f"append+decode q8 lt={lt}")
    # Reading the same keys through 8 bits costs little against the bf16 path's result.
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=np.array([S - 1]))[:, 0]
    rel = float(np.linalg.norm(f64_of(out) - ref) / np.linalg.norm(ref))
    note(f"[q8] lt={lt}: relative L2 to the unquantised attention {rel:.2e}")
    assert rel < 2e-2


def test_decode_q8_rejects_small_workspace(fga):
    import torch
    cache = fga.KVCacheQ8(oracle.FULL, 1, 64)
    q = torch.zeros(1, 16, 256, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 16, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fga.SparkError) as e:
        fga.decode_q8(oracle.FULL, q, g, cache, i32_dev([5]), 64, workspace=ws)
    assert e.value.status == 3
