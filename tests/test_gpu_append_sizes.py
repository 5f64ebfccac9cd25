"""KV append at the sizes the benchmark times, through the C ABI against the oracle: a bulk
append of 32768 tokens (batch 1; full cache, and the ring keeping the last 512) and the
one-token append of a batch-64 decode step at positions up to 32767, for the bf16 and the
8-bit cache."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_cached_keys_close, bits_of, i32_dev, note, to_dev
from test_gpu_q8 import _assert_cache

pytestmark = pytest.mark.gpu


def _host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_kv_append_bulk_32768(fga, lt):
    import torch
    n = 32768
    cap = oracle.WINDOW if lt == oracle.SLIDING else n
    note(f"bulk append lt={lt} n={n}")
    k = synth.normal_bf16(4500 + lt, 0, (1, n, 4, 256))
    v = synth.normal_bf16(4500 + lt, 1, (1, n, 4, 256))
    pos = np.zeros(1, np.int32)
    cache = fga.KVCache(lt, 1, cap)
    fga.kv_append(lt, to_dev(k), to_dev(v), i32_dev(pos), cache)
    c8 = fga.KVCacheQ8(lt, 1, cap)
    fga.kv_append_q8(lt, to_dev(k), to_dev(v), i32_dev(pos), c8)
    torch.cuda.synchronize()
    z = np.zeros((1, cap, 4, 256), np.uint16)
    ck, cv = oracle.kv_append(z, z, k, v, pos, lt)
    assert np.array_equal(bits_of(cache.v), cv), "cached values differ"
    assert_cached_keys_close(bits_of(cache.k), ck, f"bulk append lt={lt}")
    zc, zs = np.zeros((1, cap, 4, 256), np.int8), np.zeros((1, cap, 4, 8), np.float16)
    want = oracle.kv_append_q8(zc, zs, zc.copy(), zs.copy(), k, v, pos, lt)
    _assert_cache(c8, want, f"bulk 8-bit append lt={lt}")


@pytest.mark.parametrize("lt", [oracle.SLIDING, oracle.FULL], ids=["sliding", "full"])
def test_kv_append_decode_step_b64(fga, lt):
    """One token per sequence at position L_b - 1, L_b uniform in [1024, 32768]: the slot
    each sequence writes, against the oracle's append of that token alone (a cache of one
    sequence just long enough to hold the slot)."""
    import torch
    B = 64
    lens = synth.decode_seq_lens(synth.SEED_DECODE_B64, B, 1024, 32768)
    pos = (lens - 1).astype(np.int32)
    cap = oracle.WINDOW if lt == oracle.SLIDING else 32768
    note(f"decode-step append lt={lt} B={B}")
    k = synth.normal_bf16(4600 + lt, 0, (B, 1, 4, 256))
    v = synth.normal_bf16(4600 + lt, 1, (B, 1, 4, 256))
    cache = fga.KVCache(lt, B, cap)
    fga.kv_append(lt, to_dev(k), to_dev(v), i32_dev(pos), cache)
    c8 = fga.KVCacheQ8(lt, B, cap)
    fga.kv_append_q8(lt, to_dev(k), to_dev(v), i32_dev(pos), c8)
    torch.cuda.synchronize()
    slots = np.array([oracle.cache_slot(int(p), lt) for p in pos])
    idx = (torch.arange(B, device="cuda"), torch.as_tensor(slots, device="cuda"))
    gk, gv = bits_of(cache.k[idx]), bits_of(cache.v[idx])
    g8 = [_host(t[idx]) for t in (c8.k, c8.k_scale, c8.v, c8.v_scale)]
    wk = np.zeros_like(gk)
    wv = np.zeros_like(gv)
    w8 = [np.zeros_like(a) for a in g8]
    for b in range(B):
        n = int(slots[b]) + 1
        z = np.zeros((1, n, 4, 256), np.uint16)
        ck, cv = oracle.kv_append(z, z, k[b:b + 1], v[b:b + 1], pos[b:b + 1], lt)
        wk[b], wv[b] = ck[0, -1], cv[0, -1]
        zc, zs = np.zeros((1, n, 4, 256), np.int8), np.zeros((1, n, 4, 8), np.float16)
        q8 = oracle.kv_append_q8(zc, zs, zc.copy(), zs.copy(), k[b:b + 1], v[b:b + 1], pos[b:b + 1], lt)
        for i in range(4):
            w8[i][b] = q8[i][0, -1]
    assert np.array_equal(gv, wv), "cached values differ"
    assert_cached_keys_close(gk, wk, f"decode-step append lt={lt}")

    class _Written:   # the written rows, shaped as a cache for the 8-bit comparison
        k, k_scale, v, v_scale = (torch.from_numpy(a[:, None]) for a in g8)
    _assert_cache(_Written, tuple(a[:, None] for a in w8), f"decode-step 8-bit append lt={lt}")
