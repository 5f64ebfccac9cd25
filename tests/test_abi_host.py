"""The C-ABI library on the CPU: it loads, exports every function the header declares,
and its host-side argument checks reject bad calls before any HIP call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spark_attn.h")

fga = pytest.importorskip("full_gqa_attention_amd")
lib = fga._lib

FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced by rejected calls
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spark_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(fga.EXPORTED)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by {fga.LIBRARY_PATH}"


def test_version_and_status_strings():
    assert fga.abi_version() == 8
    assert fga.status_string(0) == "ok"
    assert fga.status_string(3) == "workspace too small"
    assert fga.status_string(99) == "unknown status"


def test_layer_schedule_from_the_library():
    """The stack schedule and per-type RoPE come from the C library, and agree with the
    pages' statement as the oracle writes it down (27 sliding, 9 full, last layer full)."""
    import oracle
    types = [fga.layer_type_of(i) for i in range(36)]
    assert types == [oracle.layer_type_of(i) for i in range(36)]
    assert types.count(fga.SLIDING) == 27 and types.count(fga.FULL) == 9 and types[35] == fga.FULL
    assert lib.spark_layer_type_of(-1) == -1 and lib.spark_layer_type_of(36) == -1
    for lt in (fga.SLIDING, fga.FULL):
        assert fga.layer_params(lt) == oracle.layer_params(lt)
    th = ctypes.c_double(-1.0)
    assert lib.spark_layer_params(2, ctypes.byref(th), None, None) == 1 and th.value == -1.0
    assert lib.spark_layer_params(0, None, None, None) == 0


def _cache(k=FAKE, v=FAKE, batch=1, cap=512):
    return ctypes.pointer(fga.KvCacheDesc(k.value if k else None, v.value if v else None, batch, cap))


def prefill(**kw):
    a = dict(lt=1, B=1, S=16, start=0, q=FAKE, k=FAKE, v=FAKE, g=FAKE, cache=None, ws=FAKE,
             ws_bytes=1 << 30, out=FAKE)
    a.update(kw)
    return lib.spark_attn_prefill(a["lt"], a["B"], a["S"], a["start"], a["q"], a["k"], a["v"], a["g"],
                                  a["cache"], a["ws"], a["ws_bytes"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(lt=2), 1), (dict(lt=-1), 1), (dict(B=0), 1), (dict(S=0), 1), (dict(S=(1 << 20) + 1), 1),
    (dict(q=None), 1), (dict(out=None), 1), (dict(k=MISALIGNED), 1), (dict(start=-1), 1),
    (dict(start=5), 1),                       # a prefix needs the cache it is read from
    (dict(start=16, cache=_cache(cap=31)), 1),   # full: capacity < start_pos + seq_len
    (dict(start=(1 << 20) - 15, cache=_cache(cap=1 << 21)), 1),   # start_pos + seq_len > 2^20
    (dict(lt=0, start=100, cache=_cache(batch=2)), 1),
    (dict(lt=0, cache=_cache(cap=511)), 1), (dict(lt=1, cache=_cache(cap=15)), 1),
    (dict(cache=_cache(batch=2)), 1), (dict(cache=_cache(k=None)), 1),
    (dict(ws=None), 1), (dict(ws=MISALIGNED), 1),
    (dict(ws_bytes=16 * 4 * 256 * 2 - 1), 3),
    (dict(B=65535, S=1 << 20), 1),            # batch * seq_len >= 2^32
])
def test_prefill_rejects(kw, status):
    assert prefill(**kw) == status


def test_prefill_workspace_planning():
    ws = fga.prefill_workspace_bytes
    assert ws(1, 1, 16) == 16 * 4 * 256 * 2            # rotated keys, bf16 [B, S, 4, 256]
    assert ws(0, 3, 1000) == 3 * 1000 * 4 * 256 * 2
    assert ws(2, 1, 16) == 0 and ws(1, 0, 16) == 0 and ws(1, 1, (1 << 20) + 1) == 0


def test_append_rejects():
    f = lib.spark_kv_append
    assert f(3, 1, 1, FAKE, FAKE, FAKE, _cache(), None) == 1
    assert f(0, 1, 0, FAKE, FAKE, FAKE, _cache(), None) == 1
    assert f(0, 1, 1, FAKE, FAKE, None, _cache(), None) == 1
    assert f(0, 1, 1, FAKE, FAKE, FAKE, _cache(cap=1024), None) == 1
    assert f(1, 1, 1, FAKE, FAKE, FAKE, None, None) == 1


def _layout_bytes(batch, parts):
    """The workspace layout: partition range of each sequence [batch, 2] (int32), then
    (parts + batch) partials of 16 x 256 floats and of 16 x 2 floats, each region 256-byte
    aligned."""
    up = lambda x: (x + 255) // 256 * 256
    slots = parts + batch
    return up(8 * batch) + up(slots * 16 * 256 * 4) + slots * 16 * 2 * 4


def test_workspace_planning():
    ws = fga.decode_workspace_bytes
    assert ws(1, 1, 64, 2) == _layout_bytes(1, 2)
    assert ws(1, 3, 64, 5000) == _layout_bytes(3, 5000)
    # Library's choice: never more partitions than 32-key chunks in the batch, at most one
    # per CU of MI355X (256, a constant: the size never depends on the current device).
    assert ws(1, 1, 64) == _layout_bytes(1, 2)
    assert ws(0, 1, 100000) == _layout_bytes(1, 16)       # ring: <= 512 keys = 16 chunks
    assert ws(1, 64, 32768) == _layout_bytes(64, 256)
    assert ws(1, 1, 64, -1) == 0 and ws(1, 1, 64, (1 << 20) + 1) == 0
    assert ws(2, 1, 64) == 0 and ws(1, 0, 64) == 0 and ws(1, 1, 0) == 0


def test_decode_rejects():
    f = lib.spark_attn_decode
    big = 1 << 30
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 65, 0, FAKE, big, FAKE, None) == 1   # > capacity
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, -1, FAKE, big, FAKE, None) == 1  # parts < 0
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, (1 << 20) + 1, FAKE, big, FAKE, None) == 1
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, 2, FAKE, 16, FAKE, None) == 3    # workspace
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, 0, MISALIGNED, big, FAKE, None) == 1
    assert f(0, 1, FAKE, FAKE, _cache(cap=1024), FAKE, 64, 0, FAKE, big, FAKE, None) == 1


def test_decode_noalloc_rejects():
    """Checks of the entry point without a workspace, all before any HIP call."""
    f = lib.spark_attn_decode_noalloc
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 65, 0, FAKE, None) == 1      # > capacity
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, -1, FAKE, None) == 1     # parts < 0
    assert f(1, 1, None, FAKE, _cache(cap=64), FAKE, 64, 0, FAKE, None) == 1      # no q
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, 0, MISALIGNED, None) == 1
    assert f(0, 1, FAKE, FAKE, _cache(cap=1024), FAKE, 64, 0, FAKE, None) == 1    # ring != 512
    # Beyond the 16 MiB static scratch: 256 + 1000 partial results, or 4000 + 1.
    assert fga.decode_workspace_bytes(1, 1000, 64) > fga.NOALLOC_SCRATCH_BYTES
    assert f(1, 1000, FAKE, FAKE, _cache(batch=1000, cap=64), FAKE, 64, 0, FAKE, None) == 3
    assert f(1, 1, FAKE, FAKE, _cache(cap=64), FAKE, 64, 4000, FAKE, None) == 3


def _cache_q8(k=FAKE, ks=FAKE, v=FAKE, vs=FAKE, batch=1, cap=512):
    val = lambda p: p.value if p else None
    return ctypes.pointer(fga.KvCacheQ8Desc(val(k), val(ks), val(v), val(vs), batch, cap))


def test_append_q8_rejects():
    f = lib.spark_kv_append_q8
    assert f(3, 1, 1, FAKE, FAKE, FAKE, _cache_q8(), None) == 1                  # layer type
    assert f(0, 1, 0, FAKE, FAKE, FAKE, _cache_q8(), None) == 1                  # n_new
    assert f(0, 1, 1, FAKE, FAKE, None, _cache_q8(), None) == 1                  # pos
    assert f(0, 1, 1, FAKE, FAKE, FAKE, _cache_q8(cap=1024), None) == 1          # ring != 512
    assert f(1, 1, 1, FAKE, FAKE, FAKE, None, None) == 1                         # no cache
    assert f(1, 1, 1, FAKE, FAKE, FAKE, _cache_q8(ks=None), None) == 1           # no K scales
    assert f(1, 1, 1, FAKE, FAKE, FAKE, _cache_q8(vs=MISALIGNED), None) == 1     # misaligned
    assert f(1, 1, 1, FAKE, FAKE, FAKE, _cache_q8(batch=2), None) == 1           # batch


def test_decode_q8_rejects():
    f = lib.spark_attn_decode_q8
    big = 1 << 30
    assert f(1, 1, FAKE, FAKE, _cache_q8(cap=64), FAKE, 65, 0, FAKE, big, FAKE, None) == 1  # > capacity
    assert f(1, 1, FAKE, FAKE, _cache_q8(cap=64), FAKE, 64, -1, FAKE, big, FAKE, None) == 1
    assert f(1, 1, FAKE, FAKE, _cache_q8(cap=64), FAKE, 64, 2, FAKE, 16, FAKE, None) == 3   # workspace
    assert f(1, 1, FAKE, FAKE, _cache_q8(cap=64), FAKE, 64, 0, MISALIGNED, big, FAKE, None) == 1
    assert f(0, 1, FAKE, FAKE, _cache_q8(cap=1024), FAKE, 64, 0, FAKE, big, FAKE, None) == 1
    assert f(1, 1, FAKE, FAKE, _cache_q8(k=None, cap=64), FAKE, 64, 0, FAKE, big, FAKE, None) == 1
    assert f(1, 1, FAKE, FAKE, None, FAKE, 64, 0, FAKE, big, FAKE, None) == 1


def test_workspace_planning_q8():
    ws = fga.decode_q8_workspace_bytes
    assert ws(1, 1, 64, 2) == _layout_bytes(1, 2)
    assert ws(1, 64, 32768) == _layout_bytes(64, 512)     # two partitions per CU (256 on the host)
    assert ws(0, 1, 100000) == _layout_bytes(1, 16)       # never more than the chunks
    assert ws(2, 1, 64) == 0 and ws(1, 1, 64, -1) == 0


def varlen(**kw):
    a = dict(lt=1, B=2, cu=FAKE, T=100, M=64, q=FAKE, k=FAKE, v=FAKE, g=FAKE, cache=None, ws=FAKE,
             ws_bytes=1 << 30, out=FAKE)
    a.update(kw)
    return lib.spark_attn_prefill_varlen(a["lt"], a["B"], a["cu"], a["T"], a["M"], a["q"], a["k"], a["v"],
                                         a["g"], a["cache"], a["ws"], a["ws_bytes"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(lt=2), 1), (dict(B=0), 1), (dict(M=0), 1), (dict(M=(1 << 20) + 1), 1), (dict(T=0), 1),
    (dict(cu=None), 1), (dict(cu=ctypes.c_void_p(0x10002)), 1), (dict(q=None), 1), (dict(k=MISALIGNED), 1),
    (dict(B=65535, M=1 << 20), 1),                 # batch * max_seqlen >= 2^32
    (dict(cache=_cache(batch=3)), 1), (dict(cache=_cache(cap=63)), 1), (dict(lt=0, cache=_cache(cap=100)), 1),
    (dict(ws=MISALIGNED), 1), (dict(ws_bytes=100 * 4 * 256 * 2 + 255), 3),
])
def test_prefill_varlen_rejects(kw, status):
    assert varlen(**kw) == status


def test_prefill_varlen_workspace():
    assert fga.prefill_varlen_workspace_bytes(1, 100) == 100 * 4 * 256 * 2 + 256
    assert fga.prefill_varlen_workspace_bytes(2, 100) == 0 and fga.prefill_varlen_workspace_bytes(0, 0) == 0


def test_qkv_proj_rejects():
    f = lib.spark_qkv_proj_fp8
    ok = dict(T=16, x=FAKE, w=FAKE, s=FAKE, g=FAKE, q=FAKE, k=FAKE, v=FAKE, gl=FAKE, ws=FAKE, wsb=1 << 30)
    call = lambda **kw: f(*({**ok, **kw}[n] for n in ("T", "x", "w", "s", "g", "q", "k", "v", "gl", "ws", "wsb")), None)
    assert call(T=0) == 1 and call(T=(1 << 20) + 1) == 1
    assert call(x=None) == 1 and call(s=None) == 1 and call(ws=None) == 1
    assert call(x=MISALIGNED) == 1 and call(ws=MISALIGNED) == 1 and call(s=ctypes.c_void_p(0x10002)) == 1
    assert call(wsb=16 * 2560) == 3
    assert fga.qkv_proj_fp8_workspace_bytes(16) == 16 * 2560 + 16 * 4
    assert fga.qkv_proj_fp8_workspace_bytes(5) == 12800 + 20 and fga.qkv_proj_fp8_workspace_bytes(0) == 0
