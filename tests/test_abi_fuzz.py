"""Fuzzing of the C ABI's host-side argument checks, on a host without a GPU.

Every entry point is called with random arguments: sizes in and out of range, null,
misaligned and aligned fake pointers (never dereferenced), cache descriptors of every
shape.  The status must be the one the header's rules give: SPARK_ERR_INVALID_ARG for
any broken rule, else SPARK_ERR_WORKSPACE for a short workspace, else the call passes
the checks and reaches its launch, which on a host without a GPU fails with
SPARK_ERR_HIP.  The rules below are written from include/spark_attn.h, not from the
implementation.  A second test builds the library's host code with AddressSanitizer and
runs a C driver (tests/abi_fuzz_main.c) through the same kind of calls.

These tests never run where a GPU is visible: there, a call that passes the checks
would launch kernels on the fake pointers.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

fga = pytest.importorskip("full_gqa_attention_amd")
torch = pytest.importorskip("torch")
hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fuzzing passes fake pointers: host-only (no GPU visible)")

lib = fga._lib
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, WORKSPACE, PASSED = 1, 3, 4       # PASSED: the checks passed and the launch failed (no GPU)
MAX_SEQ = 1 << 20

# Fake device addresses: aligned to 256, to 16 only, to 2 only, odd, and null.
PTRS = [0x100000, 0x100010, 0x100002, 0x100001, 0]
ptr = st.sampled_from(PTRS)
size = st.one_of(st.integers(-3, 40), st.sampled_from([511, 512, 513, 4096, 65535, 65536, MAX_SEQ,
                                                      MAX_SEQ + 1, 1 << 30, -(1 << 31)]))
ltype = st.sampled_from([0, 1, 1, 0, 2, -1])
FUZZ = settings(max_examples=1500, deadline=None, suppress_health_check=list(HealthCheck))


def aligned(p, n):
    return p != 0 and p % n == 0


def vp(p):
    return ctypes.c_void_p(p or None)


def cache_rule(lt, c, batch):
    """Rules of a spark_kv_cache: non-null 16-aligned k and v, batch equal, capacity >= 1,
    and a sliding layer's ring has exactly 512 slots."""
    k, v, cb, cap = c
    return (aligned(k, 16) and aligned(v, 16) and cb == batch and cap >= 1
            and (lt != 0 or cap == 512))


cache_st = st.tuples(ptr, ptr, st.sampled_from([1, 2, 3, 7]), st.sampled_from([1, 37, 64, 511, 512, 513, 4096]))


def cache_desc(c):
    return None if c is None else ctypes.pointer(fga.KvCacheDesc(c[0] or None, c[1] or None, c[2], c[3]))


@FUZZ
@given(lt=ltype, B=st.sampled_from([1, 2, 3, 7, 0, -1, 65535, 65536]), S=size,
       start=st.sampled_from([0, 0, 1, 37, 600, -1, MAX_SEQ - 16]), q=ptr, k=ptr, v=ptr, g=ptr, out=ptr,
       cache=st.one_of(st.none(), cache_st), ws=ptr, ws_slack=st.sampled_from([-1, 0, 256]))
def test_prefill_checks(lt, B, S, start, q, k, v, g, out, cache, ws, ws_slack):
    need = max(B, 0) * max(S, 0) * 4 * 256 * 2
    ws_bytes = max(need + ws_slack, 0)
    ok = (lt in (0, 1) and 1 <= B <= 65535 and 1 <= S <= MAX_SEQ and B * S <= 0xFFFFFFFE
          and all(aligned(p, 16) for p in (q, k, v, out)) and aligned(g, 2)
          and 0 <= start and start + S <= MAX_SEQ and not (start > 0 and cache is None)
          and (cache is None or (cache_rule(lt, cache, B) and (lt != 1 or cache[3] >= start + S)))
          and aligned(ws, 256))
    want = INVALID if not ok else (WORKSPACE if ws_bytes < need else PASSED)
    got = lib.spark_attn_prefill(lt, B, S, start, vp(q), vp(k), vp(v), vp(g), cache_desc(cache), vp(ws),
                                 ws_bytes, vp(out), None)
    assert got == want


def decode_rule(lt, B, maxlen, parts, q, g, sl, out):
    return (lt in (0, 1) and 1 <= B <= 65535 and 1 <= maxlen <= MAX_SEQ and 0 <= parts <= MAX_SEQ
            and aligned(q, 16) and aligned(out, 16) and aligned(g, 2) and aligned(sl, 4))


@FUZZ
@given(lt=ltype, B=st.sampled_from([1, 2, 3, 7, 0, -1, 65536]), maxlen=size,
       parts=st.sampled_from([0, 0, 1, 5, 256, -1, MAX_SEQ, MAX_SEQ + 1]), q=ptr, g=ptr, sl=ptr, out=ptr,
       cache=st.one_of(st.none(), cache_st), ws=ptr, ws_slack=st.sampled_from([-1, 0, 64]), q8=st.booleans())
def test_decode_checks(lt, B, maxlen, parts, q, g, sl, out, cache, ws, ws_slack, q8):
    ok = decode_rule(lt, B, maxlen, parts, q, g, sl, out) and aligned(ws, 256) and cache is not None
    ok = ok and cache_rule(lt, cache, B) and (lt != 1 or maxlen <= cache[3])
    need = (fga.decode_q8_workspace_bytes if q8 else fga.decode_workspace_bytes)(lt, B, maxlen, parts) if ok else 0
    ws_bytes = max(need + ws_slack, 0)
    want = INVALID if not ok else (WORKSPACE if ws_bytes < need else PASSED)
    if q8:
        c = None if cache is None else ctypes.pointer(fga.KvCacheQ8Desc(cache[0] or None, cache[0] or None,
                                                                         cache[1] or None, cache[1] or None,
                                                                         cache[2], cache[3]))
        got = lib.spark_attn_decode_q8(lt, B, vp(q), vp(g), c, vp(sl), maxlen, parts, vp(ws), ws_bytes, vp(out), None)
    else:
        got = lib.spark_attn_decode(lt, B, vp(q), vp(g), cache_desc(cache), vp(sl), maxlen, parts, vp(ws),
                                    ws_bytes, vp(out), None)
    assert got == want


@FUZZ
@given(lt=ltype, B=st.sampled_from([1, 2, 3, 7, 0, 1000]), maxlen=size,
       parts=st.sampled_from([0, 0, 1, 5, 256, 4000, -1, MAX_SEQ + 1]), q=ptr, g=ptr, sl=ptr, out=ptr,
       cache=st.one_of(st.none(), cache_st))
def test_decode_noalloc_checks(lt, B, maxlen, parts, q, g, sl, out, cache):
    ok = decode_rule(lt, B, maxlen, parts, q, g, sl, out) and cache is not None
    ok = ok and cache_rule(lt, cache, B) and (lt != 1 or maxlen <= cache[3])
    big = ok and fga.decode_workspace_bytes(lt, B, maxlen, parts) > fga.NOALLOC_SCRATCH_BYTES
    want = INVALID if not ok else (WORKSPACE if big else PASSED)
    got = lib.spark_attn_decode_noalloc(lt, B, vp(q), vp(g), cache_desc(cache), vp(sl), maxlen, parts, vp(out), None)
    assert got == want


@FUZZ
@given(lt=ltype, B=st.sampled_from([1, 2, 3, 0, -1, 65536]), n=size, k=ptr, v=ptr, pos=ptr,
       cache=st.one_of(st.none(), cache_st), q8=st.booleans())
def test_append_checks(lt, B, n, k, v, pos, cache, q8):
    ok = (lt in (0, 1) and 1 <= B <= 65535 and 1 <= n <= MAX_SEQ and aligned(k, 16) and aligned(v, 16)
          and aligned(pos, 4) and cache is not None and cache_rule(lt, cache, B))
    if q8:
        c = None if cache is None else ctypes.pointer(fga.KvCacheQ8Desc(cache[0] or None, cache[0] or None,
                                                                         cache[1] or None, cache[1] or None,
                                                                         cache[2], cache[3]))
        got = lib.spark_kv_append_q8(lt, B, n, vp(k), vp(v), vp(pos), c, None)
    else:
        got = lib.spark_kv_append(lt, B, n, vp(k), vp(v), vp(pos), cache_desc(cache), None)
    assert got == (PASSED if ok else INVALID)


@FUZZ
@given(lt=ltype, B=st.sampled_from([1, 2, 3, 0, -1, 65536]), T=size, M=size, cu=ptr, q=ptr, g=ptr,
       cache=st.one_of(st.none(), cache_st), ws=ptr, ws_slack=st.sampled_from([-1, 0, 256]))
def test_prefill_varlen_checks(lt, B, T, M, cu, q, g, cache, ws, ws_slack):
    need = ((max(T, 0) * 2048 + 255) // 256) * 256 + 256
    ws_bytes = max(need + ws_slack, 0)
    ok = (lt in (0, 1) and 1 <= B <= 65535 and 1 <= M <= MAX_SEQ and T >= 1 and B * M <= 0xFFFFFFFE
          and aligned(cu, 4) and aligned(q, 16) and aligned(g, 2)
          and (cache is None or (cache_rule(lt, cache, B) and (lt != 1 or cache[3] >= M))) and aligned(ws, 256))
    want = INVALID if not ok else (WORKSPACE if ws_bytes < need else PASSED)
    got = lib.spark_attn_prefill_varlen(lt, B, vp(cu), T, M, vp(q), vp(q), vp(q), vp(g), cache_desc(cache), vp(ws),
                                        ws_bytes, vp(q), None)
    assert got == want


@FUZZ
@given(T=size, x=ptr, w=ptr, s=ptr, wg=ptr, ws=ptr, ws_slack=st.sampled_from([-1, 0, 256]))
def test_qkv_proj_checks(T, x, w, s, wg, ws, ws_slack):
    need = ((max(T, 0) * 2560 + 255) // 256) * 256 + max(T, 0) * 4
    ws_bytes = max(need + ws_slack, 0)
    ok = (1 <= T <= MAX_SEQ and aligned(x, 16) and aligned(w, 16) and aligned(s, 4) and aligned(wg, 16)
          and aligned(ws, 256))
    want = INVALID if not ok else (WORKSPACE if ws_bytes < need else PASSED)
    got = lib.spark_qkv_proj_fp8(T, vp(x), vp(w), vp(s), vp(wg), vp(x), vp(x), vp(x), vp(x), vp(ws), ws_bytes, None)
    assert got == want


def test_host_checks_under_address_sanitizer(tmp_path):
    """The host code of every source, built with AddressSanitizer (the device code as
    usual), driven through random calls of every entry point by tests/abi_fuzz_main.c."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    csrc = os.path.join(ROOT, "full_gqa_attention_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    srcs = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith(".hip")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Wno-unused-result",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    main_o = str(tmp_path / "main.o")
    r = subprocess.run([clang, "-O1", "-fsanitize=address", "-fno-omit-frame-pointer", *inc, "-c",
                        os.path.join(ROOT, "tests", "abi_fuzz_main.c"), "-o", main_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_fuzz")
    r = subprocess.run([clang + "++", "-fsanitize=address", *objs, main_o, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "200000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
    assert "calls:" in r.stdout, r.stdout
    print(r.stdout)
