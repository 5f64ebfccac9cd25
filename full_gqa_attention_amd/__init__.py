"""Hybrid sliding/full GQA attention for AMD Instinct MI355X (gfx950).

Python binding of ``libspark_attn.so``, whose C ABI is ``include/spark_attn.h``.  The
functions below only check and marshal arguments: every step of the computation runs in
the library's HIP kernels.  PyTorch supplies device memory and streams.  Importing this
package raises if the library has not been built (``python -m
full_gqa_attention_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

SLIDING = 0
FULL = 1
N_Q_HEADS = 16
N_KV_HEADS = 4
HEAD_DIM = 256
WINDOW = 512
N_LAYERS = 36

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspark_attn.so")


class SparkError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.spark_status_string(status).decode()} (status {status})")
        self.status = status


class KvCacheDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class KvCacheQ8Desc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("batch", ctypes.c_int32), ("capacity", ctypes.c_int32)]


def _load():
    # torch is imported first on purpose: it ships its own HIP runtime, and the library's
    # dependency on libamdhip64.so.7 must resolve to that already-loaded copy.  Loading
    # the library first would put a second HIP runtime in the process, and launches on
    # torch's streams and memory would then fail.
    import torch  # noqa: F401

    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m full_gqa_attention_amd.build` "
            "(the attention path has no implementation outside this HIP library)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    cache_p = ctypes.POINTER(KvCacheDesc)
    lib.spark_attn_prefill_workspace_bytes.argtypes = [i32, i32, i32]
    lib.spark_attn_prefill_workspace_bytes.restype = sz
    lib.spark_attn_prefill.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, cache_p, vp, sz, vp, vp]
    lib.spark_attn_prefill.restype = i32
    lib.spark_attn_prefill_varlen_workspace_bytes.argtypes = [i32, i32]
    lib.spark_attn_prefill_varlen_workspace_bytes.restype = sz
    lib.spark_attn_prefill_varlen.argtypes = [i32, i32, vp, i32, i32, vp, vp, vp, vp, cache_p, vp, sz, vp, vp]
    lib.spark_attn_prefill_varlen.restype = i32
    lib.spark_qkv_proj_fp8_workspace_bytes.argtypes = [i32]
    lib.spark_qkv_proj_fp8_workspace_bytes.restype = sz
    lib.spark_qkv_proj_fp8.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spark_qkv_proj_fp8.restype = i32
    lib.spark_kv_append.argtypes = [i32, i32, i32, vp, vp, vp, cache_p, vp]
    lib.spark_kv_append.restype = i32
    lib.spark_attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spark_attn_decode_workspace_bytes.restype = sz
    lib.spark_attn_decode.argtypes = [i32, i32, vp, vp, cache_p, vp, i32, i32, vp, sz, vp, vp]
    lib.spark_attn_decode.restype = i32
    lib.spark_attn_decode_noalloc.argtypes = [i32, i32, vp, vp, cache_p, vp, i32, i32, vp, vp]
    lib.spark_attn_decode_noalloc.restype = i32
    q8_p = ctypes.POINTER(KvCacheQ8Desc)
    lib.spark_kv_append_q8.argtypes = [i32, i32, i32, vp, vp, vp, q8_p, vp]
    lib.spark_kv_append_q8.restype = i32
    lib.spark_attn_decode_q8_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.spark_attn_decode_q8_workspace_bytes.restype = sz
    lib.spark_attn_decode_q8.argtypes = [i32, i32, vp, vp, q8_p, vp, i32, i32, vp, sz, vp, vp]
    lib.spark_attn_decode_q8.restype = i32
    lib.spark_status_string.argtypes = [i32]
    lib.spark_status_string.restype = ctypes.c_char_p
    lib.spark_abi_version.argtypes = []
    lib.spark_abi_version.restype = i32
    lib.spark_layer_type_of.argtypes = [i32]
    lib.spark_layer_type_of.restype = i32
    lib.spark_layer_params.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32),
                                       ctypes.POINTER(i32)]
    lib.spark_layer_params.restype = i32
    return lib


_lib = _load()

LIBRARY_PATH = _LIB_PATH
EXPORTED = ("spark_attn_prefill_workspace_bytes", "spark_attn_prefill", "spark_attn_prefill_varlen_workspace_bytes",
            "spark_attn_prefill_varlen", "spark_qkv_proj_fp8_workspace_bytes", "spark_qkv_proj_fp8",
            "spark_kv_append", "spark_attn_decode_workspace_bytes",
            "spark_attn_decode", "spark_kv_append_q8", "spark_attn_decode_q8_workspace_bytes", "spark_attn_decode_q8", "spark_status_string",
            "spark_abi_version", "spark_layer_type_of", "spark_layer_params", "spark_attn_decode_noalloc")


def abi_version() -> int:
    return int(_lib.spark_abi_version())


def status_string(status: int) -> str:
    return _lib.spark_status_string(int(status)).decode()


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class KVCache:
    """One layer's KV cache: bf16 K (post-RoPE) and V, [batch, capacity, 4, 256].

    Sliding layers use a 512-slot ring (capacity is fixed at 512); full layers a
    contiguous cache whose capacity bounds the context.
    """

    def __init__(self, layer_type: int, batch: int, capacity: int | None = None, device="cuda",
                 k=None, v=None):
        torch = _torch()
        if layer_type == SLIDING:
            capacity = WINDOW if capacity is None else capacity
        elif capacity is None:
            raise ValueError("a full-layer cache needs a capacity")
        self.layer_type = int(layer_type)
        self.batch = int(batch)
        self.capacity = int(capacity)
        shape = (self.batch, self.capacity, N_KV_HEADS, HEAD_DIM)
        self.k = torch.zeros(shape, dtype=torch.bfloat16, device=device) if k is None else k
        self.v = torch.zeros(shape, dtype=torch.bfloat16, device=device) if v is None else v
        _check(self.k, "cache.k", shape, torch.bfloat16)
        _check(self.v, "cache.v", shape, torch.bfloat16)

    def desc(self) -> KvCacheDesc:
        return KvCacheDesc(self.k.data_ptr(), self.v.data_ptr(), self.batch, self.capacity)


class KVCacheQ8:
    """One layer's 8-bit KV cache (q8_0 blocks of 32 along head_dim): int8 codes
    [batch, capacity, 4, 256] and fp16 scales [batch, capacity, 4, 8] for K (post-RoPE)
    and for V.  Capacity rules as for KVCache."""

    def __init__(self, layer_type: int, batch: int, capacity: int | None = None, device="cuda",
                 k=None, k_scale=None, v=None, v_scale=None):
        torch = _torch()
        if layer_type == SLIDING:
            capacity = WINDOW if capacity is None else capacity
        elif capacity is None:
            raise ValueError("a full-layer cache needs a capacity")
        self.layer_type = int(layer_type)
        self.batch = int(batch)
        self.capacity = int(capacity)
        shape = (self.batch, self.capacity, N_KV_HEADS, HEAD_DIM)
        sshape = (self.batch, self.capacity, N_KV_HEADS, HEAD_DIM // 32)
        self.k = torch.zeros(shape, dtype=torch.int8, device=device) if k is None else k
        self.v = torch.zeros(shape, dtype=torch.int8, device=device) if v is None else v
        self.k_scale = torch.zeros(sshape, dtype=torch.float16, device=device) if k_scale is None else k_scale
        self.v_scale = torch.zeros(sshape, dtype=torch.float16, device=device) if v_scale is None else v_scale
        _check(self.k, "cache.k", shape, torch.int8)
        _check(self.v, "cache.v", shape, torch.int8)
        _check(self.k_scale, "cache.k_scale", sshape, torch.float16)
        _check(self.v_scale, "cache.v_scale", sshape, torch.float16)

    def desc(self) -> KvCacheQ8Desc:
        return KvCacheQ8Desc(self.k.data_ptr(), self.k_scale.data_ptr(), self.v.data_ptr(),
                             self.v_scale.data_ptr(), self.batch, self.capacity)


def prefill_workspace_bytes(layer_type: int, batch: int, seq_len: int) -> int:
    return int(_lib.spark_attn_prefill_workspace_bytes(int(layer_type), int(batch), int(seq_len)))


def prefill(layer_type: int, q, k, v, gate, out=None, cache: KVCache | None = None,
            start_pos: int = 0, workspace=None, stream=None):
    """spark_attn_prefill: q [B,S,16,256], k/v [B,S,4,256], gate [B,S,16] (bf16, pre-RoPE)
    of a chunk at positions start_pos .. start_pos+S-1 (start_pos > 0 reads the earlier
    positions from ``cache``); ``workspace`` (uint8, >= prefill_workspace_bytes) is
    allocated per call when omitted."""
    torch = _torch()
    B, S = int(q.shape[0]), int(q.shape[1])
    _check(q, "q", (B, S, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(k, "k", (B, S, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(v, "v", (B, S, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(gate, "gate", (B, S, N_Q_HEADS), torch.bfloat16)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", tuple(q.shape), torch.bfloat16)
    desc = None
    if cache is not None:
        if cache.layer_type != layer_type:
            raise ValueError("cache layer type differs from the call's")
        desc = ctypes.pointer(cache.desc())
    if workspace is None:
        need = prefill_workspace_bytes(layer_type, B, S)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", None, torch.uint8)
    st = _lib.spark_attn_prefill(int(layer_type), B, S, int(start_pos), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(gate), desc, _ptr(workspace), int(workspace.numel()),
                                 _ptr(out), _stream(stream))
    if st:
        raise SparkError(st, "spark_attn_prefill")
    return out


def prefill_varlen_workspace_bytes(layer_type: int, total_tokens: int) -> int:
    return int(_lib.spark_attn_prefill_varlen_workspace_bytes(int(layer_type), int(total_tokens)))


def prefill_varlen(layer_type: int, q, k, v, gate, cu_seqlens, max_seqlen: int, out=None,
                   cache: KVCache | None = None, workspace=None, stream=None):
    """spark_attn_prefill_varlen: sequences packed back to back, q [T,16,256], k/v [T,4,256],
    gate [T,16] (bf16, pre-RoPE); cu_seqlens device int32 [B+1] of token offsets."""
    torch = _torch()
    T = int(q.shape[0])
    _check(q, "q", (T, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(k, "k", (T, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(v, "v", (T, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(gate, "gate", (T, N_Q_HEADS), torch.bfloat16)
    _check(cu_seqlens, "cu_seqlens", None, torch.int32)
    B = int(cu_seqlens.shape[0]) - 1
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", tuple(q.shape), torch.bfloat16)
    desc = None
    if cache is not None:
        if cache.layer_type != layer_type:
            raise ValueError("cache layer type differs from the call's")
        desc = ctypes.pointer(cache.desc())
    if workspace is None:
        workspace = torch.empty(max(prefill_varlen_workspace_bytes(layer_type, T), 256), dtype=torch.uint8,
                                device=q.device)
    _check(workspace, "workspace", None, torch.uint8)
    st = _lib.spark_attn_prefill_varlen(int(layer_type), B, _ptr(cu_seqlens), T, int(max_seqlen), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(gate), desc, _ptr(workspace),
                                        int(workspace.numel()), _ptr(out), _stream(stream))
    if st:
        raise SparkError(st, "spark_attn_prefill_varlen")
    return out


def qkv_proj_fp8_workspace_bytes(tokens: int) -> int:
    return int(_lib.spark_qkv_proj_fp8_workspace_bytes(int(tokens)))


def qkv_proj_fp8(x, w_qkv, w_scale, w_gate, out=None, workspace=None, stream=None):
    """spark_qkv_proj_fp8: x [T,2560] bf16; w_qkv [6144,2560] uint8 E4M3FN codes; w_scale
    [6144] fp32; w_gate [16,2560] bf16.  Returns (q [T,16,256], k [T,4,256], v [T,4,256],
    gate logits [T,16]), all bf16."""
    torch = _torch()
    T = int(x.shape[0])
    _check(x, "x", (T, 2560), torch.bfloat16)
    _check(w_qkv, "w_qkv", (6144, 2560), torch.uint8)
    _check(w_scale, "w_scale", (6144,), torch.float32)
    _check(w_gate, "w_gate", (16, 2560), torch.bfloat16)
    if out is None:
        out = (torch.empty(T, N_Q_HEADS, HEAD_DIM, dtype=torch.bfloat16, device=x.device),
               torch.empty(T, N_KV_HEADS, HEAD_DIM, dtype=torch.bfloat16, device=x.device),
               torch.empty(T, N_KV_HEADS, HEAD_DIM, dtype=torch.bfloat16, device=x.device),
               torch.empty(T, N_Q_HEADS, dtype=torch.bfloat16, device=x.device))
    q, k, v, g = out
    _check(q, "q", (T, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(k, "k", (T, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(v, "v", (T, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(g, "gate", (T, N_Q_HEADS), torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(qkv_proj_fp8_workspace_bytes(T), dtype=torch.uint8, device=x.device)
    _check(workspace, "workspace", None, torch.uint8)
    st = _lib.spark_qkv_proj_fp8(T, _ptr(x), _ptr(w_qkv), _ptr(w_scale), _ptr(w_gate), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(g), _ptr(workspace), int(workspace.numel()), _stream(stream))
    if st:
        raise SparkError(st, "spark_qkv_proj_fp8")
    return q, k, v, g


def kv_append(layer_type: int, k, v, pos, cache: KVCache, stream=None):
    """spark_kv_append: k/v [B,n_new,4,256] (k pre-RoPE), pos device int32 [B]."""
    torch = _torch()
    B, n = int(k.shape[0]), int(k.shape[1])
    _check(k, "k", (B, n, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(v, "v", (B, n, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(pos, "pos", (B,), torch.int32)
    if cache.layer_type != layer_type:
        raise ValueError("cache layer type differs from the call's")
    st = _lib.spark_kv_append(int(layer_type), B, n, _ptr(k), _ptr(v), _ptr(pos),
                              ctypes.pointer(cache.desc()), _stream(stream))
    if st:
        raise SparkError(st, "spark_kv_append")


def decode_workspace_bytes(layer_type: int, batch: int, max_seq_len: int, num_parts: int = 0) -> int:
    return int(_lib.spark_attn_decode_workspace_bytes(int(layer_type), int(batch), int(max_seq_len),
                                                      int(num_parts)))


def decode(layer_type: int, q, gate, cache: KVCache, seq_lens, max_seq_len: int, out=None,
           workspace=None, num_parts: int = 0, stream=None):
    """spark_attn_decode: q [B,16,256] (pre-RoPE), gate [B,16], seq_lens device int32 [B];
    ``num_parts`` workgroups share the batch's keys (0: the library's choice)."""
    torch = _torch()
    B = int(q.shape[0])
    _check(q, "q", (B, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(gate, "gate", (B, N_Q_HEADS), torch.bfloat16)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    if cache.layer_type != layer_type:
        raise ValueError("cache layer type differs from the call's")
    need = decode_workspace_bytes(layer_type, B, max_seq_len, num_parts)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", None, torch.uint8)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", tuple(q.shape), torch.bfloat16)
    st = _lib.spark_attn_decode(int(layer_type), B, _ptr(q), _ptr(gate), ctypes.pointer(cache.desc()),
                                _ptr(seq_lens), int(max_seq_len), int(num_parts), _ptr(workspace),
                                int(workspace.numel()), _ptr(out), _stream(stream))
    if st:
        raise SparkError(st, "spark_attn_decode")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc(layer_type: int, q, gate, cache: KVCache, seq_lens, max_seq_len: int, out=None,
                   num_parts: int = 0, stream=None):
    """spark_attn_decode_noalloc: decode with the library's static device scratch instead of
    a workspace; arguments as for decode.  Calls that may overlap on one GPU race."""
    torch = _torch()
    B = int(q.shape[0])
    _check(q, "q", (B, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(gate, "gate", (B, N_Q_HEADS), torch.bfloat16)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    if cache.layer_type != layer_type:
        raise ValueError("cache layer type differs from the call's")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", tuple(q.shape), torch.bfloat16)
    st = _lib.spark_attn_decode_noalloc(int(layer_type), B, _ptr(q), _ptr(gate), ctypes.pointer(cache.desc()),
                                        _ptr(seq_lens), int(max_seq_len), int(num_parts), _ptr(out),
                                        _stream(stream))
    if st:
        raise SparkError(st, "spark_attn_decode_noalloc")
    return out


def kv_append_q8(layer_type: int, k, v, pos, cache: KVCacheQ8, stream=None):
    """spark_kv_append_q8: k/v [B,n_new,4,256] bf16 (k pre-RoPE), pos device int32 [B]."""
    torch = _torch()
    B, n = int(k.shape[0]), int(k.shape[1])
    _check(k, "k", (B, n, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(v, "v", (B, n, N_KV_HEADS, HEAD_DIM), torch.bfloat16)
    _check(pos, "pos", (B,), torch.int32)
    if cache.layer_type != layer_type:
        raise ValueError("cache layer type differs from the call's")
    st = _lib.spark_kv_append_q8(int(layer_type), B, n, _ptr(k), _ptr(v), _ptr(pos),
                                 ctypes.pointer(cache.desc()), _stream(stream))
    if st:
        raise SparkError(st, "spark_kv_append_q8")


def decode_q8_workspace_bytes(layer_type: int, batch: int, max_seq_len: int, num_parts: int = 0) -> int:
    return int(_lib.spark_attn_decode_q8_workspace_bytes(int(layer_type), int(batch), int(max_seq_len),
                                                         int(num_parts)))


def decode_q8(layer_type: int, q, gate, cache: KVCacheQ8, seq_lens, max_seq_len: int, out=None,
              workspace=None, num_parts: int = 0, stream=None):
    """spark_attn_decode_q8: decode against an 8-bit cache; arguments as for decode."""
    torch = _torch()
    B = int(q.shape[0])
    _check(q, "q", (B, N_Q_HEADS, HEAD_DIM), torch.bfloat16)
    _check(gate, "gate", (B, N_Q_HEADS), torch.bfloat16)
    _check(seq_lens, "seq_lens", (B,), torch.int32)
    if cache.layer_type != layer_type:
        raise ValueError("cache layer type differs from the call's")
    need = decode_q8_workspace_bytes(layer_type, B, max_seq_len, num_parts)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", None, torch.uint8)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", tuple(q.shape), torch.bfloat16)
    st = _lib.spark_attn_decode_q8(int(layer_type), B, _ptr(q), _ptr(gate), ctypes.pointer(cache.desc()),
                                   _ptr(seq_lens), int(max_seq_len), int(num_parts), _ptr(workspace),
                                   int(workspace.numel()), _ptr(out), _stream(stream))
    if st:
        raise SparkError(st, "spark_attn_decode_q8")
    return out


def layer_type_of(layer: int) -> int:
    """spark_layer_type_of: type of 0-based layer ``layer`` of the 36-layer stack."""
    lt = int(_lib.spark_layer_type_of(int(layer)))
    if lt < 0:
        raise ValueError(f"layer {layer} is outside the {N_LAYERS}-layer stack")
    return lt


def layer_params(layer_type: int):
    """spark_layer_params: (RoPE theta, rotated dims, window or None) of a layer type."""
    th, rd, w = ctypes.c_double(), ctypes.c_int32(), ctypes.c_int32()
    st = _lib.spark_layer_params(int(layer_type), ctypes.byref(th), ctypes.byref(rd), ctypes.byref(w))
    if st:
        raise SparkError(st, "spark_layer_params")
    return th.value, rd.value, (w.value or None)
