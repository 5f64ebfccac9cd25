"""The binding as the GPU tests call it: guarded buffers.

Every output and workspace a call leaves to the binding is allocated fresh for that
call, filled with NaN bytes, and framed by guard bands of poison on both sides; caches
made through ``Guarded.KVCache`` / ``KVCacheQ8`` are framed the same way (their
interior holds the given contents, or zeros).  After every call the stream is
synchronised and:
  * each guard band must still hold the poison (nothing wrote outside its buffer);
  * a bf16 output must hold no poison (0xFFFF, a NaN the kernels never produce from
    finite inputs), so an element the kernels skipped fails the test even when a reused
    allocation happens to hold an earlier call's correct result.
Only allocation and checking happen here; the calls themselves go to the binding.
"""
from __future__ import annotations

import numpy as np

GUARD_BYTES = 4096          # keeps the interior 256-byte aligned
POISON = 0xFF               # every byte: bf16 0xFFFF and fp32 0xFFFFFFFF are NaN


class Framed:
    """A tensor of ``shape``/``dtype`` inside a uint8 buffer with a guard band on each side."""

    def __init__(self, shape, dtype, fill=None, device="cuda"):
        import torch
        shape = tuple(int(s) for s in shape)
        itemsize = torch.empty((), dtype=dtype).element_size()
        nbytes = int(np.prod(shape)) * itemsize if shape else itemsize
        self.nbytes = nbytes
        self.buf = torch.full((2 * GUARD_BYTES + max(nbytes, 1),), POISON, dtype=torch.uint8, device=device)
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(shape)
        if fill is not None:
            if isinstance(fill, str) and fill == "zeros":
                self.t.zero_()
            else:
                self.t.copy_(fill)

    def check_guards(self, what: str):
        head = self.buf[:GUARD_BYTES]
        tail = self.buf[GUARD_BYTES + self.nbytes:]
        bad_h = int((head != POISON).sum())
        bad_t = int((tail != POISON).sum())
        assert bad_h == 0 and bad_t == 0, (
            f"{what}: {bad_h} bytes before and {bad_t} bytes after the buffer were written")

    def check_written(self, what: str):
        """bf16 interior: no element may still hold the poison."""
        import torch
        left = int((self.t.view(torch.int16) == -1).sum())
        assert left == 0, f"{what}: {left} elements were never written"


class Guarded:
    """Proxy of the ``full_gqa_attention_amd`` module with guarded buffers (see above)."""

    def __init__(self, mod):
        self._m = mod

    def __getattr__(self, name):
        return getattr(self._m, name)

    # -- caches ------------------------------------------------------------------------
    def _cap(self, lt, capacity):
        if capacity is None and lt == self._m.SLIDING:
            return self._m.WINDOW
        return capacity

    def KVCache(self, layer_type, batch, capacity=None, device="cuda", k=None, v=None):
        import torch
        cap = self._cap(layer_type, capacity)
        if cap is None:
            return self._m.KVCache(layer_type, batch, capacity, device=device, k=k, v=v)
        shape = (batch, cap, self._m.N_KV_HEADS, self._m.HEAD_DIM)
        fk = Framed(shape, torch.bfloat16, "zeros" if k is None else k, device)
        fv = Framed(shape, torch.bfloat16, "zeros" if v is None else v, device)
        c = self._m.KVCache(layer_type, batch, cap, device=device, k=fk.t, v=fv.t)
        c._frames = (("cache.k", fk), ("cache.v", fv))
        return c

    def KVCacheQ8(self, layer_type, batch, capacity=None, device="cuda", k=None, k_scale=None, v=None,
                  v_scale=None):
        import torch
        cap = self._cap(layer_type, capacity)
        if cap is None:
            return self._m.KVCacheQ8(layer_type, batch, capacity, device=device, k=k, k_scale=k_scale, v=v,
                                     v_scale=v_scale)
        shape = (batch, cap, self._m.N_KV_HEADS, self._m.HEAD_DIM)
        sshape = (batch, cap, self._m.N_KV_HEADS, self._m.HEAD_DIM // 32)
        fr = [Framed(shape, torch.int8, "zeros" if k is None else k, device),
              Framed(sshape, torch.float16, "zeros" if k_scale is None else k_scale, device),
              Framed(shape, torch.int8, "zeros" if v is None else v, device),
              Framed(sshape, torch.float16, "zeros" if v_scale is None else v_scale, device)]
        c = self._m.KVCacheQ8(layer_type, batch, cap, device=device, k=fr[0].t, k_scale=fr[1].t, v=fr[2].t,
                              v_scale=fr[3].t)
        c._frames = tuple(zip(("cache.k", "cache.k_scale", "cache.v", "cache.v_scale"), fr))
        return c

    # -- helpers -----------------------------------------------------------------------
    @staticmethod
    def _workspace(nbytes, device):
        import torch
        return Framed((max(int(nbytes), 256),), torch.uint8, None, device)

    @staticmethod
    def _finish(what, outs=(), others=(), cache=None):
        import torch
        torch.cuda.synchronize()
        for name, f in outs:
            f.check_guards(f"{what} {name}")
            f.check_written(f"{what} {name}")
        for name, f in others:
            f.check_guards(f"{what} {name}")
        for name, f in getattr(cache, "_frames", ()):
            f.check_guards(f"{what} {name}")

    # -- calls -------------------------------------------------------------------------
    def prefill(self, layer_type, q, k, v, gate, out=None, cache=None, start_pos=0, workspace=None,
                stream=None):
        import torch
        fo = Framed(q.shape, torch.bfloat16, None, q.device) if out is None else None
        fw = None
        if workspace is None:
            fw = self._workspace(self._m.prefill_workspace_bytes(layer_type, q.shape[0], q.shape[1]), q.device)
        res = self._m.prefill(layer_type, q, k, v, gate, out=fo.t if fo else out, cache=cache,
                              start_pos=start_pos, workspace=fw.t if fw else workspace, stream=stream)
        self._finish("prefill", [("out", fo)] if fo else [], [("workspace", fw)] if fw else [], cache)
        return res

    def prefill_varlen(self, layer_type, q, k, v, gate, cu_seqlens, max_seqlen, out=None, cache=None,
                       workspace=None, stream=None):
        import torch
        fo = Framed(q.shape, torch.bfloat16, None, q.device) if out is None else None
        fw = None
        if workspace is None:
            fw = self._workspace(self._m.prefill_varlen_workspace_bytes(layer_type, q.shape[0]), q.device)
        res = self._m.prefill_varlen(layer_type, q, k, v, gate, cu_seqlens, max_seqlen, out=fo.t if fo else out,
                                     cache=cache, workspace=fw.t if fw else workspace, stream=stream)
        self._finish("prefill_varlen", [("out", fo)] if fo else [], [("workspace", fw)] if fw else [], cache)
        return res

    def _decode(self, fn, ws_fn, what, layer_type, q, gate, cache, seq_lens, max_seq_len, out, workspace,
                num_parts, stream):
        import torch
        fo = Framed(q.shape, torch.bfloat16, None, q.device) if out is None else None
        fw = None
        if workspace is None:
            fw = self._workspace(ws_fn(layer_type, q.shape[0], max_seq_len, num_parts), q.device)
        res = fn(layer_type, q, gate, cache, seq_lens, max_seq_len, out=fo.t if fo else out,
                 workspace=fw.t if fw else workspace, num_parts=num_parts, stream=stream)
        self._finish(what, [("out", fo)] if fo else [], [("workspace", fw)] if fw else [], cache)
        return res

    def decode(self, layer_type, q, gate, cache, seq_lens, max_seq_len, out=None, workspace=None,
               num_parts=0, stream=None):
        return self._decode(self._m.decode, self._m.decode_workspace_bytes, "decode", layer_type, q, gate,
                            cache, seq_lens, max_seq_len, out, workspace, num_parts, stream)

    def decode_q8(self, layer_type, q, gate, cache, seq_lens, max_seq_len, out=None, workspace=None,
                  num_parts=0, stream=None):
        return self._decode(self._m.decode_q8, self._m.decode_q8_workspace_bytes, "decode_q8", layer_type, q,
                            gate, cache, seq_lens, max_seq_len, out, workspace, num_parts, stream)

    def kv_append(self, layer_type, k, v, pos, cache, stream=None):
        self._m.kv_append(layer_type, k, v, pos, cache, stream=stream)
        self._finish("kv_append", cache=cache)

    def kv_append_q8(self, layer_type, k, v, pos, cache, stream=None):
        self._m.kv_append_q8(layer_type, k, v, pos, cache, stream=stream)
        self._finish("kv_append_q8", cache=cache)

    def qkv_proj_fp8(self, x, w_qkv, w_scale, w_gate, out=None, workspace=None, stream=None):
        import torch
        T = int(x.shape[0])
        m = self._m
        fos = None
        if out is None:
            fos = [Framed((T, m.N_Q_HEADS, m.HEAD_DIM), torch.bfloat16, None, x.device),
                   Framed((T, m.N_KV_HEADS, m.HEAD_DIM), torch.bfloat16, None, x.device),
                   Framed((T, m.N_KV_HEADS, m.HEAD_DIM), torch.bfloat16, None, x.device),
                   Framed((T, m.N_Q_HEADS), torch.bfloat16, None, x.device)]
            out = tuple(f.t for f in fos)
        fw = self._workspace(m.qkv_proj_fp8_workspace_bytes(T), x.device) if workspace is None else None
        res = m.qkv_proj_fp8(x, w_qkv, w_scale, w_gate, out=out, workspace=fw.t if fw else workspace,
                             stream=stream)
        self._finish("qkv_proj_fp8", list(zip(("q", "k", "v", "gate"), fos)) if fos else [],
                     [("workspace", fw)] if fw else [])
        return res
