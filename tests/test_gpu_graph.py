"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A serving loop captures a decode step once and replays it; nothing in the captured calls
may depend on host work done at capture time.  The step here is, per layer of a 4-layer
slice of the stack (3 sliding, 1 full) at batch 64, the append of the new token's K/V and
the decode against the cache, in bf16 and in 8 bits, plus the full layer's decode through
the entry point without a workspace and a prefill call of each layer type that also writes
its cache.  Before each replay every output is filled with NaN and every decode cache is
restored to its state before the step (so a missed append shows in the decode output and
in the cache); eager work and a synchronisation run between replays, and each replay must
reproduce the eager calls' outputs and caches bit for bit (the kernels are deterministic;
the determinism tests check that)."""
import pytest

import synth
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    """The plain binding: graph capture needs calls that do not synchronise."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import full_gqa_attention_amd as m
    return m


def _normal(gen, shape):
    import torch
    return torch.randn(shape, generator=gen, device="cuda").bfloat16()


def _q8_cache(lib, gen, lt, B, cap):
    import torch
    codes = lambda: torch.randint(-127, 128, (B, cap, 4, 256), generator=gen, device="cuda", dtype=torch.int8)
    scales = lambda: (0.005 + 0.025 * torch.rand((B, cap, 4, 8), generator=gen, device="cuda")).half()
    return lib.KVCacheQ8(lt, B, cap, k=codes(), k_scale=scales(), v=codes(), v_scale=scales())


def test_step_graph_replays_match_eager(lib):
    import torch
    B, S = 64, 1536
    lens = synth.decode_seq_lens(synth.SEED_DECODE_B64 + 77, B, 600, 3000)
    maxlen = int(lens.max())
    sl = torch.as_tensor(lens).cuda()
    pos = (sl - 1).to(torch.int32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)

    calls, outputs, inouts = [], [], []   # closures that launch; tensors they write; caches they update
    for kv in ("bf16", "q8_0"):
        for layer in range(4):
            lt = lib.layer_type_of(layer)
            cap = 512 if lt == lib.SLIDING else maxlen
            if kv == "bf16":
                cache = lib.KVCache(lt, B, cap, k=_normal(gen, (B, cap, 4, 256)), v=_normal(gen, (B, cap, 4, 256)))
                ws = torch.empty(lib.decode_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
                append, dec = lib.kv_append, lib.decode
                written = [cache.k, cache.v]
            else:
                cache = _q8_cache(lib, gen, lt, B, cap)
                ws = torch.empty(lib.decode_q8_workspace_bytes(lt, B, maxlen), dtype=torch.uint8, device="cuda")
                append, dec = lib.kv_append_q8, lib.decode_q8
                written = [cache.k, cache.k_scale, cache.v, cache.v_scale]
            kn, vn = _normal(gen, (B, 1, 4, 256)), _normal(gen, (B, 1, 4, 256))
            q, g = _normal(gen, (B, 16, 256)), _normal(gen, (B, 16))
            out = torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")

            def call(lt=lt, cache=cache, ws=ws, append=append, dec=dec, kn=kn, vn=vn, q=q, g=g, out=out):
                append(lt, kn, vn, pos, cache)
                dec(lt, q, g, cache, sl, maxlen, out=out, workspace=ws)
            calls.append(call)
            outputs.append(out)
            inouts += written
            if kv == "bf16" and lt == lib.FULL:
                out_na = torch.empty_like(out)
                # The static scratch's device address is looked up on a device's first call,
                # which therefore runs before capture (in the eager pass below).
                calls.append(lambda lt=lt, cache=cache, q=q, g=g, out_na=out_na:
                             lib.decode_noalloc(lt, q, g, cache, sl, maxlen, out=out_na))
                outputs.append(out_na)
    for lt in (lib.SLIDING, lib.FULL):
        q, k, v = _normal(gen, (1, S, 16, 256)), _normal(gen, (1, S, 4, 256)), _normal(gen, (1, S, 4, 256))
        g = _normal(gen, (1, S, 16))
        cache = lib.KVCache(lt, 1, 512 if lt == lib.SLIDING else S)
        ws = torch.empty(lib.prefill_workspace_bytes(lt, 1, S), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)
        calls.append(lambda lt=lt, q=q, k=k, v=v, g=g, cache=cache, ws=ws, out=out:
                     lib.prefill(lt, q, k, v, g, out=out, cache=cache, workspace=ws))
        outputs += [out, cache.k, cache.v]

    def step():
        for c in calls:
            c()

    before = [t.clone() for t in inouts]
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs + inouts]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0xFF)        # NaN for bf16
        for t, b in zip(inouts, before):
            t.copy_(b)
        x = torch.randn(1 << 20, device="cuda")
        assert torch.isfinite(x.sum()).item()      # eager work and a synchronisation
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outputs + inouts, eager)):
            same = torch.equal(t.view(torch.uint8), e.view(torch.uint8))
            assert same, f"replay {rep}: output {i} {tuple(t.shape)} differs from the eager call"
    note(f"graph: {len(calls)} captured calls, 3 replays bit-identical to eager")
