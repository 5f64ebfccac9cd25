"""One decode step of the whole 36-layer stack (27 ring layers, 9 full layers, layer l
full iff l mod 4 = 3), each layer with its own cache, bf16 and 8-bit: every layer's
output against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, f64_of, i32_dev, note, to_dev

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("kv", ["bf16", "q8_0"])
def test_decode_step_36_layers(fga, kv):
    import torch
    B = 3
    lens = np.array([1, 700, 1300], np.int32)
    outs, wants = [], []
    for layer in range(36):
        lt = fga.layer_type_of(layer)
        assert lt == oracle.layer_type_of(layer)
        seed = 9000 + layer
        q = synth.normal_bf16(seed, 0, (B, 16, 256))
        g = synth.normal_bf16(seed, 1, (B, 16))
        cap = 512 if lt == oracle.SLIDING else int(lens.max())
        if kv == "bf16":
            d = synth.decode_inputs(seed, B, cap)
            cache = fga.KVCache(lt, B, cap, k=to_dev(d["cache_k"]), v=to_dev(d["cache_v"]))
            out = fga.decode(lt, to_dev(q), to_dev(g), cache, i32_dev(lens), int(lens.max()))
            want = oracle.decode(q, g, d["cache_k"], d["cache_v"], lens, lt)
        else:
            arrs = [np.stack(x) for x in zip(*(synth.q8_cache_rows(seed, b, cap) for b in range(B)))]
            cache = fga.KVCacheQ8(lt, B, cap, k=_dev(arrs[0]), k_scale=_dev(arrs[1]), v=_dev(arrs[2]),
                                  v_scale=_dev(arrs[3]))
            out = fga.decode_q8(lt, to_dev(q), to_dev(g), cache, i32_dev(lens), int(lens.max()))
            want = oracle.decode_q8(q, g, *arrs, lens, lt)
        outs.append(out)
        wants.append(want)
    torch.cuda.synchronize()
    note(f"decode step, 36 layers, {kv} cache")
    for layer, (o, w) in enumerate(zip(outs, wants)):
        assert_parity(f64_of(o), w, f"decode step layer {layer} ({kv})")
