"""W8A8 FP8 q_k_v_proj and bf16 g_proj through the C ABI against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import f64_of, note, to_dev

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _assert_close(got, want, what, sum_abs):
    """bf16 outputs of long sums: within one bf16 rounding of the exact value (2^-9
    relative, taken as 2^-8) plus 2^-16 of the sum of the terms' magnitudes -- the dot
    product bound; the FP8 MFMA adds the 64 products of a step at less than fp32 precision
    (about 2^-18 of that sum was seen), the gate's bf16 MFMA (fp32 sums) far less.  Relative L2 <= 5e-3."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = 2.0 ** -8 * np.abs(want) + 2.0 ** -16 * sum_abs
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    # A zero bound (an all-zero token: every term is 0) admits only an exact 0.
    ratio = np.divide(err, bound, out=np.where(err > 0, np.inf, 0.0), where=bound > 0)
    wi = int(np.argmax(ratio))
    worst = float(ratio.flat[wi])
    note(f"[proj] {what}: max |err|/bound = {worst:.3f} (err {err.flat[wi]:.3e} at |y| = "
         f"{abs(want.flat[wi]):.3e}), max err {err.max():.3e}, rel_l2 = {rel:.2e}")
    assert worst <= 1.0, f"{what}: an element is beyond one bf16 rounding"
    assert rel <= 5e-3, f"{what}: relative L2 {rel:.2e}"


def _sum_abs(inp, rows=None):
    """Sum of |term| of every output: s_x s_w sum_k |x_k w_k| (FP8 values), and for the
    gate sum_k |x_k wg_k| (bf16 values)."""
    x = inp["x"] if rows is None else inp["x"][rows]
    codes, s = oracle.quantize_tokens(x)
    T = x.shape[0]
    y = (np.abs(oracle.e4m3fn_decode(codes)) @ np.abs(oracle.e4m3fn_decode(inp["w"])).T
         * s.astype(np.float64)[:, None] * inp["w_scale"].astype(np.float64)[None, :])
    g = np.abs(oracle.bf16_to_f64(x)) @ np.abs(oracle.bf16_to_f64(inp["wg"])).T
    return (y[:, :4096].reshape(T, 16, 256), y[:, 4096:5120].reshape(T, 4, 256),
            y[:, 5120:].reshape(T, 4, 256), g)


def _run(fga, inp):
    import torch
    T = inp["x"].shape[0]
    ws = torch.zeros(fga.qkv_proj_fp8_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    q, k, v, g = fga.qkv_proj_fp8(to_dev(inp["x"]), _dev(inp["w"]), _dev(inp["w_scale"]), to_dev(inp["wg"]),
                                  workspace=ws)
    torch.cuda.synchronize()
    return q, k, v, g, ws.cpu().numpy()


@pytest.mark.parametrize("T", [1, 5, 127, 128, 129, 300, 1000])
def test_qkv_proj_all_rows(fga, T):
    note(f"qkv proj T={T}")
    inp = synth.proj_inputs(9100 + T, T)
    q, k, v, g, ws = _run(fga, inp)
    codes, scales = oracle.quantize_tokens(inp["x"])
    pad = (T * 2560 + 255) // 256 * 256
    assert np.array_equal(ws[:T * 2560].reshape(T, 2560), codes), "activation codes differ"
    assert np.array_equal(ws[pad:pad + 4 * T].view(np.float32), scales), "activation scales differ"
    wq, wk, wv, wg = oracle.qkv_proj(inp["x"], inp["w"], inp["w_scale"], inp["wg"])
    sq, sk, sv, sg = _sum_abs(inp)
    _assert_close(f64_of(q), wq, f"q T={T}", sq)
    _assert_close(f64_of(k), wk, f"k T={T}", sk)
    _assert_close(f64_of(v), wv, f"v T={T}", sv)
    _assert_close(f64_of(g), wg, f"gate T={T}", sg)


@pytest.mark.parametrize("T", [8192, 32768])
def test_qkv_proj_sampled_rows(fga, T):
    """The benchmark's shapes, 8192 and 32768 tokens: 96 sampled tokens against the oracle
    (tokens are independent: quantisation and products are per token)."""
    inp = synth.proj_inputs(9200 + T, T)
    q, k, v, g, _ = _run(fga, inp)
    rows = np.unique(np.concatenate([[0, 255, 256, T - 1], np.random.default_rng(9201).choice(T, 92, replace=False)]))
    wq, wk, wv, wg = oracle.qkv_proj(inp["x"][rows], inp["w"], inp["w_scale"], inp["wg"])
    sums = _sum_abs(inp, rows)
    for name, got, want, sa in zip(("q", "k", "v", "gate"), (q, k, v, g), (wq, wk, wv, wg), sums):
        _assert_close(f64_of(got[rows]), want, f"{name} T={T} sampled", sa)


def test_projection_feeds_prefill(fga):
    """q, k, v and the gate logits from the projection go straight into the prefill."""
    import torch
    T = 300
    inp = synth.proj_inputs(9300, T)
    q, k, v, g, _ = _run(fga, inp)
    out = fga.prefill(oracle.FULL, q[None], k[None], v[None], g[None])
    torch.cuda.synchronize()
    from gpu_util import assert_parity, bits_of
    want = oracle.prefill(bits_of(q)[None], bits_of(k)[None], bits_of(v)[None], bits_of(g)[None], oracle.FULL)
    assert_parity(f64_of(out), want, "projection -> prefill")


def test_qkv_proj_degenerate_tokens(fga):
    """Tokens the per-token quantiser treats specially, in a batch of 260 (two GEMM row
    tiles, the second ragged): an all-zero token (scale 0, codes 0, outputs 0), a token whose
    only non-zero value is a large outlier, a constant token (every code +-448) and a token
    of tiny values.  Codes and scales bit for bit, outputs to the usual bound."""
    T = 260
    inp = synth.proj_inputs(9400, T)
    x = oracle.bf16_to_f64(inp["x"]).copy()
    x[0] = 0.0
    x[1] = 0.0
    x[1, 1234] = 3.0e4
    x[2] = -1.5
    x[T - 1] *= 1e-20
    inp["x"] = oracle.round_to_bf16_bits(x)
    q, k, v, g, ws = _run(fga, inp)
    codes, scales = oracle.quantize_tokens(inp["x"])
    assert scales[0] == 0.0 and not codes[0].any()
    assert np.all((codes[2] == 0xFE))
    pad = (T * 2560 + 255) // 256 * 256
    got_codes = ws[:T * 2560].reshape(T, 2560)
    got_scales = ws[pad:pad + 4 * T].view(np.float32)
    bad = np.argwhere(got_codes != codes)
    assert bad.size == 0, f"activation codes differ at (token, k) {bad[:5].tolist()}"
    assert np.array_equal(got_scales, scales), "activation scales differ"
    wq, wk, wv, wg = oracle.qkv_proj(inp["x"], inp["w"], inp["w_scale"], inp["wg"])
    assert not f64_of(q)[0].any() and not f64_of(g)[0].any(), "a zero token must project to zeros"
    sq, sk, sv, sg = _sum_abs(inp)
    for name, got, want, sa in zip(("q", "k", "v", "gate"), (q, k, v, g), (wq, wk, wv, wg), (sq, sk, sv, sg)):
        _assert_close(f64_of(got), want, f"{name} degenerate tokens", sa)
