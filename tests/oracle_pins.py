"""Checks that pin the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes the oracle's attention module (``att``) and raises
AssertionError when the oracle disagrees with:
  * a brute-force computation on tiny inputs written differently (explicit key lists,
    complex-number rotation, ``math`` scalars);
  * closed forms (window 1, row 0, constant values, zero queries, gate limits);
  * invariants (window >= length equals causal; GQA equals repeated KV heads; RoPE
    preserves norms, depends on position differences only, leaves the unrotated
    dims of full layers bit-identical);
  * a library routine (torch's CPU fp64 scaled_dot_product_attention);
  * the KV-cache sizes printed on the pages (``tests/golden/kv_footprint_pages.json``).
``tests/test_oracle_pins.py`` runs them on the real oracle and
``tests/test_oracle_mutants.py`` runs them on oracles with a planted mistake.
"""
from __future__ import annotations

import cmath
import json
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def _small_inputs(seed, B, S, H, Hk, D):
    return {
        "q": synth.normal_bf16(seed, 0, (B, S, H, D)),
        "k": synth.normal_bf16(seed, 1, (B, S, Hk, D)),
        "v": synth.normal_bf16(seed, 2, (B, S, Hk, D)),
        "gate": synth.normal_bf16(seed, 3, (B, S, H)),
    }


def _rotate_complex(vec, p, theta, rot_dim):
    """RoPE of one vector through complex multiplication (independent formulation)."""
    half = rot_dim // 2
    out = list(vec)
    for m in range(half):
        w = theta ** (-(2.0 * m) / rot_dim)
        z = complex(vec[m], vec[m + half]) * cmath.exp(1j * p * w)
        out[m], out[m + half] = z.real, z.imag
    return out


def brute_prefill(inp, theta, rot_dim, window):
    """Loop-by-loop prefill on tiny inputs: explicit key lists, math scalars."""
    q, k, v, gate = (_f64(inp[n]) for n in ("q", "k", "v", "gate"))
    B, S, H, D = q.shape
    Hk = k.shape[2]
    out = np.zeros_like(q)
    for b in range(B):
        for i in range(S):
            for h in range(H):
                g = (h * Hk) // H
                qi = _rotate_complex(q[b, i, h], i, theta, rot_dim)
                keys = [j for j in range(S) if j <= i and (window is None or i - j < window)]
                scores = []
                for j in keys:
                    kj = _rotate_complex(k[b, j, g], j, theta, rot_dim)
                    scores.append(sum(qi[d] * kj[d] for d in range(D)) / math.sqrt(D))
                mx = max(scores)
                e = [math.exp(s - mx) for s in scores]
                z = sum(e)
                sig = 1.0 / (1.0 + math.exp(-gate[b, i, h]))
                for d in range(D):
                    out[b, i, h, d] = sig * sum(e[t] * v[b, keys[t], g, d] for t in range(len(keys))) / z
    return out


def _close(a, b, tol=1e-10, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------- masks / softmax


def pin_brute_force_tiny(att):
    """Tiny shapes, several windows and rotary widths, against the loop version."""
    inp = _small_inputs(11, 2, 9, 4, 2, 8)
    for theta, rd in ((10.0, 8), (10000.0, 4)):
        for w in (1, 3, 512, None):
            got = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], att.SLIDING,
                              theta=theta, rot_dim=rd, window=w)
            _close(got, brute_prefill(inp, theta, rd, w), 1e-12, f"brute theta={theta} r={rd} W={w}")


def pin_brute_force_real_heads(att):
    """The model's real head layout and per-type RoPE on a short sequence."""
    inp = _small_inputs(12, 1, 5, 16, 4, 256)
    for lt, theta, rd in ((att.SLIDING, 1e4, 256), (att.FULL, 5e6, 64)):
        got = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt)
        _close(got, brute_prefill(inp, theta, rd, None), 1e-11, f"brute real heads lt={lt}")


def pin_window_covering_sequence_is_causal(att):
    inp = _small_inputs(13, 1, 40, 4, 2, 16)
    a = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], att.SLIDING, theta=1e4, rot_dim=16, window=40)
    b = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], att.SLIDING, theta=1e4, rot_dim=16, window=None)
    _close(a, b, 0.0, "window >= S vs causal")
    c = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], att.SLIDING, theta=1e4, rot_dim=16, window=39)
    assert np.max(np.abs(c[:, 39] - b[:, 39])) > 1e-6, "window 39 must hide key 0 from row 39"


def pin_window_one_closed_form(att):
    """W = 1: each row sees only itself, so out = sigmoid(g) * v[i]."""
    inp = _small_inputs(14, 2, 12, 8, 2, 16)
    got = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], att.SLIDING, theta=1e4, rot_dim=16, window=1)
    v = _f64(inp["v"])
    sig = 1.0 / (1.0 + np.exp(-_f64(inp["gate"])))
    want = sig[..., None] * np.repeat(v, 4, axis=2)
    _close(got, want, 1e-14, "W=1")


def pin_row_zero_closed_form(att):
    inp = _small_inputs(15, 1, 70, 16, 4, 256)
    v = _f64(inp["v"])
    sig = 1.0 / (1.0 + np.exp(-_f64(inp["gate"])))
    for lt in (att.SLIDING, att.FULL):
        got = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=[0])
        want = sig[:, 0, :, None] * np.repeat(v[:, 0], 4, axis=1)
        _close(got[:, 0], want, 1e-14, f"row 0 lt={lt}")


def pin_constant_values(att):
    """All value rows equal: any softmax weights give that row back (times the gate)."""
    inp = _small_inputs(16, 1, 33, 16, 4, 256)
    v = np.broadcast_to(inp["v"][:, :1], inp["v"].shape).copy()
    sig = 1.0 / (1.0 + np.exp(-_f64(inp["gate"])))
    for lt in (att.SLIDING, att.FULL):
        got = att.prefill(inp["q"], inp["k"], v, inp["gate"], lt)
        want = sig[..., None] * np.repeat(_f64(v), 4, axis=2)
        _close(got, want, 1e-13, f"constant V lt={lt}")


def pin_zero_query_uniform_mean(att):
    """q = 0 gives equal weights: the plain mean of the visible values (window exact)."""
    S = 600
    inp = _small_inputs(17, 1, S, 16, 4, 256)
    q0 = np.zeros_like(inp["q"])
    v = _f64(inp["v"])
    rows = [0, 1, 510, 511, 512, 513, 599]
    sig = 1.0 / (1.0 + np.exp(-_f64(inp["gate"])))
    for lt, lo_fn in ((att.SLIDING, lambda i: max(0, i - 511)), (att.FULL, lambda i: 0)):
        got = att.prefill(q0, inp["k"], inp["v"], inp["gate"], lt, rows=rows)
        for r, i in enumerate(rows):
            mean = v[0, lo_fn(i):i + 1].mean(axis=0)                  # [4, 256]
            want = sig[0, i, :, None] * np.repeat(mean, 4, axis=0)
            _close(got[0, r], want, 1e-12, f"zero q lt={lt} row {i}")


def pin_gate_limits(att):
    inp = _small_inputs(18, 1, 20, 16, 4, 256)
    g0 = np.zeros_like(inp["gate"])
    gbig = np.full_like(inp["gate"], synth.f32_to_bf16_bits(np.array([60.0], np.float32))[0])
    half = att.prefill(inp["q"], inp["k"], inp["v"], g0, att.FULL)
    full = att.prefill(inp["q"], inp["k"], inp["v"], gbig, att.FULL)
    _close(half, 0.5 * full, 1e-12, "gate 0 = half of gate +inf")
    gneg = np.full_like(inp["gate"], synth.f32_to_bf16_bits(np.array([-60.0], np.float32))[0])
    assert np.max(np.abs(att.prefill(inp["q"], inp["k"], inp["v"], gneg, att.FULL))) < 1e-20


def pin_gqa_equals_repeated_kv(att):
    inp = _small_inputs(19, 1, 24, 16, 4, 256)
    rep = {n: np.repeat(inp[n], 4, axis=2) for n in ("k", "v")}
    for lt in (att.SLIDING, att.FULL):
        a = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt)
        b = att.prefill(inp["q"], rep["k"], rep["v"], inp["gate"], lt)
        _close(a, b, 0.0, f"GQA vs repeat_interleave lt={lt}")


def pin_torch_sdpa(att):
    """torch CPU fp64 scaled_dot_product_attention (default scale) on the same rotation."""
    import torch

    S, W = 80, 17
    inp = _small_inputs(20, 1, S, 16, 4, 256)
    q, k, v = (_f64(inp[n])[0] for n in ("q", "k", "v"))
    sig = 1.0 / (1.0 + np.exp(-_f64(inp["gate"])[0]))
    for lt, theta, rd, w in ((att.SLIDING, 1e4, 256, W), (att.FULL, 5e6, 64, None)):
        qr = np.array([[_rotate_complex(q[i, h], i, theta, rd) for h in range(16)] for i in range(S)])
        kr = np.array([[_rotate_complex(k[i, g], i, theta, rd) for g in range(4)] for i in range(S)])
        Q = torch.from_numpy(qr).permute(1, 0, 2)                             # [16, S, D]
        K = torch.from_numpy(kr).permute(1, 0, 2).repeat_interleave(4, dim=0)
        V = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(4, dim=0)
        ones = torch.ones(S, S, dtype=torch.bool)
        mask = torch.tril(ones)
        if w is not None:
            mask &= torch.triu(ones, diagonal=-(w - 1))
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        ref = ref.permute(1, 0, 2).numpy() * sig[..., None]
        got = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, window=w)[0] \
            if lt == att.SLIDING else att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt)[0]
        _close(got, ref, 1e-12, f"torch sdpa lt={lt}")


# --------------------------------------------------------------------------- RoPE


def pin_rope_properties(att):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 3, 256))
    big = 2 ** 20 - 4096
    for lt in (att.SLIDING, att.FULL):
        theta, rd, _ = att.layer_params(lt)
        pos = np.array([0, 1, 7, 511, 131071, 2 ** 20 - 1])
        y = att.rope(x, pos, theta, rd)
        assert np.array_equal(y[0], x[0]), "position 0 must be the identity"
        _close(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), 1e-12, "norm")
        half = rd // 2
        pn = lambda a: np.hypot(a[..., :half], a[..., half:rd])  # noqa: E731
        _close(pn(y), pn(x), 1e-12, "per-pair norm")
        assert np.array_equal(y[..., rd:], x[..., rd:]), "unrotated dims must be bit-identical"
        # q.k depends only on the position difference
        a, b = x[:1, :1], x[1:2, :1]
        for t in (1, 1000, big):
            d0 = np.sum(att.rope(a, [5], theta, rd) * att.rope(b, [3], theta, rd))
            d1 = np.sum(att.rope(a, [5 + t], theta, rd) * att.rope(b, [3 + t], theta, rd))
            _close(d0, d1, 1e-9, f"relative position t={t}")
        # complex-multiplication formulation
        for i, p in enumerate(pos):
            want = _rotate_complex(list(x[i, 0]), float(p), theta, rd)
            _close(y[i, 0], want, 1e-9, f"complex form p={p}")
    theta, rd, _ = att.layer_params(att.FULL)
    assert rd == 64, "full layers rotate the first 64 of 256 dims (factor 0.25)"


def pin_rope_frequencies(att):
    """Frequencies read off R_1(e_m): first is 1, geometric with ratio theta**(-2/r)."""
    for lt in (att.SLIDING, att.FULL):
        theta, rd, _ = att.layer_params(lt)
        half = rd // 2
        e = np.zeros((half, 1, 256))
        e[np.arange(half), 0, np.arange(half)] = 1.0
        y = att.rope(e, np.ones(half), theta, rd)
        w = np.arctan2(y[np.arange(half), 0, np.arange(half) + half], y[np.arange(half), 0, np.arange(half)])
        assert abs(w[0] - 1.0) < 1e-15
        ratio = w[1:] / w[:-1]
        _close(ratio, np.full(half - 1, theta ** (-2.0 / rd)), 1e-12, "frequency ratio")


def pin_layer_schedule(att):
    t = att.layer_types(36)
    assert len(t) == 36 and t.count(att.FULL) == 9 and t.count(att.SLIDING) == 27
    assert t[35] == att.FULL, "the last layer is full"
    assert all(t[4 * g:4 * g + 3] == [att.SLIDING] * 3 for g in range(9)), "3 sliding then 1 full"
    assert att.layer_params(att.SLIDING) == (1e4, 256, 512)
    assert att.layer_params(att.FULL)[:2] == (5e6, 64) and att.layer_params(att.FULL)[2] is None


# --------------------------------------------------------------------------- cache / decode


def pin_bf16_rounding(att):
    one = 1.0
    cases = {one + 2 ** -8: one, one + 3 * 2 ** -8: one + 2 ** -6, -(one + 2 ** -8): -one,
             2.0 ** -130: 2.0 ** -130, 3 * 2.0 ** -134: 2 * 2.0 ** -133, 0.0: 0.0}
    for x, want in cases.items():
        got = _f64(att.round_to_bf16_bits(np.array([x])))[0]
        assert got == want, f"bf16 rounding of {x!r}: {got!r} != {want!r}"
    x = np.random.default_rng(22).standard_normal(200000) * 3
    r = _f64(att.round_to_bf16_bits(x))
    ulp = np.ldexp(1.0, np.frexp(x)[1] - 8)
    assert np.all(np.abs(r - x) <= ulp / 2), "nearest rounding"
    x32 = x.astype(np.float32)
    assert np.array_equal(att.round_to_bf16_bits(x32.astype(np.float64)), synth.f32_to_bf16_bits(x32))


def pin_kv_append(att):
    B, cap = 2, 40
    rng_bits = synth.normal_bf16(23, 0, (B, cap, 4, 256))
    ck0, cv0 = rng_bits.copy(), synth.normal_bf16(23, 1, (B, cap, 4, 256))
    n = 6
    k = synth.normal_bf16(23, 2, (B, n, 4, 256))
    v = synth.normal_bf16(23, 3, (B, n, 4, 256))
    pos = np.array([0, 30], dtype=np.int32)
    ck, cv = att.kv_append(ck0, cv0, k, v, pos, att.FULL)
    for b in range(B):
        written = set(range(pos[b], pos[b] + n))
        for s in range(cap):
            if s in written:
                t = s - pos[b]
                assert np.array_equal(cv[b, s], v[b, t])
                exact = np.array([_rotate_complex(list(_f64(k[b, t, g])), float(s), 5e6, 64) for g in range(4)])
                ulp = np.ldexp(1.0, np.frexp(exact)[1] - 8)
                assert np.all(np.abs(_f64(ck[b, s]) - exact) <= ulp / 2 + 1e-300)
            else:
                assert np.array_equal(ck[b, s], ck0[b, s]) and np.array_equal(cv[b, s], cv0[b, s])
    # ring: 700 tokens from position 100 leave positions 288..799 in slots p mod 512
    kr = synth.normal_bf16(24, 0, (1, 700, 4, 256))
    vr = synth.normal_bf16(24, 1, (1, 700, 4, 256))
    ring_k = np.zeros((1, 512, 4, 256), np.uint16)
    rk, rv = att.kv_append(ring_k, ring_k.copy(), kr, vr, np.array([100]), att.SLIDING)
    for p in range(288, 800):
        assert np.array_equal(rv[0, p % 512], vr[0, p - 100]), f"ring slot of position {p}"
    p = 799
    exact = np.array([_rotate_complex(list(_f64(kr[0, p - 100, g])), float(p), 1e4, 256) for g in range(4)])
    ulp = np.ldexp(1.0, np.frexp(exact)[1] - 8)
    assert np.all(np.abs(_f64(rk[0, p % 512]) - exact) <= ulp / 2)


def _brute_decode_one(q, gate, ck, cv, positions_slots, qp, theta, rot_dim):
    """One sequence, loops over the visible (position, slot) list."""
    out = np.zeros((16, 256))
    for h in range(16):
        g = (h * 4) // 16
        qr = _rotate_complex(list(q[h]), float(qp), theta, rot_dim)
        sc = [sum(qr[d] * ck[s, g, d] for d in range(256)) / 16.0 for _, s in positions_slots]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = sum(e)
        sig = 1.0 / (1.0 + math.exp(-gate[h]))
        acc = np.zeros(256)
        for t, (_, s) in enumerate(positions_slots):
            acc += e[t] * cv[s, g]
        out[h] = sig * acc / z
    return out


def pin_decode_brute(att):
    B = 3
    lens = np.array([1, 300, 530], dtype=np.int32)
    d = synth.decode_inputs(25, B, 600)
    ring = {n: np.zeros((B, 512, 4, 256), np.uint16) for n in ("k", "v")}
    for b in range(B):
        for p in range(max(0, lens[b] - 512), lens[b]):
            ring["k"][b, p % 512] = d["cache_k"][b, p]
            ring["v"][b, p % 512] = d["cache_v"][b, p]
    got_full = att.decode(d["q"], d["gate"], d["cache_k"], d["cache_v"], lens, att.FULL)
    got_ring = att.decode(d["q"], d["gate"], ring["k"], ring["v"], lens, att.SLIDING)
    q, g = _f64(d["q"]), _f64(d["gate"])
    for b in range(B):
        L = int(lens[b])
        ps = [(p, p) for p in range(L)]
        want = _brute_decode_one(q[b], g[b], _f64(d["cache_k"][b]), _f64(d["cache_v"][b]), ps, L - 1, 5e6, 64)
        _close(got_full[b], want, 1e-11, f"decode full b={b}")
        ps = [(p, p % 512) for p in range(max(0, L - 512), L)]
        want = _brute_decode_one(q[b], g[b], _f64(ring["k"][b]), _f64(ring["v"][b]), ps, L - 1, 1e4, 256)
        _close(got_ring[b], want, 1e-11, f"decode ring b={b}")
    sig = 1.0 / (1.0 + np.exp(-g[0]))
    _close(got_full[0], sig[:, None] * np.repeat(_f64(d["cache_v"][0, 0]), 4, axis=0), 1e-14, "L=1")


def pin_decode_matches_prefill_row(att):
    """Prefill then append the same K/V: decode at L equals prefill row L-1 up to the
    bf16 rounding of cached keys."""
    S = 530
    inp = _small_inputs(26, 1, S, 16, 4, 256)
    for lt, cap in ((att.FULL, S), (att.SLIDING, 512)):
        ck = np.zeros((1, cap, 4, 256), np.uint16)
        ck, cv = att.kv_append(ck, ck.copy(), inp["k"], inp["v"], np.array([0]), lt)
        dec = att.decode(inp["q"][:, S - 1], inp["gate"][:, S - 1], ck, cv, np.array([S]), lt)
        pre = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=[S - 1])[:, 0]
        rel = np.linalg.norm(dec - pre) / np.linalg.norm(pre)
        assert rel < 5e-3, f"decode vs prefill row lt={lt}: rel {rel:.2e}"


# --------------------------------------------------------------------------- chunked prefill


def _chunk_case(seed, P, n, lt, att):
    """A sequence of P + n tokens whose first P sit in a cache written by the oracle's own
    append (full cache of P + n slots, or the 512-slot ring)."""
    inp = _small_inputs(seed, 1, P + n, 16, 4, 256)
    cap = P + n if lt == att.FULL else 512
    z = np.zeros((1, cap, 4, 256), np.uint16)
    ck, cv = att.kv_append(z, z.copy(), inp["k"][:, :P], inp["v"][:, :P], np.array([0]), lt)
    chunk = {name: inp[name][:, P:] for name in ("q", "k", "v", "gate")}
    return inp, chunk, ck, cv


def pin_chunk_start_zero_is_prefill(att):
    """With no cached prefix a chunk is an ordinary prefill."""
    inp = _small_inputs(31, 2, 37, 16, 4, 256)
    for lt in (att.SLIDING, att.FULL):
        z = np.zeros((2, 512, 4, 256), np.uint16)
        got = att.prefill_chunk(inp["q"], inp["k"], inp["v"], inp["gate"], z, z, 0, lt)
        _close(got, att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt), 1e-13, f"P=0 lt={lt}")


def _brute_chunk(chunk, ck, cv, P, theta, rot_dim, window):
    """Loop version: for each chunk query the explicit list of visible (position, key,
    value) triples -- cached ones as stored, the chunk's own rotated through complex
    numbers -- then one softmax per head."""
    q, k, v, gate = (_f64(chunk[n][0]) for n in ("q", "k", "v", "gate"))
    ck, cv = _f64(ck[0]), _f64(cv[0])
    n = q.shape[0]
    out = np.zeros((n, 16, 256))
    for t in range(n):
        qp = P + t
        for h in range(16):
            g = h // 4
            qr = np.array(_rotate_complex(list(q[t, h]), float(qp), theta, rot_dim))
            keys, vals = [], []
            for p in range(qp + 1):
                if window is not None and qp - p >= window:
                    continue
                if p < P:
                    s = p if window is None else p % window
                    keys.append(ck[s, g]); vals.append(cv[s, g])
                else:
                    keys.append(np.array(_rotate_complex(list(k[p - P, g]), float(p), theta, rot_dim)))
                    vals.append(v[p - P, g])
            sc = np.array([float(np.dot(qr, kk)) for kk in keys]) / 16.0
            e = np.exp(sc - sc.max())
            out[t, h] = (1.0 / (1.0 + math.exp(-gate[t, h]))) * (e @ np.array(vals)) / e.sum()
    return out


def pin_chunk_brute_force(att):
    """Cached prefix plus chunk against the loop version: full cache and a ring that wraps."""
    for lt, P, n, theta, rd, w in ((att.FULL, 40, 6, 5e6, 64, None), (att.SLIDING, 530, 5, 1e4, 256, 512)):
        _, chunk, ck, cv = _chunk_case(32 + lt, P, n, lt, att)
        got = att.prefill_chunk(chunk["q"], chunk["k"], chunk["v"], chunk["gate"], ck, cv, P, lt)
        _close(got[0], _brute_chunk(chunk, ck, cv, P, theta, rd, w), 1e-11, f"chunk brute lt={lt}")


def pin_chunk_ignores_out_of_reach_slots(att):
    """Cache slots no chunk query can see do not change the result: on a full layer the
    slots from P on, on a sliding layer the slot of position P-512 (one past the window of
    the chunk's first query)."""
    for lt, P, n, junk in ((att.FULL, 50, 4, slice(50, 54)), (att.SLIDING, 600, 4, (600 - 512) % 512)):
        _, chunk, ck, cv = _chunk_case(34 + lt, P, n, lt, att)
        base = att.prefill_chunk(chunk["q"], chunk["k"], chunk["v"], chunk["gate"], ck, cv, P, lt)
        ck2, cv2 = ck.copy(), cv.copy()
        ck2[0, junk] = 0x4120                      # bf16 10.0: would dominate any score
        cv2[0, junk] = 0x4120
        got = att.prefill_chunk(chunk["q"], chunk["k"], chunk["v"], chunk["gate"], ck2, cv2, P, lt)
        _close(got, base, 0.0, f"out-of-reach slots lt={lt}")


def pin_chunked_matches_one_shot(att):
    """Feeding a sequence as prefix (appended to the cache) plus chunk gives the one-shot
    prefill's rows, up to the bf16 rounding of the cached keys."""
    for lt in (att.SLIDING, att.FULL):
        P, n = 530, 70
        inp, chunk, ck, cv = _chunk_case(36 + lt, P, n, lt, att)
        got = att.prefill_chunk(chunk["q"], chunk["k"], chunk["v"], chunk["gate"], ck, cv, P, lt)
        want = att.prefill(inp["q"], inp["k"], inp["v"], inp["gate"], lt, rows=np.arange(P, P + n))
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert rel < 5e-3, f"chunked vs one-shot lt={lt}: rel {rel:.2e}"
        assert np.max(np.abs(got - want)) < 2e-2, f"chunked vs one-shot lt={lt}: max abs"


def pin_varlen_equal_lengths_is_batched(att):
    """Sequences of equal length packed back to back give the batched prefill's rows."""
    rng = np.random.default_rng(61)
    B, S = 3, 40
    x = {n: att.round_to_bf16_bits(rng.standard_normal(sh)) for n, sh in
         (("q", (B, S, 16, 256)), ("k", (B, S, 4, 256)), ("v", (B, S, 4, 256)), ("gate", (B, S, 16)))}
    for lt in (att.SLIDING, att.FULL):
        want = att.prefill(x["q"], x["k"], x["v"], x["gate"], lt).reshape(B * S, 16, 256)
        packed = {n: a.reshape((B * S,) + a.shape[2:]) for n, a in x.items()}
        got = att.prefill_varlen(packed["q"], packed["k"], packed["v"], packed["gate"], [0, S, 2 * S, 3 * S], lt)
        _close(got, want, 0.0, f"varlen equal lengths lt={lt}")


def pin_varlen_isolation(att):
    """A sequence's rows depend on its own tokens only: changing every other sequence (and
    inserting empty ones) leaves them unchanged, and its rows start again at position 0."""
    rng = np.random.default_rng(62)
    lens = [5, 0, 37, 1, 20]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    x = {n: att.round_to_bf16_bits(rng.standard_normal(sh)) for n, sh in
         (("q", (T, 16, 256)), ("k", (T, 4, 256)), ("v", (T, 4, 256)), ("gate", (T, 16)))}
    for lt in (att.SLIDING, att.FULL):
        base = att.prefill_varlen(x["q"], x["k"], x["v"], x["gate"], cu, lt)
        y = {n: a.copy() for n, a in x.items()}
        mine = slice(int(cu[2]), int(cu[3]))
        for n in y:
            other = np.ones(T, bool)
            other[mine] = False
            y[n][other] = att.round_to_bf16_bits(rng.standard_normal(y[n][other].shape))
        got = att.prefill_varlen(y["q"], y["k"], y["v"], y["gate"], cu, lt)
        _close(got[mine], base[mine], 0.0, f"isolation lt={lt}")
        alone = att.prefill(x["q"][mine][None], x["k"][mine][None], x["v"][mine][None], x["gate"][mine][None], lt)[0]
        _close(base[mine], alone, 0.0, f"positions restart lt={lt}")
        # row 0 of every non-empty sequence is sigma(g) v0 of that sequence
        for b in range(len(lens)):
            if lens[b] == 0:
                continue
            g0 = att.bf16_to_f64(x["gate"][cu[b]])
            v0 = att.bf16_to_f64(x["v"][cu[b]])
            want0 = (1 / (1 + np.exp(-g0)))[:, None] * np.repeat(v0, 4, axis=0)
            _close(base[cu[b]], want0, 1e-12, f"first row of sequence {b} lt={lt}")


# --------------------------------------------------------------------------- footprint


def pin_footprint(att, fp):
    gold = json.load(open(os.path.join(GOLDEN, "kv_footprint_pages.json")))
    assert fp.kv_bytes_full_layer_per_token() == gold["kv_per_full_layer_per_token_kb"] * 1024
    per9 = 9 * fp.kv_bytes_full_layer_per_token()
    assert per9 == gold["kv_9_full_layers_per_token_kb"]["f16"] * 1024
    assert round(fp.q8_0_bytes(9 * 2 * 4 * 256) / 1024) == gold["kv_9_full_layers_per_token_kb"]["q8_0"]
    sliding = 27 * fp.kv_bytes_sliding_layer()
    assert sliding == 56623104 and round(sliding / 1e6) == gold["sliding_fixed_mb"]
    assert fp.kv_bytes_model(2 * 10 ** 6) - fp.kv_bytes_model(10 ** 6) == 10 ** 6 * per9
    # the page multiplies in KB: 100 000 tokens x 36 KB = 3.6 million KB, "about 3.6 GB"
    assert round(100000 * (per9 / 1024) / 1e6, 1) == gold["kv_100k_tokens_gb"]
    # The table prints two decimals; its fixed term looks a little above 27 x 512 slots
    # (32K: 1.2646 computed vs 1.27 printed), so rows are matched to one printed digit.
    bad = set(gold["kv_table_inconsistent_rows"]["f16"])
    for ctx, row in gold["kv_table_gb"].items():
        for kind, gb in row.items():
            got = fp.kv_bytes_model(int(ctx), cache_type=kind) / 1e9
            if kind == "f16" and ctx in bad:
                assert abs(got - gb) > 0.05
            else:
                assert abs(got - gb) <= 0.0101, f"KV table {ctx} {kind}: {got:.4f} vs {gb}"


# --------------------------------------------------------------------------- 8-bit cache


def pin_q8_closed_form(q8):
    """Values that are whole multiples of a power-of-two step, with +-127 steps present in
    every block, quantise to exactly those multiples: d = step, codes = the integers."""
    rng = np.random.default_rng(51)
    ints = rng.integers(-127, 128, size=(3, 256))
    ints[:, ::32] = 127
    ints[1, 1::32] = -127
    steps = np.array([2.0 ** -(3 + (blk % 5)) for blk in range(8)])
    x = (ints.reshape(3, 8, 32) * steps[None, :, None]).reshape(3, 256)
    codes, scales = q8.q8_quantize(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    assert codes.shape == (3, 256) and scales.shape == (3, 8)
    assert np.array_equal(codes.astype(np.int64), ints), "codes"
    assert np.array_equal(scales.astype(np.float64), np.broadcast_to(steps, (3, 8))), "scales"
    assert np.array_equal(q8.q8_dequantize(codes, scales), x), "read back"


def pin_q8_zero_and_half_away(q8):
    """An all-zero block stores scale 0 and codes 0; codes round half away from zero
    (with d = 1: 2.5 -> 3, -2.5 -> -3, 0.5 -> 1, where nearest-even would give 2, -2, 0)."""
    codes, scales = q8.q8_quantize(np.zeros((2, 64)))
    assert not codes.any() and not scales.astype(np.float64).any()
    assert not q8.q8_dequantize(codes, scales).any()
    x = np.zeros(32)
    x[:8] = [127.0, 2.5, -2.5, 0.5, -0.5, 3.5, -1.5, 126.5]
    codes, scales = q8.q8_quantize(x)
    assert float(scales[0]) == 1.0
    assert codes[:8].tolist() == [127, 3, -3, 1, -1, 4, -2, 127], codes[:8].tolist()


def pin_q8_error_bound(q8):
    """Any correct q8_0 quantiser: codes within +-127, the largest magnitude of a nonzero
    block at +-127, and every value read back within half a step (plus the fp16 rounding
    of the step, up to 127 codes' worth) of the input; negating the input negates the codes."""
    rng = np.random.default_rng(52)
    x = np.concatenate([rng.standard_normal((40, 256)), rng.standard_cauchy((10, 256)),
                        1e-3 * rng.standard_normal((10, 256))]).astype(np.float32)
    codes, scales = q8.q8_quantize(x)
    assert np.abs(codes.astype(np.int64)).max() <= 127
    xb = np.abs(x.astype(np.float64)).reshape(60, 8, 32)
    cb = codes.astype(np.int64).reshape(60, 8, 32)
    top = np.take_along_axis(np.abs(cb), np.argmax(xb, axis=-1)[..., None], -1)[..., 0]
    assert (top == 127).all()
    d = xb.max(-1) / 127.0
    d16 = scales.astype(np.float64)
    err = np.abs(q8.q8_dequantize(codes, scales).reshape(60, 8, 32) - x.astype(np.float64).reshape(60, 8, 32))
    bound = 0.5 * d * (1 + 1e-6) + 127 * np.abs(d16 - d) + 1e-12
    assert (err <= bound[..., None]).all(), float((err - bound[..., None]).max())
    nc, ns = q8.q8_quantize(-x)
    assert np.array_equal(nc, -codes) and np.array_equal(ns, scales)


def pin_q8_row_bytes(q8, fp):
    """A K or V row of 256 values takes 256 code bytes and 8 fp16 scales: the q8_0 size
    the KV footprint pin checks against the pages' table."""
    codes, scales = q8.q8_quantize(np.ones((1, 256)))
    assert codes.nbytes + scales.nbytes == fp.q8_0_bytes(256) == 272


def _q8_cache(rng, B, cap):
    kc = rng.integers(-127, 128, size=(B, cap, 4, 256)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(B, cap, 4, 256)).astype(np.int8)
    ks = (rng.uniform(0.005, 0.03, size=(B, cap, 4, 8))).astype(np.float16)
    vs = (rng.uniform(0.005, 0.03, size=(B, cap, 4, 8))).astype(np.float16)
    return kc, ks, vc, vs


def pin_kv_append_q8(att, q8):
    """The 8-bit append writes what the bf16 append writes, read back within the q8_0
    error bound, into the same slots (ring wrap included); untouched slots keep their
    contents."""
    rng = np.random.default_rng(53)
    for lt, cap, pos, n in ((att.FULL, 64, [3, 20], 9), (att.SLIDING, 512, [505, 1000], 600)):
        B = 2
        k = rng.standard_normal((B, n, 4, 256)).astype(np.float32)
        v = rng.standard_normal((B, n, 4, 256)).astype(np.float32)
        kb, vb = att.round_to_bf16_bits(k), att.round_to_bf16_bits(v)
        kc, ks, vc, vs = _q8_cache(rng, B, cap)
        got = q8.kv_append_q8(kc, ks, vc, vs, kb, vb, np.array(pos), lt)
        z = np.zeros((B, cap, 4, 256), np.uint16)
        rk, rv = att.kv_append(z, z.copy(), kb, vb, np.array(pos), lt)
        for b in range(B):
            slots = sorted({att.cache_slot(p, lt) for p in range(pos[b], pos[b] + n)})
            rest = np.setdiff1d(np.arange(cap), slots)
            for name, codes, scales, old_c, old_s, ref in (("K", got[0], got[1], kc, ks, rk),
                                                           ("V", got[2], got[3], vc, vs, rv)):
                assert np.array_equal(codes[b, rest], old_c[b, rest]), f"{name} lt={lt}: untouched slots"
                assert np.array_equal(scales[b, rest], old_s[b, rest]), f"{name} lt={lt}: untouched scales"
                back = q8.q8_dequantize(codes[b, slots], scales[b, slots])
                want = att.bf16_to_f64(ref[b, slots])
                step = scales[b, slots].astype(np.float64).repeat(32, axis=-1)
                # bf16 rounding of the reference (2^-9 relative) plus half a q8 step
                assert (np.abs(back - want) <= 0.51 * step + 2.0 ** -8 * np.abs(want) + 1e-6).all(), \
                    f"{name} lt={lt}: read-back beyond the q8_0 bound"
        assert np.array_equal(got[2][0, att.cache_slot(pos[0] + n - 1, lt)], q8.q8_quantize(
            att.bf16_to_f64(vb[0, n - 1]).astype(np.float32))[0]), "last value's codes"


def pin_decode_q8(att, q8):
    """Over a cache whose read-back values bf16 holds exactly (power-of-two steps, a
    different one per block), the 8-bit decode equals the bf16 decode of those values."""
    rng = np.random.default_rng(54)
    for lt, cap, lens in ((att.FULL, 96, [1, 70, 96]), (att.SLIDING, 512, [3, 600, 1500])):
        B = len(lens)
        kc, _, vc, _ = _q8_cache(rng, B, cap)
        ks = np.broadcast_to(np.array([2.0 ** -(4 + (j % 4)) for j in range(8)]), (B, cap, 4, 8)).astype(np.float16)
        vs = np.broadcast_to(np.array([2.0 ** -(3 + (j % 3)) for j in range(8)]), (B, cap, 4, 8)).astype(np.float16)
        q = att.round_to_bf16_bits(rng.standard_normal((B, 16, 256)))
        g = att.round_to_bf16_bits(rng.standard_normal((B, 16)))
        got = q8.decode_q8(q, g, kc, ks, vc, vs, np.array(lens), lt)
        kbits = att.round_to_bf16_bits(q8.q8_dequantize(kc, ks))
        vbits = att.round_to_bf16_bits(q8.q8_dequantize(vc, vs))
        assert np.array_equal(att.bf16_to_f64(kbits), q8.q8_dequantize(kc, ks)), "values exact in bf16"
        want = att.decode(q, g, kbits, vbits, np.array(lens), lt)
        assert np.allclose(got, want, rtol=0, atol=1e-12), f"lt={lt}: {np.abs(got - want).max()}"


Q8_PINS = [pin_q8_closed_form, pin_q8_zero_and_half_away, pin_q8_error_bound]
Q8_ATT_PINS = [pin_kv_append_q8, pin_decode_q8]


# --------------------------------------------------------------------------- FP8 projections


def pin_e4m3fn_codec(pj):
    """OCP E4M3FN: closed-form codes, every finite code round-trips, ties go to the even
    mantissa, the spacing is 2^(e-3), 448 is the largest finite value."""
    cases = {1.0: 0x38, -1.0: 0xB8, 0.5: 0x30, 2.0: 0x40, -2.0: 0xC0, 448.0: 0x7E, -448.0: 0xFE,
             2.0 ** -9: 0x01, 2.0 ** -6: 0x08, 7 * 2.0 ** -9: 0x07, 240.0: 0x77, 0.0: 0x00, 1.75: 0x3E,
             1.0625: 0x38, 1.1875: 0x3A, 3 * 2.0 ** -10: 0x02, 2.0 ** -10: 0x00, 460.0: 0x7E, 17.0: 0x58, 18.0: 0x59}
    got = pj.e4m3fn_encode(list(cases))
    assert got.tolist() == list(cases.values()), [hex(int(x)) for x in got]
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(pj.e4m3fn_encode(pj.e4m3fn_decode(finite)), finite)
    pos = pj.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all() and pos[-1] == 448.0
    for c in range(0x08, 0x7E):                            # normal codes: spacing 2^(e-3)
        e = (c >> 3) - 7
        assert pos[c + 1] - pos[c] == 2.0 ** (e - 3) or (c & 7) == 7
    assert np.isnan(pj.e4m3fn_decode([0x7F, 0xFF])).all()
    assert pj.e4m3fn_encode([464.0])[0] == 0x7E          # the tie rounds to the even 448
    for bad in (464.5, 1e6):
        try:
            pj.e4m3fn_encode([bad])
        except ValueError:
            continue
        raise AssertionError(f"{bad} should not encode")


def _bf16(att, x):
    return att.round_to_bf16_bits(np.asarray(x, dtype=np.float64))


def pin_token_quantizer(att, pj):
    """Per-token scales: max |x| codes to +-448, values read back within half a step
    (2^-4 relative for normals, s 2^-10 absolute below), sign symmetric; a zero row has
    scale 0 and codes 0."""
    rng = np.random.default_rng(71)
    x = np.concatenate([rng.standard_normal((6, 2560)), 1e-3 * rng.standard_cauchy((2, 2560)),
                        np.zeros((1, 2560))])
    xb = _bf16(att, x)
    codes, s = pj.quantize_tokens(xb)
    xv = att.bf16_to_f64(xb)
    assert codes.shape == (9, 2560) and s.dtype == np.float32 and s[-1] == 0 and not codes[-1].any()
    top = np.abs(pj.e4m3fn_decode(codes[np.arange(8), np.argmax(np.abs(xv[:8]), axis=1)]))
    assert (top == 448.0).all()
    back = pj.e4m3fn_decode(codes[:8]) * s[:8, None]
    err = np.abs(back - xv[:8])
    assert (err <= np.abs(xv[:8]) / 16 + s[:8, None] * 2.0 ** -10 + 1e-12).all()
    nc, ns = pj.quantize_tokens(_bf16(att, -x))
    assert np.array_equal(ns, s) and np.array_equal(nc[:8] ^ 0x80, codes[:8]) or \
        np.array_equal(pj.e4m3fn_decode(nc), -pj.e4m3fn_decode(codes))


def pin_qkv_proj_identity(att, pj):
    """Identity-like weights (channel n reads input n mod 2560 with code 1.0, scale 1)
    return the quantised activations, in the q/k/v split and head layout; one-hot gate
    rows return the chosen inputs exactly; scales act linearly."""
    rng = np.random.default_rng(72)
    T = 5
    xb = _bf16(att, rng.standard_normal((T, 2560)))
    w = np.zeros((6144, 2560), np.uint8)
    w[np.arange(6144), np.arange(6144) % 2560] = 0x38
    ws = np.ones(6144, np.float32)
    pick = rng.choice(2560, 16, replace=False)
    wg = np.zeros((16, 2560), np.uint16)
    wg[np.arange(16), pick] = 0x3F80                     # bf16 1.0
    q, k, v, g = pj.qkv_proj(xb, w, ws, wg)
    codes, s = pj.quantize_tokens(xb)
    xq = pj.e4m3fn_decode(codes) * s[:, None]
    full = xq[:, np.arange(6144) % 2560]
    _close(q, full[:, :4096].reshape(T, 16, 256), 1e-12, "q")
    _close(q[:, 3, 7], xq[:, 3 * 256 + 7], 1e-12, "q head 3 dim 7")
    _close(k, full[:, 4096:5120].reshape(T, 4, 256), 1e-12, "k")
    _close(v[:, 2, 5], xq[:, (5120 + 2 * 256 + 5) % 2560], 1e-12, "v head 2 dim 5")
    _close(g, att.bf16_to_f64(xb)[:, pick], 0.0, "gate one-hot")
    q2, _, v2, _ = pj.qkv_proj(xb, w, 2 * ws, wg)
    _close(q2, 2 * q, 1e-12, "linear in the channel scale")


PROJ_PINS = [pin_e4m3fn_codec]
PROJ_ATT_PINS = [pin_token_quantizer, pin_qkv_proj_identity]


ALL_PINS = [
    pin_brute_force_tiny, pin_brute_force_real_heads, pin_window_covering_sequence_is_causal,
    pin_window_one_closed_form, pin_row_zero_closed_form, pin_constant_values,
    pin_zero_query_uniform_mean, pin_gate_limits, pin_gqa_equals_repeated_kv, pin_torch_sdpa,
    pin_rope_properties, pin_rope_frequencies, pin_layer_schedule, pin_bf16_rounding,
    pin_kv_append, pin_decode_brute, pin_decode_matches_prefill_row,
    pin_chunk_start_zero_is_prefill, pin_chunk_brute_force, pin_chunk_ignores_out_of_reach_slots,
    pin_chunked_matches_one_shot, pin_varlen_equal_lengths_is_batched, pin_varlen_isolation,
]
