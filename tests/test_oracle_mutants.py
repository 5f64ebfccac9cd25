"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check
that at least one pin in ``oracle_pins`` fails for it.  This shows the pins are strong
enough that a dropped term, a wrong sign, an off-by-one window or a wrong head map in
the oracle would not go unnoticed."""
import os
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "window_boundary_off_by_one": ("vis &= (q - k) < int(window)", "vis &= (q - k) <= int(window)"),
    "causal_excludes_self": ("vis = k <= q", "vis = k < q"),
    "scale_one_over_d": ("return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    "gqa_modulo_map": ("return h // (n_q_heads // n_kv_heads)", "return h % n_kv_heads"),
    "rope_sign_flip": ("y[..., :half] = x1 * c - x2 * s", "y[..., :half] = x1 * c + x2 * s"),
    "rope_freq_missing_factor_2": ("-2.0 * m / float(rot_dim)", "-1.0 * m / float(rot_dim)"),
    "rope_pairs_adjacent": ("x2 = x[..., half:rot_dim]", "x2 = x[..., half:rot_dim][..., ::-1]"),
    "gate_dropped": ("return o * g[:, None]", "return o"),
    "gate_sign": ("np.exp(-np.asarray(gate_logit", "np.exp(np.asarray(gate_logit"),
    "ring_modulo": ("position % window", "position % (window - 1)"),
    "bf16_truncates": ("np.rint(np.ldexp(x, -qexp))", "np.trunc(np.ldexp(x, -qexp))"),
    "schedule_first_of_group_full": ("layer % 4 == 3", "layer % 4 == 0"),
    "full_layer_rotates_all_dims": ("return 5000000.0, HEAD_DIM // 4, None", "return 5000000.0, HEAD_DIM, None"),
    "sliding_theta_wrong": ("return 10000.0, HEAD_DIM, WINDOW", "return 5000000.0, HEAD_DIM, WINDOW"),
    "decode_query_position": ("qp = L - 1", "qp = L"),
    "decode_window_short": ("lo = 0 if w is None else max(0, L - w)", "lo = 0 if w is None else max(0, L - w + 1)"),
    "value_head_fixed": ("vb[:nk, g]", "vb[:nk, 0]"),
    "append_position_shift": ("p = int(pos[b]) + np.arange(n_new)", "p = int(pos[b]) + 1 + np.arange(n_new)"),
    "chunk_query_positions": ("qpos = P + rr", "qpos = rr"),
    "chunk_key_positions": ("new_pos = P + np.arange(n)", "new_pos = np.arange(n) + 1"),
    "chunk_history_from_keys": ("bf16_to_f64(np.asarray(cache_v)[b, h_slot])", "bf16_to_f64(np.asarray(cache_k)[b, h_slot])"),
    "chunk_history_one_short": ("h_pos = np.arange(h_lo, P)", "h_pos = np.arange(h_lo + 1, P)"),
    "varlen_sequence_starts_early": ("one = lambda x: np.asarray(x)[lo:hi][None]",
                                     "one = lambda x: np.asarray(x)[max(lo - 1, 0):hi - 1 if lo > 0 else hi][None]"),
    "varlen_skips_single_token": ("if hi <= lo or len(sel) == 0:", "if hi <= lo + 1 or len(sel) == 0:"),
}


def _mutant_module(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site must occur exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    att = _mutant_module(*MUTANTS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(att)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin fails for the planted mistake {name}"


Q8_SRC = os.path.join(os.path.dirname(SRC), "kvq8.py")
Q8_MUTANTS = {
    "q8_divisor_128": ("amax / np.float32(127.0)", "amax / np.float32(128.0)"),
    "q8_round_nearest_even": ("np.floor(np.abs(y64) + 0.5)", "np.round(np.abs(y64))"),
    "q8_truncate": ("np.floor(np.abs(y64) + 0.5)", "np.floor(np.abs(y64))"),
    "q8_scale_of_reversed_block": ("np.asarray(scales, dtype=np.float64)[..., None]",
                                   "np.asarray(scales, dtype=np.float64)[..., ::-1, None]"),
    "q8_key_not_rotated": ("kr = rope(bf16_to_f64(k[b]), p, th, rd).astype(np.float32)",
                           "kr = bf16_to_f64(k[b]).astype(np.float32)"),
    "q8_value_from_key": ("qv, dv = q8_quantize(bf16_to_f64(v[b]).astype(np.float32))",
                          "qv, dv = q8_quantize(bf16_to_f64(k[b]).astype(np.float32))"),
    "q8_decode_values_from_keys": ("lambda b, slots, g: q8_dequantize(vc[b, slots, g], vs[b, slots, g])",
                                   "lambda b, slots, g: q8_dequantize(kc[b, slots, g], ks[b, slots, g])"),
    "q8_append_slot_shift": ("s = cache_slot(int(p[t]), layer_type)", "s = cache_slot(int(p[t]) + 1, layer_type)"),
}


@pytest.mark.parametrize("name", sorted(Q8_MUTANTS))
def test_planted_q8_mistake_is_caught(name):
    import oracle.attention as att
    old, new = Q8_MUTANTS[name]
    src = open(Q8_SRC).read()
    assert src.count(old) == 1, f"mutation site must occur exactly once: {old!r}"
    mod = types.ModuleType("oracle_q8_mutant")
    exec(compile(src.replace(old, new), "oracle_q8_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in P.Q8_PINS + P.Q8_ATT_PINS:
        try:
            pin(mod) if pin in P.Q8_PINS else pin(att, mod)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin fails for the planted mistake {name}"


PROJ_SRC = os.path.join(os.path.dirname(SRC), "proj.py")
PROJ_MUTANTS = {
    "e4m3_bias_8": ("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_round_half_up": ("q = np.rint(a / step)", "q = np.floor(a / step + 0.5)"),
    "token_scale_range_240": ("amax / np.float32(E4M3_MAX)", "amax / np.float32(240.0)"),
    "kv_split_swapped": ("y[:, 4096:5120].reshape(T, 4, 256),\n            y[:, 5120:].reshape(T, 4, 256)",
                         "y[:, 5120:].reshape(T, 4, 256),\n            y[:, 4096:5120].reshape(T, 4, 256)"),
    "gate_from_quantised_x": ("gate = bf16_to_f64(x_bits) @", "gate = (e4m3fn_decode(xc) * xs[:, None]) @"),
    "channel_scale_dropped": (" * np.asarray(w_scales, dtype=np.float64)[None, :]", ""),
}


@pytest.mark.parametrize("name", sorted(PROJ_MUTANTS))
def test_planted_proj_mistake_is_caught(name):
    import oracle.attention as att
    old, new = PROJ_MUTANTS[name]
    src = open(PROJ_SRC).read()
    assert src.count(old) == 1, f"mutation site must occur exactly once: {old!r}"
    mod = types.ModuleType("oracle_proj_mutant")
    exec(compile(src.replace(old, new), "oracle_proj_mutant", "exec"), mod.__dict__)
    caught = []
    for pin in P.PROJ_PINS + P.PROJ_ATT_PINS:
        try:
            pin(mod) if pin in P.PROJ_PINS else pin(att, mod)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin fails for the planted mistake {name}"
