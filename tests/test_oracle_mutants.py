"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is the oracle's own source with one plausible error written into
it (a dropped term, a wrong sign or index, a transposed operand, ...), loaded
as a separate module on the CPU.  The real oracle is never modified.
"""

import os
import types

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention.py")

MUTANTS = {
    "dropped_scale": ("scores = (qh @ kh.T) * scale", "scores = (qh @ kh.T)"),
    "transposed_scores": ("scores = (qh @ kh.T) * scale", "scores = (kh @ qh.T) * scale"),
    "causal_wrong_direction": ("ok = ok & (j <= i)", "ok = ok & (j >= i)"),
    "causal_strict": ("ok = ok & (j <= i)", "ok = ok & (j < i)"),
    "padding_off_by_one": ("    ok = j < key_len\n    if causal:", "    ok = j <= key_len\n    if causal:"),
    "rows_padding_off_by_one": ("        ok = j < key_len\n", "        ok = j <= key_len\n"),
    "gqa_interleaved": ("return (h * n_kv_heads) // n_q_heads", "return h % n_kv_heads"),
    "no_max_subtraction": ("e = np.exp(scores - m[:, None])", "e = np.exp(scores)"),
    "no_normalisation": ("p = e / safe[:, None]", "p = e"),
    "lse_missing_max": ("lse = np.where(has_key, m + np.log(safe), -np.inf)",
                        "lse = np.where(has_key, np.log(safe), -np.inf)"),
    "lse_log2": ("lse = np.where(has_key, m + np.log(safe), -np.inf)",
                 "lse = np.where(has_key, m + np.log2(safe), -np.inf)"),
    "transposed_pv": ("out = p @ vh", "out = p.T @ vh"),
    "default_scale_1_over_d": ("return 1.0 / math.sqrt(d)", "return 1.0 / d"),
    "rows_dropped_scale": ("sc = (kh @ qi) * scale", "sc = (kh @ qi)"),
    "rows_causal_strict": ("ok &= j <= i", "ok &= j < i"),
    "rows_no_max": ("e = np.exp(sc - m)", "e = np.exp(sc)"),
    "rows_masked_not_zeroed": ("            out[n] = 0.0\n            lse[n] = -np.inf\n            continue",
                               "            lse[n] = -np.inf\n            out[n] = 1.0\n            continue"),
    "rows_lse_missing_max": ("lse[n] = m + np.log(den)", "lse[n] = np.log(den)"),
    "rows_gqa_wrong_head": ("kh = np.asarray(k[b, :, g, :], dtype=np.float64)",
                            "kh = np.asarray(k[b, :, h % k.shape[2], :], dtype=np.float64)"),
    "pad_key_len_ignores_batch": ("return int(min(max(int(pad_lens[b]), 0), s))",
                                  "return int(min(max(int(pad_lens[0]), 0), s))"),
}


def _load_mutant(find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(find, repl), "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(*MUTANTS[name])
    caught = []
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, FloatingPointError, ValueError, IndexError) as e:
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# rotary embedding (oracle/rope.py) against tests/oracle_rope_pins.py
# --------------------------------------------------------------------------
import oracle_rope_pins  # noqa: E402

ROPE_SRC = os.path.join(os.path.dirname(oracle.__file__), "rope.py")

ROPE_MUTANTS = {
    "sign_even": ("out[..., 0::2] = even * c - odd * sn", "out[..., 0::2] = even * c + odd * sn"),
    "sign_odd": ("out[..., 1::2] = odd * c + even * sn", "out[..., 1::2] = odd * c - even * sn"),
    "cos_sin_swapped": ("c = np.cos(ang)[:, :, None, :]", "c = np.sin(ang)[:, :, None, :]"),
    "exponent_doubled": ("return np.power(float(base), -2.0 * i / d)", "return np.power(float(base), -4.0 * i / d)"),
    "exponent_not_halved": ("return np.power(float(base), -2.0 * i / d)", "return np.power(float(base), -1.0 * i / d)"),
    "base_ignored": ("return np.power(float(base), -2.0 * i / d)", "return np.power(10000.0, -2.0 * i / d)"),
    "half_split_pairs": ("    even = x[..., 0::2]\n    odd = x[..., 1::2]",
                         "    even = x[..., : d // 2]\n    odd = x[..., d // 2:]"),
    "positions_ignored": ("    if positions is None:\n        return",
                          "    if True:\n        return"),
    "positions_batch0": ("    return pos\n", "    return np.broadcast_to(pos[0], (b, s))\n"),
    "positions_from_one": ("return np.broadcast_to(np.arange(s, dtype=np.int64), (b, s))",
                           "return np.broadcast_to(np.arange(1, s + 1, dtype=np.int64), (b, s))"),
    "odd_not_rotated": ("out[..., 1::2] = odd * c + even * sn", "out[..., 1::2] = odd"),
}


def _load_rope_mutant(find, repl):
    src = open(ROPE_SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    mod = types.ModuleType("oracle_rope_mutant")
    exec(compile(src.replace(find, repl), "oracle_rope_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_mutant_is_caught(name):
    mod = _load_rope_mutant(*ROPE_MUTANTS[name])
    caught = []
    for pin in oracle_rope_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# decode attention (oracle/decode.py) against tests/oracle_decode_pins.py
# --------------------------------------------------------------------------
import oracle_decode_pins  # noqa: E402

DECODE_SRC = os.path.join(os.path.dirname(oracle.__file__), "decode.py")

DECODE_MUTANTS = {
    "top_left_alignment": ("return j <= key_len - sq + i", "return j <= i"),
    "alignment_off_by_one": ("return j <= key_len - sq + i", "return j < key_len - sq + i"),
    "alignment_past_end": ("return j <= key_len - sq + i", "return j <= key_len - sq + i + 1"),
    "cache_lens_ignored": ("L = sk if cache_lens is None else", "L = sk if True else"),
    "cache_lens_batch0": ("int(min(max(int(cache_lens[b]), 0), sk))", "int(min(max(int(cache_lens[0]), 0), sk))"),
    "non_causal_sees_nothing_past_query": ("        return np.ones(key_len, dtype=bool)",
                                           "        return np.arange(key_len) <= i"),
    "lse_missing_max": ("lse[b, h, i] = m + np.log(den)", "lse[b, h, i] = np.log(den)"),
    "dropped_scale": ("s = (kh[ok] @ q[b, i, h, :]) * scale", "s = (kh[ok] @ q[b, i, h, :])"),
    "unnormalised": ("out[b, i, h, :] = (e / den) @ vh[ok]", "out[b, i, h, :] = e @ vh[ok]"),
    "gqa_wrong_head": ("g = kv_head_for(h, hq, hkv)", "g = h % hkv"),
}


def _load_decode_mutant(find, repl):
    src = open(DECODE_SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    src = src.replace(find, repl).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_decode_mutant")
    exec(compile(src, "oracle_decode_mutant.py", "exec"), mod.__dict__)
    # the pins also use the (pinned) prefill oracle through the same module
    mod.attention = oracle.attention
    return mod


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    mod = _load_decode_mutant(*DECODE_MUTANTS[name])
    caught = []
    for pin in oracle_decode_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# packed variable-length attention (oracle/varlen.py) against
# tests/oracle_varlen_pins.py
# --------------------------------------------------------------------------
import oracle_varlen_pins  # noqa: E402

VARLEN_SRC = os.path.join(os.path.dirname(oracle.__file__), "varlen.py")

VARLEN_MUTANTS = {
    "end_off_by_one": ("s0, s1 = int(cu[b]), int(cu[b + 1])", "s0, s1 = int(cu[b]), int(cu[b + 1]) + 1"),
    "start_off_by_one": ("s0, s1 = int(cu[b]), int(cu[b + 1])", "s0, s1 = max(int(cu[b]) - 1, 0), int(cu[b + 1])"),
    "causal_strict": ("visible = (j_loc <= i_loc) if causal", "visible = (j_loc < i_loc) if causal"),
    "causal_wrong_direction": ("visible = (j_loc <= i_loc) if causal", "visible = (j_loc >= i_loc) if causal"),
    "causal_ignored": ("visible = (j_loc <= i_loc) if causal", "visible = (j_loc <= i_loc) if False"),
    "gqa_interleaved": ("g = (h * hkv) // hq", "g = h % hkv"),
    "dropped_scale": ("scores = (q[s0:s1, h, :] @ k[s0:s1, g, :].T) * scale",
                      "scores = (q[s0:s1, h, :] @ k[s0:s1, g, :].T)"),
    "transposed_scores": ("scores = (q[s0:s1, h, :] @ k[s0:s1, g, :].T) * scale",
                          "scores = (k[s0:s1, g, :] @ q[s0:s1, h, :].T) * scale"),
    "unnormalised": ("out[s0:s1, h, :] = (e / den[:, None]) @ v[s0:s1, g, :]",
                     "out[s0:s1, h, :] = e @ v[s0:s1, g, :]"),
    "v_from_query_head": ("out[s0:s1, h, :] = (e / den[:, None]) @ v[s0:s1, g, :]",
                          "out[s0:s1, h, :] = (e / den[:, None]) @ v[s0:s1, h % hkv, :]"),
    "lse_missing_max": ("lse[h, s0:s1] = m + np.log(den)", "lse[h, s0:s1] = np.log(den)"),
    "default_scale_1_over_d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "offsets_unchecked": ("    if np.any(np.diff(cu) < 0) or cu[0] < 0 or cu[-1] > total:",
                          "    if False:"),
}


def _load_varlen_mutant(find, repl):
    src = open(VARLEN_SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    mod = types.ModuleType("oracle_varlen_mutant")
    exec(compile(src.replace(find, repl), "oracle_varlen_mutant.py", "exec"), mod.__dict__)
    # the pins also use the (pinned) prefill oracle through the same module
    mod.attention = oracle.attention
    mod.MASK_KEY_PADDING = oracle.MASK_KEY_PADDING
    return mod


@pytest.mark.parametrize("name", sorted(VARLEN_MUTANTS))
def test_varlen_mutant_is_caught(name):
    mod = _load_varlen_mutant(*VARLEN_MUTANTS[name])
    caught = []
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin in oracle_varlen_pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# additive mask tensor (oracle/masked.py) against tests/oracle_masked_pins.py
# --------------------------------------------------------------------------
import oracle_masked_pins  # noqa: E402

MASKED_SRC = os.path.join(os.path.dirname(oracle.__file__), "masked.py")

MASKED_MUTANTS = {
    "mask_before_scale": ("scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale + mask_slice(mask, b, h)",
                          "scores = (q[b, :, h, :] @ k[b, :, g, :].T + mask_slice(mask, b, h)) * scale"),
    "mask_subtracted": ("scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale + mask_slice(mask, b, h)",
                        "scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale - mask_slice(mask, b, h)"),
    "mask_ignored": ("scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale + mask_slice(mask, b, h)",
                     "scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale"),
    "mask_transposed": ("return mask[b if bm > 1 else 0, h if hm > 1 else 0]",
                        "return mask[b if bm > 1 else 0, h if hm > 1 else 0].T"),
    "mask_batch_broadcast_wrong": ("return mask[b if bm > 1 else 0, h if hm > 1 else 0]",
                                   "return mask[0, h if hm > 1 else 0]"),
    "mask_head_from_kv": ("return mask[b if bm > 1 else 0, h if hm > 1 else 0]",
                          "return mask[b if bm > 1 else 0, (h // 2) if hm > 1 else 0]"),
    "causal_ignored": ("            if causal:\n                scores = np.where(above, -np.inf, scores)",
                       "            if False:\n                scores = np.where(above, -np.inf, scores)"),
    "causal_strict": ("above = np.triu(np.ones((s, s), dtype=bool), k=1)",
                      "above = np.triu(np.ones((s, s), dtype=bool), k=0)"),
    "masked_rows_unguarded": ("has_key = np.isfinite(m)", "has_key = np.ones_like(m, dtype=bool)"),
    "lse_missing_max": ("lse[b, h, :] = np.where(has_key, m_safe + np.log(safe), -np.inf)",
                        "lse[b, h, :] = np.where(has_key, np.log(safe), -np.inf)"),
    "gqa_interleaved": ("g = (h * hkv) // hq", "g = h % hkv"),
    "default_scale_1_over_d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "bool_inverted": ("return np.where(mask.astype(bool), 0.0, -np.inf)",
                      "return np.where(mask.astype(bool), -np.inf, 0.0)"),
}


def _load_masked_mutant(find, repl):
    src = open(MASKED_SRC).read()
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    mod = types.ModuleType("oracle_masked_mutant")
    exec(compile(src.replace(find, repl), "oracle_masked_mutant.py", "exec"), mod.__dict__)
    # the pins also use the (pinned) prefill oracle through the same module
    mod.attention = oracle.attention
    mod.MASK_KEY_PADDING = oracle.MASK_KEY_PADDING
    return mod


@pytest.mark.parametrize("name", sorted(MASKED_MUTANTS))
def test_masked_mutant_is_caught(name):
    mod = _load_masked_mutant(*MASKED_MUTANTS[name])
    caught = []
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin in oracle_masked_pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
