"""The oracle's pins must catch plausible mistakes: each case plants one slip
in a copy of the oracle's source (on the CPU, never in the product) and
checks that at least one pin fails against the mutated copy."""
import inspect
import os
import types

import pytest

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "bifocal_oracle.py")

MUTATIONS = {
    "window_strict": ("S = np.where(dist <= w0, s_local, s_remote) * scale",
                      "S = np.where(dist < w0, s_local, s_remote) * scale"),
    "keys_not_remapped": ("kr_all = rope(xk, remap(kpos, G, continuous), theta)",
                          "kr_all = rope(xk, kpos, theta)"),
    "query_not_remapped": ("qr_all = rope(xq[rows], remap(rows, G, continuous), theta)",
                           "qr_all = rope(xq[rows], rows, theta)"),
    "gqa_modulo": ("        g = h // r\n        for c0", "        g = h % Hkv\n        for c0"),
    "rotation_sign": ("[a * c - b * s, a * s + b * c]", "[a * c + b * s, -a * s + b * c]"),
    "group_floor": ("return max(1, -(-L // w_pre))", "return max(1, L // w_pre)"),
    "group_plus_one": ("return max(1, -(-L // w_pre))", "return max(1, L // w_pre + 1)"),
    "causal_strict": ("S = np.where(dist >= 0, S, -np.inf)", "S = np.where(dist > 0, S, -np.inf)"),
    "scale_1_over_d": ("scale = 1.0 / math.sqrt(d)\n    rows =", "scale = 1.0 / d\n    rows ="),
    "freq_ladder": ("return np.power(np.float64(theta), -2.0 * i / d)",
                    "return np.power(np.float64(theta), -1.0 * i / d)"),
    "pairs_interleaved": ("    a = x[..., :half]\n    b = x[..., half:]",
                          "    a = x[..., 0::2]\n    b = x[..., 1::2]"),
    "ie_sign": ("den = WA + WB - WC", "den = WA + WB + WC"),
    "decode_L": ("    L = pos + 1\n    G = group_size(L, w_pre)",
                 "    L = pos + 1\n    G = group_size(pos, w_pre) if pos else 1"),
    "tile_diag_flag": ("    if (~causal).any():\n        cls += 4", "    if (~causal).all():\n        cls += 4"),
    "lse_log2": ("lse = (m + np.log(l))[:, 0]", "lse = (m + np.log2(l))[:, 0]"),
    "continuous_floored": ("return np.asarray(p, dtype=np.int64).astype(np.float64) / float(G)",
                           "return (np.asarray(p, dtype=np.int64) // int(G)).astype(np.float64)"),
    "continuous_times_g": ("return np.asarray(p, dtype=np.int64).astype(np.float64) / float(G)",
                           "return np.asarray(p, dtype=np.int64).astype(np.float64) * float(G)"),
    "continuous_decode_query_floor": (
        "k_rem_pos, q_rem_pos = keys / float(G), pos / float(G)",
        "k_rem_pos, q_rem_pos = keys / float(G), pos // G"),
    "continuous_ie_floor": ("p_rot = pos / float(G) if continuous else pos // G",
                            "p_rot = pos // G"),
    "batch_start_ignored": ("k_rows[s0:s0 + p + 1], v_rows[s0:s0 + p + 1]",
                            "k_rows[:p + 1], v_rows[:p + 1]"),
    "batch_bound_inclusive": ("s0 + p >= rows or", "s0 + p > rows or"),
    "scores_window_strict": ("return np.where(dist <= w0, s_local, s_remote)",
                             "return np.where(dist < w0, s_local, s_remote)"),
    "scores_keys_not_remapped": ("kr = rope(xk, remap(k_pos, G, continuous), theta)",
                                 "kr = rope(xk, k_pos, theta)"),
    "scores_query_not_remapped": ("qr = rope(xq_rows, remap(q_pos, G, continuous), theta)",
                                  "qr = rope(xq_rows, q_pos, theta)"),
    "scores_routes_swapped": ("return np.where(dist <= w0, s_local, s_remote)",
                              "return np.where(dist <= w0, s_remote, s_local)"),
}


def _load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: anchor not unique/present"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """(name, zero-arg callable) for every pin, with representative params."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn))
            continue
        combos = [{}]
        for m in params:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) \
                else list(m.args[0])
            new = []
            for c in combos:
                for val in m.args[1]:
                    vals = val if len(argnames) > 1 else (val,)
                    new.append({**c, **dict(zip(argnames, vals))})
            combos = new
        for kw in combos:
            calls.append((f"{name}{kw}", (lambda f, k: (lambda: f(**k)))(fn, kw)))
    # cheap pins first; the 2^17-position composition sweep last
    calls.sort(key=lambda c: "composition" in c[0])
    return calls


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    mod = _load_mutant(name, *MUTATIONS[name])
    for attr in ("bifocal_attention", "bifocal_scores", "bifocal_varlen", "decode_batch",
                 "decode_row",
                 "group_size", "ie_merge", "ie_pass", "remap", "rope", "rope_frequencies",
                 "tile_class", "tile_class_map"):
        monkeypatch.setattr(pins, attr, getattr(mod, attr))
    failed = []
    for pin_name, call in _pin_calls():
        if "bruteforce_small" in pin_name or "vectorized_large" in pin_name:
            if not name.startswith("group"):
                continue
        try:
            call()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin_name)
            break
    assert failed, f"no pin caught mutation {name}"
