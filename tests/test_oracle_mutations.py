"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutation edits one expression of a copy of the oracle's source, loads the
copy as a fresh module and runs every pin on it; at least one pin must fail.
One edit that is *not* a mistake (reversing the roll direction, which the method
is invariant to) must pass every pin.
"""

import importlib.util
import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "s2attn_oracle.py")

# (name, original text, replacement, occurrence index to replace)
MUTATIONS = [
    ("shift-first-heads", "return G // 2 if h >= H - shift_heads else 0",
     "return G // 2 if h < shift_heads else 0", 0),
    ("shift-by-quarter", "return G // 2 if h >= H - shift_heads else 0",
     "return G // 4 if h >= H - shift_heads else 0", 0),
    ("strict-causal-fwd", "allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]",
     "allowed = np.arange(r1)[None, :] < np.arange(r0, r1)[:, None]", 0),
    ("anti-causal-bwd", "allowed = np.arange(r1)[None, :] <= np.arange(r0, r1)[:, None]",
     "allowed = np.arange(r1)[None, :] >= np.arange(r0, r1)[:, None]", 1),
    ("no-scale-fwd", "group_forward(Qg, Kg, Vg, 1.0 / np.sqrt(d))",
     "group_forward(Qg, Kg, Vg, 1.0)", 0),
    ("kv-head-modulo", "return h // (H // Hkv)", "return h % Hkv", 0),
    ("drop-dvec", "dS = P * (dP - Dvec[r0:r1, None])", "dS = P * dP", 0),
    ("dvec-wrong-operand", "Dvec = np.sum(dOg * Og, axis=1)", "Dvec = np.sum(dOg * Qg, axis=1)", 0),
    ("dk-no-scale", "dK[:r1] += scale * (dS.T @ Qg[r0:r1])", "dK[:r1] += dS.T @ Qg[r0:r1]", 0),
    ("dq-wrong-operand", "dQ[r0:r1] = scale * (dS @ Kg[:r1])", "dQ[r0:r1] = scale * (dS @ Vg[:r1])", 0),
    ("dv-scaled", "dV[:r1] += P.T @ dOg[r0:r1]", "dV[:r1] += scale * (P.T @ dOg[r0:r1])", 0),
    ("no-rollback-o", "o[b, rows, h] = Og", "o[b, g * G:(g + 1) * G, h] = Og", 0),
    ("lse-drops-max", "lse[r0:r1] = (m + np.log(l))[:, 0]", "lse[r0:r1] = np.log(l)[:, 0]", 0),
    ("bwd-unmasked-P", "P = np.where(allowed, np.exp(S - lseg[r0:r1, None]), 0.0)",
     "P = np.exp(S - lseg[r0:r1, None])", 0),
    ("gqa-overwrite-dk", "dk[b, rows, c] += dKg", "dk[b, rows, c] = dKg", 0),
    ("transposed-scores", "S = scale * (Qg[r0:r1] @ Kg[:r1].T)\n        allowed",
     "S = scale * (Kg[r0:r1] @ Qg[:r1].T)\n        allowed", 0),
    ("lse-of-rolled-row", "lse[b, h, rows] = lseg", "lse[b, h, g * G:(g + 1) * G] = lseg", 0),
    ("split-ignored", 'if wrap == "split" and sigma:', 'if wrap == "none" and sigma:', 0),
    ("split-in-roll-mode", 'if wrap == "split" and sigma:', 'if sigma:', 0),
    ("split-at-quarter", "return [slice(0, cut), slice(cut, len(rows))]",
     "return [slice(0, cut // 2), slice(cut // 2, len(rows))]", 0),
    ("split-every-group", "        cut = _wrap_cut(rows)\n        if cut is not None:\n            return [slice",
     "        cut = len(rows) // 2\n        if cut is not None:\n            return [slice", 0),
    ("wrap-cut-off-by-one", "return int(wraps[0]) + 1 if len(wraps) else None",
     "return int(wraps[0]) if len(wraps) else None", 0),
    ("swap-ignored", 'if wrap == "swap" and sigma:', 'if wrap == "none" and sigma:', 0),
    ("swap-in-roll-mode", 'if wrap == "swap" and sigma:', 'if sigma:', 0),
    ("swap-keeps-rolled-order", "return np.concatenate([rows[cut:], rows[:cut]])",
     "return np.concatenate([rows[:cut], rows[cut:]])", 0),
    ("swap-every-group", "        cut = _wrap_cut(rows)\n        if cut is not None:\n            return np.concatenate",
     "        cut = len(rows) // 2\n        if cut is not None:\n            return np.concatenate", 0),
    ("swap-front-reversed", "return np.concatenate([rows[cut:], rows[:cut]])",
     "return np.concatenate([rows[cut:][::-1], rows[:cut]])", 0),
    ("rope-interleaved-pairs", "x1, x2 = x[..., :half], x[..., half:]", "x1, x2 = x[..., 0::2], x[..., 1::2]", 0),
    ("rope-sign", "return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)",
     "return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)", 0),
    ("rope-frequency-exponent", "inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)",
     "inv_freq = base ** (-1.0 * np.arange(half, dtype=np.float64) / d)", 0),
    ("rope-scale-ignored", "t = (np.arange(N, dtype=np.float64) * pos_scale)", "t = (np.arange(N, dtype=np.float64) * 1.0)", 0),
    ("rope-position-offset", "t = (np.arange(N, dtype=np.float64) * pos_scale)", "t = (np.arange(1, N + 1, dtype=np.float64) * pos_scale)", 0),
    ("rope-inverse-ignored", "    if inverse:\n        s = -s\n", "", 0),
    ("row-drops-own-key", "keys = rows[part.start:pos + 1]", "keys = rows[part.start:pos]", 0),
    ("row-group-start", "keys = rows[part.start:pos + 1]", "keys = rows[0:pos + 1]", 0),
    ("row-drops-dvec", "ds = p * (dp - np.dot(dot, o))", "ds = p * dp", 0),
    ("groups-rounded-down", "return (N + G - 1) // G", "return N // G", 0),
    ("odd-shift-rounded-up", "return G // 2 if h >= H - shift_heads else 0",
     "return (G + 1) // 2 if h >= H - shift_heads else 0", 0),
    ("split-keeps-wrap-keys", "return [slice(0, cut), slice(cut, len(rows))]",
     "return [slice(0, cut), slice(0, len(rows))]", 0),
]

NEUTRAL = ("reverse-roll-direction", "return (np.arange(N) + sigma) % N", "return (np.arange(N) - sigma) % N", 0)


def _mutant(name, old, new, occ):
    src = open(SRC).read()
    parts = src.split(old)
    assert len(parts) > occ + 1, f"mutation {name}: pattern not found"
    mutated = old.join(parts[:occ + 1]) + new + old.join(parts[occ + 1:])
    assert mutated != src
    mod = types.ModuleType(f"oracle_mutant_{name.replace('-', '_')}")
    exec(compile(mutated, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(mutation):
    mod = _mutant(*mutation)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError) as e:
            failed.append((pin.__name__, str(e)[:80]))
    assert failed, f"no pin caught mutation {mutation[0]}"


def test_direction_reversal_is_not_a_mistake():
    """Every output is invariant; only the index map itself shows the direction.

    That holds when G divides N (the two rolls differ by one whole group).  When
    it does not, the reversed roll puts the group grid elsewhere, so the
    unaligned pins must notice it (the pages' direction, -G/2, is the one taken).
    """
    mod = _mutant(*NEUTRAL)
    direction_sensitive = (pins.pin_worked_example_index_map, pins.pin_unaligned_bruteforce,
                           pins.pin_unaligned_cut_sdpa, pins.pin_unaligned_row_attention,
                           pins.pin_unaligned_swap_gathered_sdpa)
    for pin in pins.ALL_PINS:
        if pin in direction_sensitive:
            with pytest.raises(AssertionError):
                pin(mod)
        else:
            pin(mod)
