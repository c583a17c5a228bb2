"""Plant plausible mistakes in the oracle (on the CPU) and check the pins
reject every one of them.

Each mutant replaces the oracle's per-chunk evaluation with a copy that has
one mistake (a dropped term, a wrong sign, index or operand, a wrong log
base, an off-by-one mask).  The pin set below (the hand-worked fixture,
brute force, the library routine) must fail on each.
"""
from pathlib import Path

import numpy as np
import pytest

import oracle.attention_fp64 as ref_mod
from oracle import attention_ref
from tests.oracle_pin_checks import brute_force, golden_cases, rng_qkv

GOLDEN = Path(__file__).parent / "golden" / "hand_softmax_weights.txt"


def _make_mutant(kind):
    def chunk(q64, k64, v64, rows, causal, scale, want_p, window=None, keys=None):
        left, right = window if window is not None else (None, None)
        if kind == "window_sides_swapped":
            left, right = right, left
        Lk = k64.shape[0]
        ncols = Lk if not causal else min(Lk, int(rows.max()) + 1)
        if kind == "causal_plus_one":
            ncols = Lk if not causal else min(Lk, int(rows.max()) + 2)
        s = q64 @ k64[:ncols].T
        if kind != "no_scale":
            s = s * scale
        if kind == "sign":
            s = -s
        cols = np.arange(ncols)[None, :]
        if causal:
            if kind == "strict_causal":
                allowed = cols < rows[:, None]
            elif kind == "causal_plus_one":
                allowed = cols <= rows[:, None] + 1
            elif kind == "bottom_right":
                allowed = cols <= rows[:, None] + (Lk - int(rows.max()) - 1)
            else:
                allowed = cols <= rows[:, None]
        else:
            allowed = np.ones((len(rows), ncols), dtype=bool)
        if left is not None:
            if kind == "window_left_strict":
                allowed = allowed & (cols > rows[:, None] - left)
            elif kind == "window_left_plus_one":
                allowed = allowed & (cols >= rows[:, None] - left - 1)
            else:
                allowed = allowed & (cols >= rows[:, None] - left)
        if right is not None:
            allowed = allowed & (cols <= rows[:, None] + right)
        sm = np.where(allowed, s, -np.inf)
        m = sm.max(axis=1)
        with np.errstate(invalid="ignore", divide="ignore"):
            e = np.where(allowed, np.exp(sm - m[:, None]), 0.0)
        l = e.sum(axis=1)
        if kind == "column_normalise":
            p = e / np.maximum(e.sum(axis=0, keepdims=True), 1e-300)
        else:
            p = e / l[:, None]
        vals = k64 if kind == "keys_as_values" else v64
        o = p @ vals[:ncols]
        if kind == "lse_log2":
            lse = m + np.log2(l)
        elif kind == "lse_no_max":
            lse = np.log(l)
        else:
            lse = m + np.log(l)
        return o, lse, None
    return chunk


MUTANTS = ["no_scale", "sign", "strict_causal", "causal_plus_one",
           "bottom_right", "column_normalise", "keys_as_values", "lse_log2",
           "lse_no_max", "window_left_strict", "window_left_plus_one",
           "window_sides_swapped"]


def _pins_pass():
    try:
        g = golden_cases(GOLDEN)
        for case in ("noncausal", "causal", "rect_causal"):
            q = g["q"][:2] if case == "rect_causal" else g["q"]
            O, L = attention_ref(q[None, None], g["k"][None, None],
                                 g["v"][None, None], case != "noncausal",
                                 g["scale"])
            np.testing.assert_allclose(O[0, 0], g[f"{case} O"], atol=1e-12)
            np.testing.assert_allclose(L[0, 0], g[f"{case} LSE"], atol=1e-12)
        for causal in (False, True):
            for (Lq, Lk, d) in ((5, 3, 4), (3, 6, 2)):
                q, k, v = rng_qkv(1, 1, 1, Lq, Lk, d)
                O, L = attention_ref(q, k, v, causal, 0.7)
                Ob, Lb = brute_force(q[0, 0], k[0, 0], v[0, 0], causal, 0.7)
                np.testing.assert_allclose(O[0, 0], Ob, atol=1e-12)
                np.testing.assert_allclose(L[0, 0], Lb, atol=1e-12)
        # sliding windows: left only (with causal), both sides, right only
        for causal, window in ((True, (2, None)), (False, (1, 3)), (False, (None, 1))):
            q, k, v = rng_qkv(2, 1, 1, 7, 7, 3)
            O, L = attention_ref(q, k, v, causal, 0.7, window=window)
            Ob, Lb = brute_force(q[0, 0], k[0, 0], v[0, 0], causal, 0.7, window)
            np.testing.assert_allclose(O[0, 0], Ob, atol=1e-12)
            np.testing.assert_allclose(L[0, 0], Lb, atol=1e-12)
    except AssertionError:
        return False
    return True


def test_unmutated_oracle_passes_the_pin_set():
    assert _pins_pass()


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ref_mod, "_chunk_ref", _make_mutant(kind))
    assert not _pins_pass(), f"pins failed to catch mutant {kind!r}"
