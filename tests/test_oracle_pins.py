"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against something the pages or the mathematics
fix independently of the oracle's own code: a hand-worked example with exact
rational answers, a brute-force evaluation of the definition, a library
routine (torch's fp64 scaled-dot-product attention, scipy's logsumexp),
closed forms, and invariants of softmax.  ``test_oracle_mutants.py`` plants
plausible mistakes in copies of the oracle and checks these pins catch them.
"""
import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

from oracle import attention_ref
from tests.oracle_pin_checks import (
    brute_force, golden_cases, online_blocked, rng_qkv,
)

GOLDEN = Path(__file__).parent / "golden" / "hand_softmax_weights.txt"


# --- hand-worked example -------------------------------------------------

GOLDEN_CASES = {            # case -> (causal, window)
    "noncausal": (False, None), "causal": (True, None), "rect_causal": (True, None),
    "window_causal": (True, (1, None)), "band": (False, (1, 1)),
}


@pytest.mark.parametrize("case", list(GOLDEN_CASES))
def test_golden_hand_example(case):
    g = golden_cases(GOLDEN)
    q, k, v, scale = g["q"], g["k"], g["v"], g["scale"]
    if case == "rect_causal":
        q = q[:2]
    causal, window = GOLDEN_CASES[case]
    O, L = attention_ref(q[None, None], k[None, None], v[None, None],
                         causal, scale, window=window)
    np.testing.assert_allclose(O[0, 0], g[f"{case} O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], g[f"{case} LSE"], rtol=0, atol=1e-12)


# --- brute force on tiny inputs ------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk,d", [(1, 1, 1), (3, 5, 2), (5, 3, 4),
                                     (8, 8, 3), (7, 2, 4), (2, 8, 1)])
def test_brute_force(causal, Lq, Lk, d):
    for seed in range(3):
        q, k, v = rng_qkv(seed, 2, 1, Lq, Lk, d)
        scale = 0.7
        O, L = attention_ref(q, k, v, causal, scale)
        for b in range(2):
            Ob, Lb = brute_force(q[b, 0], k[b, 0], v[b, 0], causal, scale)
            np.testing.assert_allclose(O[b, 0], Ob, rtol=0, atol=1e-13)
            np.testing.assert_allclose(L[b, 0], Lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_seeded_sweep(seed):
    """The definition by brute force over seeded random tiny problems: any
    Lq, Lk in 1..10 and d in 1..5, B and H up to 2, full, causal or a random
    window (either side unbounded or not, rows with no key included), scale
    from 0 to 3 and scores up to 300 in magnitude (peaky rows)."""
    rng = np.random.default_rng(7000 + seed)
    for _ in range(12):
        B, H = (int(x) for x in rng.integers(1, 3, size=2))
        Lq, Lk = (int(x) for x in rng.integers(1, 11, size=2))
        d = int(rng.integers(1, 6))
        mode = ("full", "causal", "window")[int(rng.integers(3))]
        scale = float(rng.choice([0.0, 0.05, 0.3, 1.0, 3.0]))
        sigma = float(rng.choice([0.5, 1.0, 4.0, 10.0]))
        q, k, v = (sigma * rng.standard_normal((B, H, n, d)) for n in (Lq, Lk, Lk))
        # keep every score within math.exp's range (|s| <= 300)
        smax = scale * np.abs(np.einsum("bhid,bhjd->bhij", q, k)).max()
        if smax > 300.0:
            q, k = q * math.sqrt(300.0 / smax), k * math.sqrt(300.0 / smax)
        window = None
        if mode == "window":
            window = tuple(None if rng.random() < 0.25 else int(rng.integers(0, 6))
                           for _ in range(2))
        causal = mode == "causal"
        O, L = attention_ref(q, k, v, causal, scale, window=window)
        for b in range(B):
            for h in range(H):
                Ob, Lb = brute_force(q[b, h], k[b, h], v[b, h], causal, scale, window)
                np.testing.assert_allclose(O[b, h], Ob, rtol=1e-12, atol=1e-12)
                np.testing.assert_array_equal(np.isinf(L[b, h]), np.isinf(Lb))
                fin = np.isfinite(Lb)
                np.testing.assert_allclose(L[b, h][fin], Lb[fin], rtol=1e-13, atol=1e-12)


# --- library routines ----------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Lq,Lk,d", [(2, 3, 37, 37, 16), (1, 2, 64, 100, 8),
                                         (1, 1, 90, 33, 32)])
def test_sdpa_library(causal, B, H, Lq, Lk, d):
    import torch
    import torch.nn.functional as F
    q, k, v = rng_qkv(11, B, H, Lq, Lk, d)
    scale = 1.0 / math.sqrt(d)
    O, _ = attention_ref(q, k, v, causal, scale)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_scipy_logsumexp(causal):
    from scipy.special import logsumexp
    q, k, v = rng_qkv(5, 1, 2, 40, 50, 8)
    scale = 0.35
    _, L = attention_ref(q, k, v, causal, scale)
    s = np.einsum("bhid,bhjd->bhij", q, k) * scale
    if causal:
        mask = np.arange(50)[None, :] <= np.arange(40)[:, None]
        s = np.where(mask, s, -np.inf)
    np.testing.assert_allclose(L, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


# --- softmax invariants --------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    q, k, v = rng_qkv(3, 1, 2, 33, 45, 8, sigma=3.0)
    scale = 0.5
    O, L, P = attention_ref(q, k, v, causal, scale, return_p=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (P >= 0).all() and (P <= 1).all()
    s = np.einsum("bhid,bhjd->bhij", q, k) * scale
    vis = np.ones_like(s, dtype=bool)
    if causal:
        vis = np.broadcast_to(np.arange(45)[None, :] <= np.arange(33)[:, None],
                              s.shape)
    # P is recovered from the scores and LSE alone (chuoer47 section 3:
    # softmax(x_i) = exp(x_i - LSE))
    rebuilt = np.where(vis, np.exp(s - L[..., None]), 0.0)
    np.testing.assert_allclose(P, rebuilt, rtol=0, atol=1e-12)
    m = np.where(vis, s, -np.inf).max(-1)
    n = vis.sum(-1)
    assert (L >= m - 1e-12).all() and (L <= m + np.log(n) + 1e-12).all()
    # O lies in the convex hull of the visible values, per coordinate
    for b in range(1):
        for h in range(2):
            for i in range(33):
                vv = v[b, h][vis[b, h, i]]
                assert (O[b, h, i] >= vv.min(0) - 1e-12).all()
                assert (O[b, h, i] <= vv.max(0) + 1e-12).all()


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    # adding the same vector u to every key shifts row i's scores by
    # scale*q_i.u: P and O unchanged, LSE shifted by that amount
    q, k, v = rng_qkv(8, 1, 2, 30, 30, 6)
    u = np.random.default_rng(1).standard_normal(6)
    scale = 0.4
    O1, L1 = attention_ref(q, k, v, causal, scale)
    O2, L2 = attention_ref(q, k + u, v, causal, scale)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L1 + scale * (q @ u), rtol=0, atol=1e-12)


def test_permutation_equivariance():
    q, k, v = rng_qkv(9, 1, 1, 20, 24, 5)
    O, L = attention_ref(q, k, v, False, 0.6)
    pk = np.random.default_rng(2).permutation(24)
    O2, L2 = attention_ref(q, k[:, :, pk], v[:, :, pk], False, 0.6)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L, rtol=0, atol=1e-12)
    pq = np.random.default_rng(3).permutation(20)
    O3, L3 = attention_ref(q[:, :, pq], k, v, False, 0.6)
    np.testing.assert_allclose(O3, O[:, :, pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L3, L[:, :, pq], rtol=0, atol=1e-12)


def test_causality():
    q, k, v = rng_qkv(10, 1, 1, 16, 16, 4)
    O, L = attention_ref(q, k, v, True, 0.5)
    for i in [0, 5, 14]:
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] += 7.0
        v2[:, :, i + 1:] -= 3.0
        O2, L2 = attention_ref(q, k2, v2, True, 0.5)
        np.testing.assert_array_equal(O2[:, :, i], O[:, :, i])
        np.testing.assert_array_equal(L2[:, :, i], L[:, :, i])
        assert np.abs(O2[:, :, i + 1:] - O[:, :, i + 1:]).max() > 1e-3


# --- closed forms --------------------------------------------------------

def test_scale_zero_means():
    q, k, v = rng_qkv(12, 1, 2, 9, 13, 3)
    O, L = attention_ref(q, k, v, False, 0.0)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(2, keepdims=True),
                                                  O.shape), atol=1e-13)
    np.testing.assert_allclose(L, math.log(13), atol=1e-13)
    Oc, Lc = attention_ref(q, k, v, True, 0.0)
    prefix = np.cumsum(v, axis=2)[:, :, :9] / np.arange(1, 10)[:, None]
    np.testing.assert_allclose(Oc, prefix, atol=1e-13)
    np.testing.assert_allclose(Lc, np.broadcast_to(np.log(np.arange(1, 10)),
                                                   Lc.shape), atol=1e-13)


def test_causal_first_row_and_single_key():
    q, k, v = rng_qkv(13, 2, 2, 11, 11, 7)
    O, L = attention_ref(q, k, v, True, 0.3)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0],
                               0.3 * (q[:, :, 0] * k[:, :, 0]).sum(-1),
                               atol=1e-13)
    O1, L1 = attention_ref(q, k[:, :, :1], v[:, :, :1], False, 0.3)
    np.testing.assert_array_equal(O1, np.broadcast_to(v[:, :, :1], O1.shape))
    np.testing.assert_allclose(L1, 0.3 * (q * k[:, :, :1]).sum(-1), atol=1e-13)


def test_identical_keys_uniform_and_one_hot():
    q, k, v = rng_qkv(14, 1, 1, 6, 10, 4)
    kk = np.broadcast_to(k[:, :, :1], k.shape).copy()
    O, _ = attention_ref(q, kk, v, False, 0.9)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(2, keepdims=True),
                                                  O.shape), atol=1e-13)
    # one key dominates each row by a gap of >100 in score: O = that value
    kp = np.zeros((1, 1, 10, 4))
    qp = np.zeros((1, 1, 6, 4))
    for i in range(6):
        qp[0, 0, i, i % 4] = 1.0
    for j in range(4):
        kp[0, 0, 2 * j + 1, j] = 400.0
    O, L = attention_ref(qp, kp, v, False, 1.0)
    for i in range(6):
        j = 2 * (i % 4) + 1
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, j], atol=1e-12)
        np.testing.assert_allclose(L[0, 0, i], 400.0, atol=1e-12)


# --- the online recurrence the kernel runs -------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 16, 64, 1000])
def test_online_recurrence_equals_oracle(causal, block):
    q, k, v = rng_qkv(15, 1, 2, 70, 90, 8, sigma=2.0)
    O, L = attention_ref(q, k, v, causal, 0.45)
    for h in range(2):
        Ob, Lb = online_blocked(q[0, h], k[0, h], v[0, h], causal, 0.45, block)
        np.testing.assert_allclose(Ob, O[0, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lb, L[0, h], rtol=0, atol=1e-12)


# --- evaluation helpers --------------------------------------------------

def test_row_subset_and_workers_agree():
    q, k, v = rng_qkv(16, 2, 3, 300, 310, 16)
    O, L = attention_ref(q, k, v, True, 0.25, chunk=64)
    rows = np.array([0, 1, 63, 64, 299, 150])
    Os, Ls = attention_ref(q, k, v, True, 0.25, rows=rows, chunk=4)
    np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Ls, L[:, :, rows], rtol=0, atol=1e-13)
    Ow, Lw = attention_ref(q, k, v, True, 0.25, chunk=64, workers=4)
    np.testing.assert_array_equal(Ow, O)
    np.testing.assert_array_equal(Lw, L)


def test_algorithmic_flops_closed_form():
    from oracle import algorithmic_flops
    L, d = 1000, 64
    # causal: pairs (i, j) with j <= i -> L(L+1)/2; non-causal L*Lk
    assert algorithmic_flops(np.arange(L), L, d, True) == 4 * d * L * (L + 1) / 2
    assert algorithmic_flops(np.arange(L), 700, d, False) == 4 * d * L * 700
    # causal with Lk < Lq: rows past Lk see all Lk keys
    assert algorithmic_flops(np.arange(10), 4, 2, True) == 4 * 2 * (1 + 2 + 3 + 4 * 7)


# --- sliding window ("Flash Attention 原理与实现详解" (tbr8.org), section 6.3
# "滑动窗口注意力": a (left, right) window-size pair, (1024, 0) with causal) --

WINDOWS = [(True, (0, None)), (True, (3, None)), (False, (2, 2)),
           (False, (None, 1)), (False, (4, 0)), (True, (1, 5))]


@pytest.mark.parametrize("causal,window", WINDOWS)
@pytest.mark.parametrize("Lq,Lk,d", [(9, 9, 3), (6, 11, 2), (12, 5, 4)])
def test_window_brute_force(causal, window, Lq, Lk, d):
    q, k, v = rng_qkv(21, 1, 2, Lq, Lk, d)
    O, L = attention_ref(q, k, v, causal, 0.6, window=window)
    for h in range(2):
        Ob, Lb = brute_force(q[0, h], k[0, h], v[0, h], causal, 0.6, window)
        np.testing.assert_allclose(O[0, h], Ob, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(L[0, h]), np.isneginf(Lb))
        fin = np.isfinite(Lb)
        np.testing.assert_allclose(L[0, h][fin], Lb[fin], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", WINDOWS)
def test_window_sdpa_band_mask(causal, window):
    """torch's fp64 SDPA with an explicit boolean band mask (rows that keep
    at least one key; SDPA has no convention for empty rows)."""
    import torch
    import torch.nn.functional as F
    Lq, Lk, d = 40, 52, 8
    q, k, v = rng_qkv(22, 1, 2, Lq, Lk, d)
    O, _ = attention_ref(q, k, v, causal, 0.3, window=window)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    keep = np.ones((Lq, Lk), dtype=bool)
    if causal:
        keep &= j <= i
    if window[0] is not None:
        keep &= j >= i - window[0]
    if window[1] is not None:
        keep &= j <= i + window[1]
    rows = keep.any(axis=1)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(keep), scale=0.3).numpy()
    np.testing.assert_allclose(O[:, :, rows], ref[:, :, rows], rtol=0, atol=1e-12)


def test_window_zero_is_identity():
    """window (0, 0): each query sees only its own key: O_i = v_i and
    LSE_i = scale q_i . k_i exactly."""
    q, k, v = rng_qkv(23, 1, 1, 30, 30, 5)
    O, L = attention_ref(q, k, v, False, 0.8, window=(0, 0))
    np.testing.assert_allclose(O[0, 0], v[0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[0, 0], 0.8 * np.einsum("id,id->i", q[0, 0], k[0, 0]),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("left,right", [(3, 0), (5, 2), (None, 4), (0, None)])
def test_window_scale_zero_band_means(left, right):
    """scale 0: uniform weights over the band, O_i = mean of v over
    [max(0, i-left), min(Lk-1, i+right)] and LSE_i = ln(count)."""
    Lq, Lk = 20, 17
    q, k, v = rng_qkv(24, 1, 1, Lq, Lk, 3)
    O, L = attention_ref(q, k, v, False, 0.0, window=(left, right))
    csum = np.concatenate([np.zeros((1, 3)), np.cumsum(v[0, 0], axis=0)])
    for i in range(Lq):
        lo = 0 if left is None else max(0, i - left)
        hi = Lk - 1 if right is None else min(Lk - 1, i + right)
        if hi < lo:
            assert np.isneginf(L[0, 0, i]) and not O[0, 0, i].any()
            continue
        n = hi - lo + 1
        np.testing.assert_allclose(O[0, 0, i], (csum[hi + 1] - csum[lo]) / n,
                                   rtol=0, atol=1e-13)
        assert abs(L[0, 0, i] - math.log(n)) < 1e-13


def test_window_reduces_to_causal_and_full():
    q, k, v = rng_qkv(25, 2, 2, 33, 33, 6)
    Oc, Lc = attention_ref(q, k, v, True, 0.5)
    Ow, Lw = attention_ref(q, k, v, False, 0.5, window=(None, 0))
    np.testing.assert_allclose(Ow, Oc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Lw, Lc, rtol=0, atol=1e-14)
    Ow, Lw = attention_ref(q, k, v, True, 0.5, window=(33, None))
    np.testing.assert_allclose(Ow, Oc, rtol=0, atol=1e-14)
    Of, Lf = attention_ref(q, k, v, False, 0.5)
    Ow, Lw = attention_ref(q, k, v, False, 0.5, window=(40, 40))
    np.testing.assert_allclose(Ow, Of, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Lw, Lf, rtol=0, atol=1e-14)


def test_window_empty_rows():
    """Lq > Lk with a left bound: rows i > Lk - 1 + left see no key; they
    read O = 0 and LSE = -inf, every other row is finite."""
    q, k, v = rng_qkv(26, 1, 1, 12, 4, 3)
    O, L = attention_ref(q, k, v, True, 0.5, window=(2, None))
    empty = np.arange(12) > 4 - 1 + 2
    assert np.isneginf(L[0, 0, empty]).all() and not O[0, 0, empty].any()
    assert np.isfinite(L[0, 0, ~empty]).all()


@pytest.mark.parametrize("window", [(5, None), (7, 3), (None, 2)])
@pytest.mark.parametrize("block", [1, 7, 16, 64])
def test_window_online_recurrence(window, block):
    causal = window[1] is None
    q, k, v = rng_qkv(27, 1, 1, 70, 90, 8, sigma=2.0)
    O, L = attention_ref(q, k, v, causal, 0.45, window=window)
    Ob, Lb = online_blocked(q[0, 0], k[0, 0], v[0, 0], causal, 0.45, block, window)
    np.testing.assert_allclose(Ob, O[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lb, L[0, 0], rtol=0, atol=1e-12)


def test_window_algorithmic_flops_closed_form():
    from oracle import algorithmic_flops
    L, W, d = 1000, 100, 64
    # causal, left window W: row i sees min(i, W) + 1 keys
    pairs = sum(min(i, W) + 1 for i in range(L))
    assert pairs == L * (W + 1) - W * (W + 1) // 2
    assert algorithmic_flops(np.arange(L), L, d, True, (W, None)) == 4 * d * pairs
    # window (0, 0): one pair per row that has a key
    assert algorithmic_flops(np.arange(10), 6, d, False, (0, 0)) == 4 * d * 6


# --- key splits and their merge ("Flash Attention 原理与实现详解" (tbr8.org),
# section 2.1 "Tiling（分块计算）策略", the block-merge step) ------------------

def _split_points(Lk, splits, rng):
    cuts = np.sort(rng.choice(np.arange(1, Lk), size=splits - 1, replace=False))
    return [0, *cuts.tolist(), Lk]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_merge_of_key_splits_equals_full(causal, splits):
    """Partials over disjoint key ranges, merged, give the full result; for
    causal rows some ranges are empty (LSE = -inf) and must drop out."""
    from oracle import merge_partials
    q, k, v = rng_qkv(40 + splits, 1, 2, 37, 53, 6, sigma=1.5)
    O, L = attention_ref(q, k, v, causal, 0.4)
    cut = _split_points(53, splits, np.random.default_rng(splits))
    parts = [attention_ref(q, k, v, causal, 0.4, keys=(a, b))
             for a, b in zip(cut[:-1], cut[1:])]
    Om, Lm = merge_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-13)


def test_key_range_partial_is_attention_over_that_range():
    """A partial is plain attention over the keys of its range (brute force
    on the sliced K and V), and a row with no key in range is empty."""
    q, k, v = rng_qkv(44, 1, 1, 9, 12, 3)
    O, L = attention_ref(q, k, v, True, 0.9, keys=(4, 10))
    for i in range(9):
        js = [j for j in range(4, 10) if j <= i]
        if not js:
            assert np.isneginf(L[0, 0, i]) and not O[0, 0, i].any()
            continue
        Ob, Lb = brute_force(q[0, 0, i:i + 1], k[0, 0, js], v[0, 0, js], False, 0.9)
        np.testing.assert_allclose(O[0, 0, i], Ob[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[0, 0, i], Lb[0], rtol=0, atol=1e-13)


def test_merge_lse_is_logsumexp_and_order_free():
    from scipy.special import logsumexp
    from oracle import merge_partials
    rng = np.random.default_rng(45)
    Op = rng.standard_normal((5, 2, 3, 4))
    Lp = rng.standard_normal((5, 2, 3)) * 4
    Lp[1, 0, 0] = -np.inf                      # an empty partial
    Om, Lm = merge_partials(Op, Lp)
    np.testing.assert_allclose(Lm, logsumexp(Lp, axis=0), rtol=0, atol=1e-13)
    w = np.exp(Lp - Lm[None])
    np.testing.assert_allclose(Om, (w[..., None] * Op).sum(axis=0), rtol=0, atol=1e-13)
    perm = [3, 0, 4, 2, 1]
    Op2, Lp2 = merge_partials(Op[perm], Lp[perm])
    np.testing.assert_allclose(Op2, Om, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Lp2, Lm, rtol=0, atol=1e-13)
    # all partials empty: the row is empty
    Oe, Le = merge_partials(np.zeros((3, 1, 2)), np.full((3, 1), -np.inf))
    assert np.isneginf(Le).all() and not Oe.any()
