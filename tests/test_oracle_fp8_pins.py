"""Pins of the FP8 oracle (oracle/attention_fp8.py) and of the E4M3 input
codec (seeded_inputs) to things other than themselves.

* The format: named E4M3 codes whose values follow from the OCP FP8 E4M3
  definition (bias 7, 3 mantissa bits, no infinities, 448 the largest
  finite value), and torch's own float8_e4m3fn conversions (a library
  routine) for every code and a dense grid of values.
* The algebra: the blocked algorithm without rounding equals the exact
  fp64 definition for many block sizes; a pure-Python loop evaluation of the
  blocked FP8 algorithm (math.exp, torch's E4M3 rounding) on tiny inputs.
* Closed forms: scale 0 (every 2^8 P is exactly 256, so no rounding error),
  a two-key row whose rounded P is a known E4M3 tie.
* The derived error bound holds on random and peaky inputs and is nearly
  attained where it should be.
* With an S error inside the stated bound (random noise on the scores),
  the blocked result stays within its allowance and the exact definition's
  bound.
* Planted mistakes in copies of the oracle (dropped 2^8 shift, l from the
  rounded P, no rescale, ties away from zero) are each rejected.
* The S-error model (fp32_sum_error_factor): products of E4M3 values are
  exact in fp32; fp32 sums of such products in random orders, rounded to
  nearest or toward zero, stay within the factor; and a sum built so that
  truncation loses almost a whole unit at every addition comes within 1 %
  of it, so a factor of half the size would be violated.
"""
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle.attention_fp8 as f8
from oracle import attention_ref
from seeded_inputs import (e4m3_decode, e4m3_encode, make_inputs_fp8, quantize_e4m3,
                           widen_fp8)

SRC = Path(f8.__file__).read_text()


def torch_e4m3(x):
    """torch's float32 -> float8_e4m3fn -> float64 (round to nearest even)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---- the format ------------------------------------------------------------

NAMED = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
         0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x78: 256.0,
         0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}


@pytest.mark.parametrize("code,value", sorted(NAMED.items()))
def test_e4m3_named_codes(code, value):
    got = float(e4m3_decode(np.array([code], dtype=np.uint8))[0])
    assert got == value and math.copysign(1, got) == math.copysign(1, value)
    assert e4m3_encode(np.array([value]))[0] == code


def test_e4m3_nan_codes():
    d = e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(d).all()


def test_decode_matches_torch_all_codes():
    c = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3_decode(c), t, equal_nan=True)


def test_encode_matches_torch_dense_grid():
    x = np.concatenate([np.linspace(-448, 448, 400001), np.linspace(-0.02, 0.02, 40001)])
    x = x.astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), codes)


def test_oracle_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([np.linspace(0, 448, 300001), rng.uniform(0, 300, 20000),
                        rng.uniform(0, 2.0 ** -6, 20000), -rng.uniform(0, 448, 1000)])
    x = x.astype(np.float32)
    assert np.array_equal(f8.e4m3_round(x), torch_e4m3(x))


def test_rounding_ties_to_even():
    # 136 lies halfway between 128 (mantissa 000) and 144 (mantissa 001)
    assert f8.e4m3_round(np.array([136.0, 152.0, 3 * 2.0 ** -10]))[0] == 128.0
    assert f8.e4m3_round(np.array([152.0]))[0] == 160.0
    assert f8.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8


def test_quantize_roundtrip_and_scale():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 300)).astype(np.float32)
    codes, ds = quantize_e4m3(x)
    assert ds == np.float32(np.abs(x).max() / 448.0)
    y = widen_fp8(codes, ds)
    # within half a spacing of E4M3 (relative 2^-4) or of the subnormals
    assert (np.abs(y - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * ds) * (1 + 1e-6)).all()
    assert np.abs(y).max() == pytest.approx(np.abs(x).max(), rel=1e-6)


# ---- the algebra --------------------------------------------------------------

def fp8_case(seed, B, H, Lq, Lk, d, sigma=1.0):
    q8, k8, v8, (qd, kd, vd) = make_inputs_fp8(seed, B, H, Lq, Lk, d, sigma_qk=sigma)
    return widen_fp8(q8, qd), widen_fp8(k8, kd), widen_fp8(v8, vd)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 16, 64, 1000])
def test_blocked_without_rounding_is_exact(causal, block):
    q, k, v = fp8_case(11, 1, 2, 70, 90, 16)
    scale = 0.25
    O, L = f8.attention_fp8_blocked(q, k, v, causal, scale, block, round_p=False)
    Or, Lr = attention_ref(q, k, v, causal, scale)
    assert np.abs(O - Or).max() <= 1e-12
    assert np.abs(L - Lr).max() <= 1e-12


def _loop_blocked(q, k, v, causal, scale, block):
    """Pure-Python evaluation of the blocked FP8 algorithm for one head:
    math.exp, and torch's E4M3 conversion to round 2^8 P."""
    Lq, d = q.shape
    Lk = k.shape[0]
    O, LSE = np.zeros((Lq, d)), np.zeros(Lq)
    for i in range(Lq):
        m, l, acc = -math.inf, 0.0, [0.0] * d
        for j0 in range(0, Lk, block):
            js = [j for j in range(j0, min(j0 + block, Lk)) if not causal or j <= i]
            if not js:
                continue
            s = {j: scale * math.fsum(q[i, t] * k[j, t] for t in range(d)) for j in js}
            m_new = max(m, max(s.values()))
            alpha = math.exp(m - m_new) if m > -math.inf else 0.0
            l *= alpha
            acc = [a * alpha for a in acc]
            for j in js:
                p = math.exp(s[j] - m_new) * 256.0
                pr = float(torch.tensor(p, dtype=torch.float64).to(torch.float8_e4m3fn)
                           .to(torch.float64))
                l += p
                for t in range(d):
                    acc[t] += pr * v[j, t]
            m = m_new
        O[i] = [a / l for a in acc]
        LSE[i] = m + math.log(l) - 8 * math.log(2)
    return O, LSE


@pytest.mark.parametrize("causal", [False, True])
def test_blocked_matches_loop_evaluation(causal):
    q, k, v = fp8_case(12, 1, 1, 6, 8, 4, sigma=2.0)
    scale = 0.5
    for block in (1, 3, 8):
        O, L = f8.attention_fp8_blocked(q, k, v, causal, scale, block)
        Ob, Lb = _loop_blocked(q[0, 0], k[0, 0], v[0, 0], causal, scale, block)
        assert np.abs(O[0, 0] - Ob).max() <= 1e-12
        assert np.abs(L[0, 0] - Lb).max() <= 1e-12


# ---- closed forms -------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_closed_form(causal):
    q, k, v = fp8_case(13, 1, 2, 40, 40, 8)
    O, L = f8.attention_fp8_blocked(q, k, v, causal, 0.0, 16)
    if causal:
        want = np.cumsum(v, axis=2) / np.arange(1, 41)[None, None, :, None]
        wantL = np.log(np.arange(1, 41))[None, None, :]
    else:
        want = np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape)
        wantL = np.full(L.shape, math.log(40))
    assert np.abs(O - want).max() <= 1e-12
    assert np.abs(L - wantL).max() <= 1e-12


def test_two_key_tie_closed_form():
    """Scores 0 and ln(17/32): 2^8 P = (256, 136); 136 is an E4M3 tie that
    rounds to 128.  O = (256 v0 + 128 v1) / (256 + 136), LSE = ln(1 + 17/32)."""
    d = 2
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, d)); k[0, 0, 1, 0] = math.log(17 / 32)
    v = np.array([[[[1.0, -2.0], [3.0, 5.0]]]])
    O, L = f8.attention_fp8_blocked(q, k, v, False, 1.0, 2)
    want = (256 * v[0, 0, 0] + 128 * v[0, 0, 1]) / (256 + 136)
    assert np.abs(O[0, 0, 0] - want).max() <= 1e-13
    assert abs(L[0, 0, 0] - math.log(1 + 17 / 32)) <= 1e-13
    # and the bound holds and is nearly attained there
    Or, _ = attention_ref(q, k, v, False, 1.0)
    bound = f8.fp8_error_bound(q, k, v, False, 1.0)
    err = np.abs(O - Or)
    assert (err <= bound).all() and (err >= 0.5 * bound).any()


# ---- the error bound -----------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sigma,block", [(1.0, 64), (3.0, 32), (1.0, 5)])
def test_rounding_error_within_bound(causal, sigma, block):
    q, k, v = fp8_case(14, 1, 2, 150, 200, 32, sigma=sigma)
    scale = 1 / math.sqrt(32)
    O, L = f8.attention_fp8_blocked(q, k, v, causal, scale, block)
    Or, Lr = attention_ref(q, k, v, causal, scale)
    bound = f8.fp8_error_bound(q, k, v, causal, scale)
    assert (np.abs(O - Or) <= bound + 1e-12).all()
    assert np.abs(L - Lr).max() <= 1e-12          # l comes from the unrounded P
    assert np.abs(O - Or).max() > 0               # the rounding does act


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s_err", [f8.fp32_sum_error_factor(128), 2.0 ** -8])
def test_s_error_allowance_and_bound(causal, s_err):
    """S perturbed within the stated bound (random noise up to
    s_err * scale * sum|q||k| per score): the blocked result moves by no more
    than its allowance, and stays within the exact definition's bound."""
    q, k, v = fp8_case(15, 1, 2, 120, 150, 32)
    scale = 1 / math.sqrt(32)
    O, L, allow = f8.attention_fp8_blocked(q, k, v, causal, scale, 32, s_err=s_err)
    O0, _ = f8.attention_fp8_blocked(q, k, v, causal, scale, 32)
    assert np.array_equal(O, O0)
    Oe, _ = attention_ref(q, k, v, causal, scale)
    bound = f8.fp8_error_bound(q, k, v, causal, scale, s_err=s_err)
    dmax = s_err * scale * np.einsum("bhid,bhjd->bhij", np.abs(q), np.abs(k))
    rng = np.random.default_rng(4)
    moved = 0.0
    for _ in range(4):
        noise = rng.uniform(-1, 1, dmax.shape) * dmax
        On, Ln = f8.attention_fp8_blocked(q, k, v, causal, scale, 32, s_noise=noise)
        assert (np.abs(On - O) <= allow * (1 + 1e-9) + 1e-13).all()
        assert (np.abs(On - Oe) <= bound * (1 + 1e-9) + 1e-13).all()
        moved = max(moved, float(np.abs(On - O).max()))
    assert moved > 0
    if s_err < 2.0 ** -8:
        # at the model's bound, the allowance is far below the size of O
        assert allow.max() < 0.05 * np.abs(O).max()


# ---- the S-error model ------------------------------------------------------

def _f32_add(a, b, toward_zero):
    """One fp32 addition of fp32 values, rounded to nearest even or toward
    zero (the exact sum of two fp32 values of nearby magnitude is exact in
    fp64, then rounded once to fp32)."""
    exact = float(a) + float(b)
    r = np.float32(exact)
    if toward_zero and abs(float(r)) > abs(exact):
        r = np.nextafter(r, np.float32(0.0), dtype=np.float32)
    return r


def _f32_sum(x, order, toward_zero):
    acc = np.float32(0.0)
    for i in order:
        acc = _f32_add(acc, x[i], toward_zero)
    return float(acc)


def test_e4m3_products_exact_in_fp32():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    vals = vals[np.isfinite(vals)]
    prod = np.outer(vals, vals)
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)


@pytest.mark.parametrize("n", [64, 128])
def test_sum_error_factor_holds_on_fp32_sums(n):
    gamma = f8.fp32_sum_error_factor(n)
    assert gamma == pytest.approx((n - 1) * 2.0 ** -23, rel=1e-4)
    rng = np.random.default_rng(n)
    worst = 0.0
    for trial in range(60):
        q = e4m3_decode(rng.integers(0, 256, n, dtype=np.uint8))
        k = e4m3_decode(rng.integers(0, 256, n, dtype=np.uint8))
        q = np.where(np.isfinite(q), q, 1.0)
        k = np.where(np.isfinite(k), k, 1.0)
        x = (q * k).astype(np.float32)
        exact = math.fsum(float(t) for t in x)
        total = float(np.abs(x.astype(np.float64)).sum())
        for order in (np.arange(n), rng.permutation(n), np.argsort(np.abs(x))):
            for tz in (False, True):
                err = abs(_f32_sum(x, order, tz) - exact)
                assert err <= gamma * total
                worst = max(worst, err / (gamma * total))
    assert worst > 0


def test_sum_error_factor_nearly_attained_by_truncation():
    # 1 followed by n - 1 terms just below one unit of 1.0 (2^-23): toward
    # zero, every addition drops almost a whole unit of the running sum
    n = 128
    x = np.full(n, np.float32(2.0 ** -23 * (1 - 2.0 ** -10)), dtype=np.float32)
    x[0] = np.float32(1.0)
    exact = math.fsum(float(t) for t in x)
    err = abs(_f32_sum(x, np.arange(n), True) - exact)
    gamma = f8.fp32_sum_error_factor(n)
    total = float(np.abs(x.astype(np.float64)).sum())
    assert err <= gamma * total
    assert err >= 0.99 * gamma * total   # so a factor half the size would fail


def test_flops_count():
    assert f8.fp8_flops(4, 4, 8, False) == 4 * 8 * 16
    assert f8.fp8_flops(4, 4, 8, True) == 4 * 8 * 10


# ---- planted mistakes -----------------------------------------------------------

MUTANTS = {
    "no_shift": ("p = np.where(vis, np.exp(s - m_use[:, None]), 0.0) * 2.0 ** P_SHIFT",
                 "p = np.where(vis, np.exp(s - m_use[:, None]), 0.0)"),
    "l_from_rounded": ("l = l * alpha + p.sum(axis=1)", "l = l * alpha + pr.sum(axis=1)"),
    "no_rescale": ("acc = acc * alpha[:, None] + pr @ v[b, h, keys]",
                   "acc = acc + pr @ v[b, h, keys]"),
    "ties_away": ("r = np.rint(a / spacing) * spacing",
                  "r = np.floor(a / spacing + 0.5) * spacing"),
    "lse_no_unshift": ("LSE[b, h] = m + np.log(l) - P_SHIFT * math.log(2.0)",
                       "LSE[b, h] = m + np.log(l)"),
}


def _mutant(kind):
    old, new = MUTANTS[kind]
    assert SRC.count(old) == 1, kind
    ns = {"__name__": f"fp8_mutant_{kind}"}
    exec(compile(SRC.replace(old, new), f"<mutant {kind}>", "exec"), ns)
    return ns


def _pins_pass(ns):
    try:
        q, k, v = fp8_case(14, 1, 2, 150, 200, 32, sigma=1.0)
        scale = 1 / math.sqrt(32)
        O, L = ns["attention_fp8_blocked"](q, k, v, True, scale, 64)
        Or, Lr = attention_ref(q, k, v, True, scale)
        bound = f8.fp8_error_bound(q, k, v, True, scale)
        if not ((np.abs(O - Or) <= bound + 1e-12).all() and np.abs(L - Lr).max() <= 1e-12):
            return False
        d = 2
        q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
        k = np.zeros((1, 1, 2, d)); k[0, 0, 1, 0] = math.log(17 / 32)
        v = np.array([[[[1.0, -2.0], [3.0, 5.0]]]])
        O, L = ns["attention_fp8_blocked"](q, k, v, False, 1.0, 2)
        want = (256 * v[0, 0, 0] + 128 * v[0, 0, 1]) / (256 + 136)
        if np.abs(O[0, 0, 0] - want).max() > 1e-13:
            return False
        x = np.linspace(0, 448, 100001).astype(np.float32)
        return bool(np.array_equal(ns["e4m3_round"](x), torch_e4m3(x)))
    except AssertionError:
        return False


def test_pins_pass_on_the_oracle():
    assert _pins_pass(vars(f8))


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_pins_reject_mutant(kind):
    assert not _pins_pass(_mutant(kind))
