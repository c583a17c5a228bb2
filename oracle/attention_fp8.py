"""CPU oracle for the FP8 attention forward (test infrastructure only).

Not part of the product: only the tests, the package smoke check and the
bench's CPU-baseline leg may import it.  It shares no code with the HIP
library or its binding.

The pages name an FP8 variant of the method ("Flash Attention 原理与实现详解"
(tbr8.org), section 4.3 "FP8 支持": FP8 matrix units for more throughput)
and warn that it loses more precision than the exact bf16/fp32 forms, to be
judged per task (same page, section 6.1 "精度问题"); they give no scaling or
rounding recipe.  The reading used here (each point is listed in the design
notes):

  * Q, K, V arrive as OCP FP8 E4M3 codes with one fp32 descale factor per
    tensor; the values they stand for are decode(code) * descale.  S = scale
    Q K^T is formed from those values (products of E4M3 values are exact).
  * The second product takes P in E4M3 as well: P is multiplied by 2^8
    before rounding (round to nearest even), so values down to 2^-14 of the
    row maximum stay in E4M3's normal range; the factor cancels between the
    numerator and the row sum l, which is accumulated from the unrounded P.
  * O is the normalised result, LSE the natural log of sum_j exp(s_ij), as
    in the bf16 path.

Two functions pin such a kernel from two sides:

  attention_fp8_blocked  the pages' tiled online softmax ("Flash Attention
      原理与实现详解" (tbr8.org), section 2.1 "Tiling（分块计算）策略": per
      key block, a new running max, rescale of l and O by exp(m - m_new),
      then l += rowsum P, O += P V) with P rounded to E4M3 as above, in
      fp64.  The block size is the kernel's key tile: the rounding depends
      on the running max at the block where a key is seen, so this matches
      a kernel up to fp32 arithmetic.
  fp8_error_bound        a per-element bound on |O_fp8 - O| against the exact
      definition (the fp64 oracle on the dequantised inputs), whatever the
      block order: each rounded P_j (in units of the row max) is off by at
      most 2^-4 P_j (normal range) or 2^-18 (below it), so
          |O_fp8 - O|_id <= 2^-4 sum_j P_ij |v_jd| + 2^-18 sum_j |v_jd| / l_i
      with P_ij = p_j / l_i the exact softmax weights.

Both take an optional bound on the error of S itself, s_err: |s~_ij - s_ij|
<= s_err * scale * sum_t |q_it| |k_jt|.  Its value comes from a stated model
of the matrix unit, not from measuring it: each product of two E4M3 values
is exact in fp32 (at most 8 significant bits, exponents within range), and
the d products of a score are added in some order, each addition rounded to
fp32's 24-bit significand in some direction (the accumulator format the
instruction names; round-to-nearest is not assumed).  Any such sum is
within gamma_{d-1} sum_t |q_t k_t| of the exact one, gamma_k = k u / (1 - k
u) with u = 2^-23 (fp32_sum_error_factor: the recursive-summation bound of
N. J. Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed.,
section 4.2, with the unit roundoff of directed rounding).  With D_i = max_j of that bound,
every p_j moves by a factor within e^(+-D_i) (its score and the max both
move), which adds (e^(2 D_i) - 1)(sum_j P_ij |v_jd| + |O_id|) to the bound
and scales its rounding terms by e^(2 D_i); the blocked algorithm then also
returns an allowance: that continuous term plus, for every P whose 2^8
multiple lies within that relative window of an E4M3 rounding midpoint,
one E4M3 spacing of it (it may round the other way), carried through the
rescaling and normalisation like O itself.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
P_SHIFT = 8   # P is rounded as P * 2^8
# unit roundoff of fp32 (24-bit significand) under any rounding direction
FP32_DIRECTED_U = 2.0 ** -23
# key-block size of the blocked algorithm when it serves as a diagnostic
# beside the exact definition (a fixed choice, 128 keys; pass/fail never
# depends on it)
FP8_DIAG_BLOCK = 128


def fp32_sum_error_factor(n: int) -> float:
    """gamma_{n-1} = (n - 1) u / (1 - (n - 1) u), u = 2^-23: any fp32 sum of n
    terms, in any order, every addition rounded in any direction, lies
    within gamma_{n-1} sum_i |x_i| of the exact sum (Higham, "Accuracy and
    Stability of Numerical Algorithms", 2nd ed., section 4.2)."""
    k = n - 1
    return k * FP32_DIRECTED_U / (1.0 - k * FP32_DIRECTED_U)


def e4m3_round(x):
    """Round to the nearest OCP FP8 E4M3 value, ties to even; |x| <= 448.

    Written from the format: 3 mantissa bits, so a normal value in
    [2^e, 2^(e+1)) (e >= -6) has spacing 2^(e-3); below 2^-6 the spacing is
    the subnormal 2^-9.  np.rint rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.isfinite(a).all() and (a <= E4M3_MAX).all()
    _, e2 = np.frexp(a)                      # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, -6)               # binade exponent, floored at the subnormals
    spacing = np.ldexp(1.0, e - 3)
    r = np.rint(a / spacing) * spacing
    return np.copysign(r, x)


def _causal_visible(rows, keys):
    return keys[None, :] <= rows[:, None]


def _e4m3_midpoint_gap(x):
    """For x >= 0 (<= 448): distance to the nearest E4M3 rounding midpoint,
    and the E4M3 spacing at x (the change of a flipped rounding)."""
    _, e2 = np.frexp(x)
    e = np.maximum(e2 - 1, -6)
    spacing = np.ldexp(1.0, e - 3)
    frac = x / spacing - np.floor(x / spacing)
    return np.abs(frac - 0.5) * spacing, spacing


def attention_fp8_blocked(q, k, v, causal: bool, scale: float, block: int,
                          round_p: bool = True, rows=None, s_err=None, s_noise=None):
    """The tiled online softmax with P rounded to E4M3 (see module doc).

    q [B,H,Lq,d], k, v [B,H,Lk,d]: the dequantised float64 values.  Keys are
    visited in blocks of `block`, in ascending order; a block with no visible
    key for a row changes nothing for it.  round_p=False skips the rounding
    (then the result is the exact definition, up to fp64 rounding).  rows:
    optional query indexes to evaluate (default all).  s_err: also return the
    per-element allowance for an S error bounded as in the module doc.
    s_noise: optional [B,H,R,Lk] additions to s (natural units), to test that
    allowance.
    Returns O [B,H,R,d], LSE [B,H,R] (natural log) for the R rows, and the
    allowance [B,H,R,d] when s_err is given."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    R = len(rows)
    O = np.zeros((B, H, R, d))
    LSE = np.zeros((B, H, R))
    ALLOW = np.zeros((B, H, R, d)) if s_err is not None else None
    for b in range(B):
        for h in range(H):
            qr = q[b, h, rows]
            m = np.full(R, -np.inf)           # running max of s (natural units)
            l = np.zeros(R)                   # running sum of unrounded 2^8 P
            acc = np.zeros((R, d))            # running sum of rounded 2^8 P times V
            flip = np.zeros((R, d))           # running sum of possible flips times |V|
            if s_err is not None:
                sabs = s_err * abs(scale) * (np.abs(qr) @ np.abs(k[b, h]).T)
            for j0 in range(0, Lk, block):
                keys = np.arange(j0, min(j0 + block, Lk))
                s = scale * (qr @ k[b, h, keys].T)
                if s_noise is not None:
                    s = s + s_noise[b, h][:, keys]
                vis = _causal_visible(rows, keys) if causal else np.ones(s.shape, bool)
                s = np.where(vis, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)     # rows that have seen a key
                m_use = np.where(live, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - m_use), 0.0)
                p = np.where(vis, np.exp(s - m_use[:, None]), 0.0) * 2.0 ** P_SHIFT
                pr = e4m3_round(p) if round_p else p
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + pr @ v[b, h, keys]
                if s_err is not None:
                    # a relative window of e^(2 D) - 1 around each 2^8 P, plus
                    # fp32 slack for the exponent argument and exp2
                    win = np.expm1(2.0 * sabs.max(axis=1, keepdims=True)) + 2.0 ** -19
                    gap, spacing = _e4m3_midpoint_gap(p)
                    near = vis & (gap <= p * win)
                    flip = flip * alpha[:, None] + np.where(near, spacing, 0.0) @ np.abs(v[b, h, keys])
                m = m_new
            O[b, h] = acc / l[:, None]
            LSE[b, h] = m + np.log(l) - P_SHIFT * math.log(2.0)
            if s_err is not None:
                Dm = sabs.max(axis=1)[:, None]
                pw = np.abs(pr_weights(qr, k[b, h], v[b, h], rows, causal, scale))
                ALLOW[b, h] = flip / l[:, None] + np.expm1(2.0 * Dm) * (pw + np.abs(O[b, h]))
    if s_err is not None:
        return O, LSE, ALLOW
    return O, LSE


def pr_weights(qr, k, v, rows, causal, scale):
    """sum_j P_ij |v_jd| with the exact softmax weights of the given rows."""
    Lk = k.shape[0]
    s = scale * (qr @ k.T)
    vis = _causal_visible(rows, np.arange(Lk)) if causal else np.ones(s.shape, bool)
    s = np.where(vis, s, -np.inf)
    p = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
    return (p / p.sum(axis=1, keepdims=True)) @ np.abs(v)


def fp8_error_bound(q, k, v, causal: bool, scale: float, rows=None, s_err: float = 0.0):
    """Per-element bound on |O_fp8 - O_exact| from rounding P to E4M3, and
    from an S error bounded by s_err (see module doc); fp64, shape of O (of
    the selected rows).  Output rounding is not included."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    out = np.zeros((B, H, len(rows), d))
    keys = np.arange(Lk)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h, rows] @ k[b, h].T)
            vis = _causal_visible(rows, keys) if causal else np.ones(s.shape, bool)
            s = np.where(vis, s, -np.inf)
            p = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            av = np.abs(v[b, h])
            pw = (p / l) @ av
            g = np.exp(2.0 * s_err * abs(scale) * (np.abs(q[b, h, rows]) @ np.abs(k[b, h]).T).max(
                axis=1, keepdims=True))
            O = (p / l) @ v[b, h]
            out[b, h] = (g * (2.0 ** -4 * pw + 2.0 ** -18 * (vis.astype(np.float64) @ av) / l)
                         + (g - 1.0) * (pw + np.abs(O)))
    return out


def fp8_flops(Lq: int, Lk: int, d: int, causal: bool) -> float:
    """Matmul flops of one head's FP8 forward: 4 d per visible pair, as the
    bf16 forward."""
    rows = np.arange(Lq, dtype=np.int64)
    vis = np.minimum(rows + 1, Lk) if causal else np.full(Lq, Lk)
    return float(4.0 * d * vis.sum())


__all__ = ["e4m3_round", "attention_fp8_blocked", "fp8_error_bound", "fp8_flops",
           "fp32_sum_error_factor", "E4M3_MAX", "P_SHIFT", "FP32_DIRECTED_U", "FP8_DIAG_BLOCK"]
