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
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
P_SHIFT = 8   # P is rounded as P * 2^8


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


def attention_fp8_blocked(q, k, v, causal: bool, scale: float, block: int,
                          round_p: bool = True):
    """The tiled online softmax with P rounded to E4M3 (see module doc).

    q [B,H,Lq,d], k, v [B,H,Lk,d]: the dequantised float64 values.  Keys are
    visited in blocks of `block`, in ascending order; a block with no visible
    key for a row changes nothing for it.  round_p=False skips the rounding
    (then the result is the exact definition, up to fp64 rounding).
    Returns O [B,H,Lq,d], LSE [B,H,Lq] (natural log)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    O = np.zeros((B, H, Lq, d))
    LSE = np.zeros((B, H, Lq))
    rows = np.arange(Lq)
    for b in range(B):
        for h in range(H):
            m = np.full(Lq, -np.inf)          # running max of s (natural units)
            l = np.zeros(Lq)                  # running sum of unrounded 2^8 P
            acc = np.zeros((Lq, d))           # running sum of rounded 2^8 P times V
            for j0 in range(0, Lk, block):
                keys = np.arange(j0, min(j0 + block, Lk))
                s = scale * (q[b, h] @ k[b, h, keys].T)
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
                m = m_new
            O[b, h] = acc / l[:, None]
            LSE[b, h] = m + np.log(l) - P_SHIFT * math.log(2.0)
    return O, LSE


def fp8_error_bound(q, k, v, causal: bool, scale: float):
    """Per-element bound on |O_fp8 - O_exact| from rounding P to E4M3 (see
    module doc); fp64, shape of O.  Output rounding is not included."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    out = np.zeros((B, H, Lq, d))
    rows = np.arange(Lq)
    keys = np.arange(Lk)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            vis = _causal_visible(rows, keys) if causal else np.ones(s.shape, bool)
            s = np.where(vis, s, -np.inf)
            p = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            av = np.abs(v[b, h])
            out[b, h] = 2.0 ** -4 * (p / l) @ av + 2.0 ** -18 * (vis.astype(np.float64) @ av) / l
    return out


def fp8_flops(Lq: int, Lk: int, d: int, causal: bool) -> float:
    """Matmul flops of one head's FP8 forward: 4 d per visible pair, as the
    bf16 forward."""
    rows = np.arange(Lq, dtype=np.int64)
    vis = np.minimum(rows + 1, Lk) if causal else np.full(Lq, Lk)
    return float(4.0 * d * vis.sum())


__all__ = ["e4m3_round", "attention_fp8_blocked", "fp8_error_bound", "fp8_flops",
           "E4M3_MAX", "P_SHIFT"]
