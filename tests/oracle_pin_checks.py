"""Independent evaluations used to pin the CPU oracle (test helpers).

None of these functions is the oracle and none is used by the HIP path:

* ``brute_force``: the definition softmax(scale*Q K^T) V evaluated with
  pure-Python loops, ``math.exp`` without any max subtraction and
  ``math.fsum``; the plain statement of scaled dot-product attention
  ("Flash Attention 原理与实现详解" (tbr8.org), section 一).
* ``online_blocked``: the per-tile online-softmax update the tiled method
  runs, in fp64 and natural-exp form, in the order the pages give it
  ("第 08 章: Flash Attention——分块注意力" (chuoer47.github.io), section 2
  "在线 softmax", steps 1-7 and the final division; the same update in
  "從零開始用自定義 Triton 內核編寫 FlashAttention-2" (digipub.cc), section
  "部分分數計算和在線更新").  Agreement with the oracle for every block size
  shows that the recurrence reaches the definition.
* ``golden_cases``: parser for the hand-worked fixture under tests/golden.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def rng_qkv(seed, B, H, Lq, Lk, d, sigma=1.0):
    rng = np.random.default_rng(1000 + seed)
    q = rng.standard_normal((B, H, Lq, d)) * sigma
    k = rng.standard_normal((B, H, Lk, d)) * sigma
    v = rng.standard_normal((B, H, Lk, d))
    return q, k, v


def visible(i, j, causal, window):
    """Key j visible to query i: top-left causal mask and an optional
    (left, right) window, either side None for unbounded."""
    left, right = window if window is not None else (None, None)
    if causal and j > i:
        return False
    if left is not None and j < i - left:
        return False
    if right is not None and j > i + right:
        return False
    return True


def brute_force(q, k, v, causal, scale, window=None):
    """q [Lq,d], k,v [Lk,d] -> O [Lq,d], LSE [Lq] with pure-Python loops.
    A row with no visible key gets O = 0 and LSE = -inf."""
    Lq, d = q.shape
    Lk = k.shape[0]
    O = np.zeros((Lq, d))
    L = np.zeros(Lq)
    for i in range(Lq):
        js = [j for j in range(Lk) if visible(i, j, causal, window)]
        if not js:
            L[i] = -math.inf
            continue
        w = []
        for j in js:
            s = scale * math.fsum(float(q[i, t]) * float(k[j, t])
                                  for t in range(d))
            w.append(math.exp(s))
        Z = math.fsum(w)
        for t in range(d):
            O[i, t] = math.fsum(w[n] * float(v[j, t])
                                for n, j in enumerate(js)) / Z
        L[i] = math.log(Z)
    return O, L


def online_blocked(q, k, v, causal, scale, block, window=None):
    """Stream K/V in tiles of ``block`` keys with the online-softmax update.

    State per query row: running max M, running sum L, unnormalised output
    O.  Per tile: M_new = max(M, rowmax S); P = exp(S - M_new);
    alpha = exp(M - M_new); L = L*alpha + rowsum P; O = O*alpha + P V;
    M = M_new.  After the last tile: O / L and LSE = M + log L.
    """
    Lq, d = q.shape
    Lk = k.shape[0]
    M = np.full(Lq, -np.inf)
    L = np.zeros(Lq)
    O = np.zeros((Lq, d))
    rows = np.arange(Lq)[:, None]
    for j0 in range(0, Lk, block):
        j1 = min(Lk, j0 + block)
        S = (q @ k[j0:j1].T) * scale
        cols = np.arange(j0, j1)[None, :]
        if causal:
            S = np.where(cols <= rows, S, -np.inf)
        if window is not None and window[0] is not None:
            S = np.where(cols >= rows - window[0], S, -np.inf)
        if window is not None and window[1] is not None:
            S = np.where(cols <= rows + window[1], S, -np.inf)
        M_new = np.maximum(M, S.max(axis=1))
        safe = np.where(np.isneginf(M_new), 0.0, M_new)   # fully masked rows
        P = np.exp(S - safe[:, None])
        alpha = np.exp(M - safe)
        L = L * alpha + P.sum(axis=1)
        O = O * alpha[:, None] + P @ v[j0:j1]
        M = M_new
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(L[:, None] > 0, O / np.where(L > 0, L, 1.0)[:, None], 0.0), M + np.log(L)


def _parse_value(tok: str) -> float:
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(Fraction(tok[3:-1]))
    return float(Fraction(tok))


def golden_cases(path):
    """Parse the hand-worked fixture into arrays (see its header)."""
    lines = [ln.split("#", 1)[0].strip() for ln in open(path, encoding="utf-8")]
    lines = [ln for ln in lines if ln]
    out = {}
    i = 0
    while i < len(lines):
        parts = lines[i].split()
        if parts[0] == "scale":
            out["scale"] = float(parts[1])
            i += 1
        elif parts[0] in ("q", "k", "v"):
            n, d = int(parts[1]), int(parts[2])
            out[parts[0]] = np.array([[float(x) for x in lines[i + 1 + r].split()]
                                      for r in range(n)])
            assert out[parts[0]].shape == (n, d)
            i += 1 + n
        elif parts[0] == "expect":
            key = f"{parts[1]} {parts[2]}"
            i += 1
            rows = []
            while i < len(lines) and lines[i].split()[0] not in (
                    "expect", "scale", "q", "k", "v"):
                rows.append([_parse_value(t) for t in lines[i].split()])
                i += 1
            arr = np.array(rows)
            out[key] = arr[:, 0] if arr.shape[1] == 1 else arr
        else:
            raise ValueError(f"bad fixture line: {lines[i]!r}")
    return out
