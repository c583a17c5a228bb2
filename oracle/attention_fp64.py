"""CPU oracle for the attention forward pass (test infrastructure only).

This is the plain, slow, fp64 definition of what the GPU path computes.  It
is NOT part of the product: only the test suite, the package smoke check and
the bench's CPU-baseline leg may import it, and nothing it computes ever
feeds the HIP path.  It shares no code with the HIP library or its binding.

What it computes, per batch b, head h and query row i (sources: the pages'
definition of scaled dot-product attention, "Flash Attention 原理与实现详解：
如何通过 IO-Aware 算法突破注意力机制的计算瓶颈" (tbr8.org), section 一
"注意力机制的计算瓶颈", Attention(Q,K,V) = softmax(QK^T/sqrt(d)) V; the
statement that the tiled method returns exactly this result, "從零開始用自定義
Triton 內核編寫 FlashAttention-2" (digipub.cc), section "核心方案——讓注意力具備
IO 感知能力"; the log-sum-exp output, "第 08 章: Flash Attention——分块注意力"
(chuoer47.github.io), section 3 "LSE"; the causal mask, same page, section 4
"因果掩码的分块遍历", lower triangle including the diagonal):

  1. s_ij  = scale * sum_d q_id k_jd                 (fp64, j < Lk)
  2. A_i   = {j < Lk}  (non-causal)  or  {j < Lk : j <= i}  (causal),
     intersected, for a sliding window (left, right), with
     {j : i - left <= j <= i + right} (either bound may be absent)
  3. m_i   = max_{j in A_i} s_ij ;  l_i = sum_{j in A_i} exp(s_ij - m_i)
  4. P_ij  = exp(s_ij - m_i) / l_i  for j in A_i, else 0
  5. O_i   = sum_j P_ij v_j
  6. LSE_i = m_i + ln(l_i)                           (natural log)

Subtracting m_i in step 3 is the safe-softmax form of the same quantity
("FlashAttention的Triton实现：IO-aware注意力机制底层原理", gitcode.csdn.net,
section "Safe Softmax 的数学推导"); it changes nothing mathematically.

The sliding window follows the pages' window-size pair (left, right) used
together with the causal flag ("Flash Attention 原理与实现详解" (tbr8.org),
section 6.3 "滑动窗口注意力", where (1024, 0) means 1024 keys to the left and
none to the right).

Readings where the pages are silent or disagree (each listed in the design
notes): LSE uses the natural log of the scaled scores; causal alignment is
top-left (key j visible to query i iff j <= i) for any Lq, Lk; masked keys
are excluded exactly (weight 0), not given a large negative score; keys at
or beyond Lk never take part; a window bound w admits keys at distance up to
and including w; a row left with no key (possible only with a left bound
and Lq > Lk) has O = 0 and LSE = -inf.

S and P are formed explicitly, one (b, h, row-chunk) at a time to bound
memory.  A thread pool over those chunks keeps BLAS at one thread per worker.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # optional: bound BLAS threads inside the pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


def _chunk_ref(q64, k64, v64, rows, causal, scale, want_p, window=None,
               keys=None):
    """One (b, h, row-chunk): q64 [R, d] rows at absolute indices ``rows``."""
    left, right = window if window is not None else (None, None)
    Lk = k64.shape[0]
    k_lo, k_hi = keys if keys is not None else (0, Lk)
    # columns that any row of this chunk may see
    hi = min(Lk, k_hi)
    if causal:
        hi = min(hi, int(rows.max()) + 1)
    if right is not None:
        hi = min(hi, int(rows.max()) + right + 1)
    lo = k_lo if left is None else max(k_lo, int(rows.min()) - left)
    hi = max(hi, lo)
    cols = np.arange(lo, hi)
    s = (q64 @ k64[lo:hi].T) * scale                         # step 1
    allowed = np.ones((len(rows), len(cols)), dtype=bool)    # step 2
    if causal:
        allowed &= cols[None, :] <= rows[:, None]
    if left is not None:
        allowed &= cols[None, :] >= rows[:, None] - left
    if right is not None:
        allowed &= cols[None, :] <= rows[:, None] + right
    s_masked = np.where(allowed, s, -np.inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        m = s_masked.max(axis=1, initial=-np.inf)            # step 3
        e = np.where(allowed, np.exp(s_masked - m[:, None]), 0.0)
        l = e.sum(axis=1)
        p = e / np.where(l > 0, l, 1.0)[:, None]             # step 4 (empty row: 0)
        o = p @ v64[lo:hi]                                   # step 5
        lse = m + np.log(l)                                  # step 6 (empty row: -inf)
    if want_p:
        full = np.zeros((len(rows), Lk))
        full[:, lo:hi] = p
        return o, lse, full
    return o, lse, None


def attention_ref(q, k, v, causal: bool, scale: float, *, rows=None,
                  return_p: bool = False, workers: int | None = None,
                  chunk: int = 512, window=None, keys=None):
    """fp64 attention forward.

    q: [B, H, Lq, d]; k, v: [B, H, Lk, d]; any real dtype (widened exactly
    to fp64 by the caller or here).  ``scale`` is used as given (pass the
    same fp32 value the GPU receives).  ``rows``: optional 1-D array of
    query indices to evaluate (each output row depends only on its own q row
    and on all of K, V, so a subset is the same definition).

    ``window``: optional (left, right) sliding window; each entry a
    non-negative int or None (no bound on that side).
    ``keys``: optional (k0, k1): only keys k0 <= j < k1 take part (the
    partial result of one key split; rows left empty read O = 0,
    LSE = -inf).

    Returns O [B, H, R, d] and LSE [B, H, R] in fp64 (R = Lq or len(rows)),
    plus P [B, H, R, Lk] when ``return_p``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, H, Lk, d) and v.shape == (B, H, Lk, d)
    assert Lk >= 1 and Lq >= 1
    scale = float(scale)
    if rows is None:
        rows = np.arange(Lq)
    rows = np.asarray(rows, dtype=np.int64)
    assert rows.ndim == 1 and (rows >= 0).all() and (rows < Lq).all()
    if window is not None:
        assert len(window) == 2 and all(w is None or int(w) >= 0 for w in window)
    R = len(rows)
    O = np.empty((B, H, R, d))
    LSE = np.empty((B, H, R))
    P = np.empty((B, H, R, Lk)) if return_p else None

    jobs = []
    for b in range(B):
        for h in range(H):
            for c0 in range(0, R, chunk):
                jobs.append((b, h, c0, min(R, c0 + chunk)))

    def run(job):
        b, h, c0, c1 = job
        r = rows[c0:c1]
        o, lse, p = _chunk_ref(q[b, h, r], k[b, h], v[b, h], r, causal,
                               scale, return_p, window, keys)
        O[b, h, c0:c1] = o
        LSE[b, h, c0:c1] = lse
        if return_p:
            P[b, h, c0:c1] = p

    if workers is None:
        workers = 1
    if workers <= 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        ctx = threadpool_limits(limits=1) if threadpool_limits else None
        try:
            if ctx is not None:
                ctx.__enter__()
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(run, jobs))
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
    if return_p:
        return O, LSE, P
    return O, LSE


def merge_partials(O_parts, LSE_parts):
    """Combine partial results over disjoint key sets into the result over
    their union: the block-merge step of "Flash Attention 原理与实现详解"
    (tbr8.org), section 2.1 "Tiling（分块计算）策略" -- with running max m,
    sum l and unnormalised output O, merging a block (m_b, l_b, O_b) gives
    m' = max(m, m_b), O' = O e^(m - m') + O_b e^(m_b - m'),
    l' = l e^(m - m') + l_b e^(m_b - m').  A normalised partial
    (O_s, LSE_s) is the state m = LSE_s, l = 1, O = O_s, so folding the
    partials in one after another and dividing by l at the end gives
    O = sum_s e^(LSE_s - LSE) O_s and LSE = m + ln l.

    O_parts [S, ..., d], LSE_parts [S, ...] (fp64).  Partials with
    LSE_s = -inf (no key of the set visible) contribute nothing; if every
    partial is empty the row is empty (O = 0, LSE = -inf).
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    m = np.full(LSE_parts.shape[1:], -np.inf)
    l = np.zeros(LSE_parts.shape[1:])
    O = np.zeros(O_parts.shape[1:])
    with np.errstate(invalid="ignore"):
        for O_b, m_b in zip(O_parts, LSE_parts):
            m_new = np.maximum(m, m_b)
            safe = np.where(np.isneginf(m_new), 0.0, m_new)
            a = np.exp(m - safe)        # 0 where m = -inf
            b = np.exp(m_b - safe)      # 0 where m_b = -inf
            O = O * a[..., None] + O_b * b[..., None]
            l = l * a + b
            m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(l[..., None] > 0, O / np.where(l > 0, l, 1.0)[..., None], 0.0)
        return O, m + np.log(l)


def default_workers() -> int:
    """Cores this process may use (the count the CPU baseline reports)."""
    try:
        return len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def algorithmic_flops(Lq_rows, Lk: int, d: int, causal: bool, window=None) -> float:
    """Matmul flops of the method for the given query rows of one head:
    4*d per visible (query, key) pair, the count used for TFLOP/s
    ("第 08 章" benchmark harness: 2 matmuls x 2 flops per MAC, halved for
    the causal mask at full size)."""
    rows = np.asarray(Lq_rows, dtype=np.int64)
    left, right = window if window is not None else (None, None)
    hi = np.full(rows.shape, Lk - 1)
    if causal:
        hi = np.minimum(hi, rows)
    if right is not None:
        hi = np.minimum(hi, rows + right)
    lo = np.zeros(rows.shape, dtype=np.int64)
    if left is not None:
        lo = np.maximum(lo, rows - left)
    vis = np.maximum(hi - lo + 1, 0)
    return float(4.0 * d * vis.sum())


__all__ = ["attention_ref", "merge_partials", "default_workers", "algorithmic_flops"]
