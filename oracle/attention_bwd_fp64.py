"""CPU oracle for the attention backward pass (test infrastructure only).

Like the forward oracle, this is NOT part of the product: only the test
suite, the package smoke check and the bench's CPU-baseline leg may import
it.  It shares no code with the HIP library or its binding.

Given Q, K, V and the upstream gradient dO of O = softmax(scale Q K^T) V
(same allowed set A_i as the forward: all keys, or j <= i when causal), it
returns dQ, dK, dV in fp64, following the derivation of "第 08 章: Flash
Attention——分块注意力" (chuoer47.github.io), section 6 "反向":

  P_ij  = softmax over j in A_i of s_ij,  s_ij = scale q_i . k_j   (6.1)
  dV    = P^T dO                                                    (6.4)
  dP    = dO V^T                                                    (6.4)
  dS_ij = P_ij (dP_ij - sum_b P_ib dP_ib)     softmax backward      (6.3)
  dQ    = scale dS K,   dK = scale dS^T Q     S = scale Q K^T       (6.4)

The row sum in dS is written out as the plain softmax Jacobian requires;
the pages replace it by Delta_i = sum_d dO_id O_id (6.2-6.3), an identity
the tests check separately.  The pages' base-2 factor ln 2 (6.3) belongs to
their base-2 logits; with natural-exp logits, as here, it does not appear.
S and P are formed explicitly, one (b, h) at a time.
"""
from __future__ import annotations

import numpy as np


def attention_bwd_ref(q, k, v, do, causal: bool, scale: float):
    """fp64 gradients of sum(dO * O) with respect to Q, K, V.

    q, do: [B, H, Lq, d]; k, v: [B, H, Lk, d].  Returns dQ, dK, dV with the
    shapes of q, k, v.  Rows with no visible key cannot occur (the causal
    mask is top-left, so key 0 is always visible)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    assert k.shape == (B, H, Lk, d) and v.shape == (B, H, Lk, d) and do.shape == q.shape
    scale = float(scale)
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    allowed = np.ones((Lq, Lk), dtype=bool)
    if causal:
        allowed = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None]
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)                    # 6.1
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.where(allowed, np.exp(s - m), 0.0)
            p = e / e.sum(axis=1, keepdims=True)
            dV[b, h] = p.T @ do[b, h]                            # 6.4
            dp = do[b, h] @ v[b, h].T                            # 6.4
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # 6.3
            dQ[b, h] = scale * (ds @ k[b, h])                    # 6.4
            dK[b, h] = scale * (ds.T @ q[b, h])
    return dQ, dK, dV


def attention_bwd_sampled(q, k, v, do, causal: bool, scale: float, qrows, krows,
                          chunk: int = 1024):
    """The same gradients for a sample, one (b, h) slice: q, do [Lq, d], k, v
    [Lk, d].  Returns dQ for the query rows qrows and dK, dV for the key rows
    krows, in fp64.

    Written out from the same definition for large L: every row's softmax
    statistics come first (m_i and l_i over all visible keys, chunk by chunk,
    so LSE_i = m_i + ln l_i), then Delta_i = sum_j P_ij dP_ij for every row;
    then for a sampled query row i, dS_i. = P_i. (dP_i. - Delta_i) over all
    keys, dQ_i = scale dS_i. K, and for a sampled key j, over all queries,
    dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij q_i, with P_ij =
    exp(s_ij - LSE_i)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    Lq, d = q.shape
    Lk = k.shape[0]
    scale = float(scale)
    keys = np.arange(Lk)
    qrows = np.asarray(qrows, dtype=np.int64)
    krows = np.asarray(krows, dtype=np.int64)

    def block(i0, i1):
        rows = np.arange(i0, i1)
        s = scale * (q[i0:i1] @ k.T)
        vis = keys[None, :] <= rows[:, None] if causal else np.ones(s.shape, bool)
        return np.where(vis, s, -np.inf), vis

    lse = np.empty(Lq)
    delta = np.empty(Lq)
    for i0 in range(0, Lq, chunk):
        i1 = min(Lq, i0 + chunk)
        s, vis = block(i0, i1)
        m = s.max(axis=1, keepdims=True)
        e = np.where(vis, np.exp(s - m), 0.0)
        l = e.sum(axis=1, keepdims=True)
        lse[i0:i1] = (m + np.log(l))[:, 0]
        p = e / l
        dp = do[i0:i1] @ v.T
        delta[i0:i1] = (p * dp).sum(axis=1)
    dQ = np.empty((len(qrows), d))
    for n, i in enumerate(qrows):
        s, vis = block(i, i + 1)
        p = np.where(vis, np.exp(s - lse[i]), 0.0)[0]
        dp = v @ do[i]
        dQ[n] = scale * ((p * (dp - delta[i])) @ k)
    dK = np.zeros((len(krows), d))
    dV = np.zeros((len(krows), d))
    kk, vk = k[krows], v[krows]
    for i0 in range(0, Lq, chunk):
        i1 = min(Lq, i0 + chunk)
        rows = np.arange(i0, i1)
        s = scale * (q[i0:i1] @ kk.T)
        vis = krows[None, :] <= rows[:, None] if causal else np.ones(s.shape, bool)
        p = np.where(vis, np.exp(s - lse[i0:i1, None]), 0.0)
        dp = do[i0:i1] @ vk.T
        ds = p * (dp - delta[i0:i1, None])
        dV += p.T @ do[i0:i1]
        dK += scale * (ds.T @ q[i0:i1])
    return dQ, dK, dV


def delta_ref(o, do):
    """Delta_i = sum_d dO_id O_id (section 6.2's preprocess quantity)."""
    return (np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum(axis=-1)


def backward_flops(Lq: int, Lk: int, d: int, causal: bool) -> float:
    """Matmul flops of the backward for one head: five products of 2*d
    flops per visible (query, key) pair (S recomputed, dV, dP, dQ, dK),
    i.e. 2.5 times the forward's 4*d (the pages' benchmark harness counts
    the backward as 2.5 forward passes)."""
    rows = np.arange(Lq, dtype=np.int64)
    vis = np.minimum(rows + 1, Lk) if causal else np.full(Lq, Lk)
    return float(10.0 * d * vis.sum())


__all__ = ["attention_bwd_ref", "attention_bwd_sampled", "delta_ref", "backward_flops"]
