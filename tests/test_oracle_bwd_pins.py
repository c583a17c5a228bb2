"""Pins of the backward oracle (oracle/attention_bwd_fp64.py) to things
other than itself: central finite differences of sum(dO * O) using the
forward oracle, torch's fp64 autograd through scaled_dot_product_attention,
the Delta identity of "第 08 章: Flash Attention——分块注意力"
(chuoer47.github.io), sections 6.2-6.3, closed forms and invariants.  Six
planted mistakes must each fail the pin set.
"""
import numpy as np
import pytest

import oracle.attention_bwd_fp64 as bwd_mod
from oracle import attention_ref
from oracle.attention_bwd_fp64 import (attention_bwd_ref, attention_bwd_sampled,
                                       backward_flops, delta_ref)
from tests.oracle_pin_checks import rng_qkv


def rng_do(seed, shape):
    return np.random.default_rng(2000 + seed).standard_normal(shape)


def finite_differences(q, k, v, do, causal, scale, h=1e-6):
    """Central differences of L = sum(dO * O(q, k, v)), O from the forward
    oracle, for every input element."""
    def loss(q_, k_, v_):
        O, _ = attention_ref(q_, k_, v_, causal, scale)
        return float((O * do).sum())
    grads = []
    for x_idx in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[x_idx])
        for idx in np.ndindex(g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[x_idx][idx] += h
            minus[x_idx][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def _fd_case(causal, Lq, Lk, d, seed):
    q, k, v = rng_qkv(seed, 1, 1, Lq, Lk, d)
    do = rng_do(seed, q.shape)
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk,d", [(4, 4, 3), (5, 3, 2), (3, 6, 2)])
def test_finite_differences(causal, Lq, Lk, d):
    q, k, v, do = _fd_case(causal, Lq, Lk, d, 50 + Lq)
    got = attention_bwd_ref(q, k, v, do, causal, 0.8)
    fd = finite_differences(q, k, v, do, causal, 0.8)
    for g, f, name in zip(got, fd, ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g, f, rtol=0, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Lq,Lk,d", [(2, 2, 37, 37, 16), (1, 3, 50, 70, 8), (1, 1, 64, 30, 32)])
def test_torch_autograd(causal, B, H, Lq, Lk, d):
    import torch
    import torch.nn.functional as F
    q, k, v = rng_qkv(51, B, H, Lq, Lk, d)
    do = rng_do(51, q.shape)
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(do))
    got = attention_bwd_ref(q, k, v, do, causal, scale)
    for g, t, name in zip(got, (tq, tk, tv), ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk,chunk", [(90, 90, 16), (70, 130, 1000), (130, 70, 7)])
def test_sampled_gradients_match_torch_autograd(causal, Lq, Lk, chunk):
    """The sampled form (for large L) against torch's fp64 autograd of
    scaled_dot_product_attention on a whole head, rows chosen at the edges
    and at random."""
    import torch
    import torch.nn.functional as F
    q, k, v = rng_qkv(52, 1, 1, Lq, Lk, 16)
    do = rng_do(52, q.shape)
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(Lk)[None, :] <= np.arange(Lq)[:, None])
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    out.backward(torch.from_numpy(do))
    qrows = np.array([0, 1, Lq // 2, Lq - 1, 17])
    krows = np.array([0, 5, Lk // 3, Lk - 1])
    dQ, dK, dV = attention_bwd_sampled(q[0, 0], k[0, 0], v[0, 0], do[0, 0], causal, scale,
                                       qrows, krows, chunk=chunk)
    np.testing.assert_allclose(dQ, tq.grad.numpy()[0, 0, qrows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy()[0, 0, krows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy()[0, 0, krows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_delta_identity(causal):
    """sum_j P_ij dP_ij = Delta_i = sum_d dO_id O_id (section 6.3, third step)."""
    q, k, v = rng_qkv(52, 1, 2, 40, 45, 8)
    do = rng_do(52, q.shape)
    O, _, P = attention_ref(q, k, v, causal, 0.5, return_p=True)
    dP = np.einsum("bhid,bhjd->bhij", do, v)
    np.testing.assert_allclose((P * dP).sum(-1), delta_ref(O, do), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_closed_form(causal):
    """scale 0: uniform P over the visible keys, so dS = 0 gives dQ = dK = 0
    and dV_j = sum over the rows i that see j of dO_i / |A_i|."""
    Lq, Lk = 9, 7
    q, k, v = rng_qkv(53, 1, 1, Lq, Lk, 3)
    do = rng_do(53, q.shape)
    dQ, dK, dV = attention_bwd_ref(q, k, v, do, causal, 0.0)
    assert not dQ.any() and not dK.any()
    want = np.zeros((Lk, 3))
    for i in range(Lq):
        js = [j for j in range(Lk) if not causal or j <= i]
        for j in js:
            want[j] += do[0, 0, i] / len(js)
    np.testing.assert_allclose(dV[0, 0], want, rtol=0, atol=1e-14)


def test_single_key_and_invariants():
    q, k, v = rng_qkv(54, 1, 2, 6, 1, 4)
    do = rng_do(54, q.shape)
    dQ, dK, dV = attention_bwd_ref(q, k, v, do, False, 0.7)
    assert not dQ.any() and not dK.any()             # P = 1, dS = 0
    np.testing.assert_allclose(dV[:, :, 0], do.sum(axis=2), rtol=0, atol=1e-14)
    # sum_j dS_ij = 0 for every row, hence sum_j dK_j = 0
    q, k, v = rng_qkv(55, 1, 2, 30, 40, 6)
    do = rng_do(55, q.shape)
    for causal in (False, True):
        _, dK, _ = attention_bwd_ref(q, k, v, do, causal, 0.6)
        np.testing.assert_allclose(dK.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    # causal with Lk > Lq: keys past the last query are never seen
    q, k, v = rng_qkv(56, 1, 1, 5, 9, 3)
    do = rng_do(56, q.shape)
    _, dK, dV = attention_bwd_ref(q, k, v, do, True, 0.6)
    assert not dK[0, 0, 5:].any() and not dV[0, 0, 5:].any()


def test_backward_flops_is_two_and_a_half_forward():
    from oracle import algorithmic_flops
    for causal in (False, True):
        assert backward_flops(300, 300, 64, causal) == \
            2.5 * algorithmic_flops(np.arange(300), 300, 64, causal)


# --- planted mistakes ----------------------------------------------------

def _mutant(kind):
    def ref(q, k, v, do, causal, scale):
        B, H, Lq, d = q.shape
        Lk = k.shape[2]
        dQ, dK, dV = np.empty_like(q), np.empty_like(k), np.empty_like(v)
        allowed = np.ones((Lq, Lk), dtype=bool)
        if causal and kind != "no_mask":
            allowed = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None]
        for b in range(B):
            for h in range(H):
                s = np.where(allowed, scale * (q[b, h] @ k[b, h].T), -np.inf)
                e = np.where(allowed, np.exp(s - s.max(1, keepdims=True)), 0.0)
                p = e / e.sum(1, keepdims=True)
                dV[b, h] = (p @ do[b, h][:Lk]) if kind == "dv_no_transpose" else p.T @ do[b, h]
                dp = do[b, h] @ v[b, h].T
                if kind == "no_rowsum":
                    ds = p * dp
                elif kind == "rowsum_sign":
                    ds = p * (dp + (p * dp).sum(1, keepdims=True))
                else:
                    ds = p * (dp - (p * dp).sum(1, keepdims=True))
                dQ[b, h] = scale * (ds @ k[b, h])
                dK[b, h] = (ds.T @ q[b, h]) if kind == "dk_no_scale" else scale * (ds.T @ q[b, h])
                if kind == "dq_from_v":
                    dQ[b, h] = scale * (ds @ v[b, h])
        return dQ, dK, dV
    return ref


MUTANTS = ["no_rowsum", "rowsum_sign", "dk_no_scale", "dq_from_v", "no_mask", "dv_no_transpose"]


def _pins_pass():
    try:
        for causal in (False, True):
            q, k, v, do = _fd_case(causal, 4, 4, 2, 60)
            got = bwd_mod.attention_bwd_ref(q, k, v, do, causal, 0.8)
            fd = finite_differences(q, k, v, do, causal, 0.8)
            for g, f in zip(got, fd):
                np.testing.assert_allclose(g, f, rtol=0, atol=2e-8)
    except (AssertionError, ValueError):
        return False
    return True


def test_unmutated_backward_passes_pins():
    assert _pins_pass()


@pytest.mark.parametrize("kind", MUTANTS)
def test_backward_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(bwd_mod, "attention_bwd_ref", _mutant(kind))
    assert not _pins_pass(), f"pins failed to catch backward mutant {kind!r}"
