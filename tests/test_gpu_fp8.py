"""GPU parity of the FP8 (E4M3) forward, fa_fwd_fp8, through the C ABI.

Pass/fail is the exact fp64 definition on the dequantised inputs, element by
element, under a bound whose every term is derived on the CPU
(oracle/attention_fp8.py):

* |O - O_exact| <= bound + 2^-8 |O_exact| + 1e-4, with bound the worst case
  of rounding P (times 2^8) to E4M3 plus the effect of an error in S of at
  most S_ERR * scale * sum_t |q_t||k_t|; S_ERR = gamma_{d-1} for fp32
  additions in any order and rounding direction (fp32_sum_error_factor: the
  products of E4M3 values are exact, the accumulator is fp32); 2^-8 covers
  the bf16 output rounding with room for fp32;
* |LSE - LSE_exact| <= 1e-3 (LSE takes the unrounded P).

The blocked FP8 algorithm at a fixed 128-key block is computed beside it as
a diagnostic (printed, never asserted): its block size and rounding points
follow one tiling, not the definition.  The full-size workload is checked on
every row of two heads.
"""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from oracle import attention_fp8_blocked, attention_ref, fp8_error_bound
from oracle.attention_fp8 import FP8_DIAG_BLOCK, fp32_sum_error_factor
from seeded_inputs import WORKLOADS, make_inputs_fp8, round_to_bf16_bits, widen, widen_fp8
from tests.gpu_helpers import GUARD, SENTINEL_BF16, say

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3


def f32_scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def run_fp8(q8, k8, v8, ds, causal, scale):
    """fa_fwd_fp8 on E4M3 code arrays; returns (O as float64, LSE float32).
    The outputs carry canaries on both sides."""
    import torch
    B, H, Lq, d = q8.shape
    Lk = k8.shape[2]
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8))
    n_o, n_l = B * H * Lq * d, B * H * Lq
    obuf = torch.full((n_o + 2 * GUARD,), SENTINEL_BF16, dtype=torch.int16, device="cuda")
    lbuf = torch.full((n_l + 2 * GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = obuf[GUARD:GUARD + n_o], lbuf[GUARD:GUARD + n_l]
    fa.fa_fwd_fp8(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale, *ds,
                  torch.cuda.current_stream())
    torch.cuda.synchronize()
    ob = obuf.cpu().numpy().view(np.uint16)
    lb = lbuf.cpu().numpy()
    assert (ob[:GUARD] == SENTINEL_BF16).all() and (ob[-GUARD:] == SENTINEL_BF16).all()
    assert np.isnan(lb[:GUARD]).all() and np.isnan(lb[-GUARD:]).all()
    O = widen(ob[GUARD:-GUARD].reshape(B, H, Lq, d))
    L = lb[GUARD:-GUARD].reshape(B, H, Lq).astype(np.float64)
    return O, L


def check(O, L, q, k, v, causal, scale, label, rows=None):
    """The exact-definition bar on the (selected rows of the) GPU result O,
    L; the blocked algorithm alongside, reported only."""
    s_err = fp32_sum_error_factor(q.shape[-1])
    bound = fp8_error_bound(q, k, v, causal, scale, rows=rows, s_err=s_err)
    if rows is None:
        Oe, Le = attention_ref(q, k, v, causal, scale)
    else:
        Oe, Le = attention_ref(q, k, v, causal, scale, rows=rows)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    e_ex = np.abs(O - Oe)
    bar = bound + 2.0 ** -8 * np.abs(Oe) + 1e-4
    Ob, _ = attention_fp8_blocked(q, k, v, causal, scale, FP8_DIAG_BLOCK, rows=rows)
    say(f"{label}: max|O-O_exact| {e_ex.max():.3e} (worst ratio to bar {float((e_ex / bar).max()):.3f}); "
        f"max|LSE-LSE_exact| {np.abs(L - Le).max():.2e}; diagnostic: max|O-O_blocked128| "
        f"{np.abs(O - Ob).max():.3e}")
    assert (e_ex <= bar).all(), f"{label}: O outside the E4M3 error bound"
    assert np.abs(L - Le).max() <= LSE_ATOL, f"{label}: LSE"


def fp8_case(seed, B, H, Lq, Lk, d, causal, sigma=1.0):
    q8, k8, v8, ds = make_inputs_fp8(seed, B, H, Lq, Lk, d, sigma_qk=sigma)
    q, k, v = (widen_fp8(x, s) for x, s in zip((q8, k8, v8), ds))
    scale = f32_scale(d)
    label = f"fp8 B={B} H={H} Lq={Lq} Lk={Lk} d={d} causal={causal} sigma={sigma}"
    say(f"case {label}")
    O, L = run_fp8(q8, k8, v8, ds, causal, scale)
    check(O, L, q, k, v, causal, scale, label)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(300, 300), (257, 500), (500, 257), (130, 70), (64, 1000),
                                   (20, 45), (1, 33), (256, 256)])
def test_fp8_small(causal, Lq, Lk):
    fp8_case(71, 1, 2, Lq, Lk, 128, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_multihead_and_peaky(causal):
    fp8_case(72, 2, 4, 384, 384, 128, causal)
    fp8_case(73, 1, 2, 320, 256, 128, causal, sigma=3.0)


def test_fp8_2k_causal_all_rows():
    fp8_case(74, 1, 4, 2048, 2048, 128, True)


def test_fp8_16k_workload_two_heads_all_rows():
    """The FP8 bench workload (B=1, H=16, L=16384, d=128, causal) in the
    bench's launch configuration; every row of two heads against both
    oracles, in chunks of rows (each row depends only on its own q row)."""
    w = WORKLOADS["fp8_causal_16k_d128"]
    q8, k8, v8, ds = make_inputs_fp8(w.seed, w.B, w.H, w.Lq, w.Lk, w.d)
    O, L = run_fp8(q8, k8, v8, ds, True, w.scale)
    for h in (0, w.H - 1):
        sl = (slice(0, 1), slice(h, h + 1))
        q, k, v = (widen_fp8(x[sl], s) for x, s in zip((q8, k8, v8), ds))
        for r0 in range(0, w.Lq, 4096):
            rows = np.arange(r0, min(w.Lq, r0 + 4096))
            check(O[sl][:, :, rows], L[sl][:, :, rows], q, k, v, True, w.scale,
                  f"fp8 16k head {h} rows {r0}..{rows[-1]}", rows=rows)


@pytest.mark.parametrize("scale", [0.0, 1e-30])
def test_fp8_zero_scale_closed_form(scale):
    """scale = 0 (and a tiny one): every 2^8 P is 256 (no rounding), so O is
    the mean of the visible V rows and LSE = ln(count), up to the bf16
    output."""
    q8, k8, v8, ds = make_inputs_fp8(75, 1, 2, 200, 200, 128)
    v = widen_fp8(v8, ds[2])
    O, L = run_fp8(q8, k8, v8, ds, True, scale)
    want = np.cumsum(v, axis=2) / np.arange(1, 201)[None, None, :, None]
    assert np.abs(O - want).max() <= 2.0 ** -8 * np.abs(want).max() + 1e-4
    assert np.abs(L - np.log(np.arange(1, 201))[None, None, :]).max() <= 1e-5
    O, L = run_fp8(q8, k8, v8, ds, False, scale)
    want = v.mean(axis=2, keepdims=True)
    assert np.abs(O - want).max() <= 2.0 ** -8 * np.abs(want).max() + 1e-4
    assert np.abs(L - np.log(200)).max() <= 1e-5
