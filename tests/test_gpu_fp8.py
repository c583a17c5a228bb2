"""GPU parity of the FP8 (E4M3) forward, fa_fwd_fp8, through the C ABI.

The matrix unit's FP8 product does not accumulate S in full fp32: on random
E4M3 operands, two chained 32x32x64 products (the kernel's 128-deep S) are
off by at most 1.44e-5 of sum_t |q_t k_t| (8192 dot products measured on
the GPU), so the bars below take |S error| <= S_ERR * scale * sum_t |q_t||k_t|
with S_ERR = 2^-13, eight times that.  Two oracles, two bars (derivations in
oracle/attention_fp8.py):

* against the exact fp64 definition on the dequantised inputs, element by
  element: |O - O_exact| <= bound + 2^-8 |O_exact| + 1e-4, with bound the
  derived worst case of rounding P to E4M3 plus the S error, and 2^-8
  covering the bf16 output rounding with room for fp32; |LSE - LSE_exact|
  <= 1e-3 (LSE takes the unrounded P);
* against the blocked FP8 algorithm at the kernel's key-tile size, element
  by element: |O - O_blk| <= 2^-8 |O_blk| + 1e-5 + allowance (half a bf16
  step of the output, fp32 slack, and the allowance: one E4M3 spacing for
  each P that the S error could move across a rounding midpoint plus the
  continuous effect of the S error); and, with O_blk rounded to bf16 like
  the kernel's output, RMS(O - O_blk16) <= 3e-3 RMS(O_blk).
The full-size workload is checked on every row of two heads.
"""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from oracle import attention_fp8_blocked, attention_ref, fp8_error_bound
from seeded_inputs import WORKLOADS, make_inputs_fp8, round_to_bf16_bits, widen, widen_fp8
from tests.gpu_helpers import GUARD, SENTINEL_BF16, say

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3
S_ERR = 2.0 ** -13
BLK_RMS = 3e-3


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
    """Both bars on the (selected rows of the) GPU result O, L."""
    block = fa.tile_config("fp8", q.shape[-1])[1]
    Ob, Lb, allow = attention_fp8_blocked(q, k, v, causal, scale, block, rows=rows, s_err=S_ERR)
    bound = fp8_error_bound(q, k, v, causal, scale, rows=rows, s_err=S_ERR)
    if rows is None:
        Oe, Le = attention_ref(q, k, v, causal, scale)
    else:
        Oe, Le = attention_ref(q, k, v, causal, scale, rows=rows)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{label}: non-finite output"
    e_ex = np.abs(O - Oe)
    bar = bound + 2.0 ** -8 * np.abs(Oe) + 1e-4
    e_blk = np.abs(O - Ob)
    bar_blk = 2.0 ** -8 * np.abs(Ob) + 1e-5 + allow
    Ob16 = widen(round_to_bf16_bits(Ob.astype(np.float32)))
    rms = float(np.sqrt(((O - Ob16) ** 2).mean()) / np.sqrt((Ob ** 2).mean()))
    say(f"{label}: max|O-O_exact| {e_ex.max():.3e} (worst ratio to bar {float((e_ex / bar).max()):.3f}); "
        f"vs blocked: max {e_blk.max():.3e} (worst ratio to bar {float((e_blk / bar_blk).max()):.3f}), "
        f"rms ratio {rms:.2e}; max|LSE-LSE_exact| {np.abs(L - Le).max():.2e}")
    assert (e_ex <= bar).all(), f"{label}: O outside the E4M3 error bound"
    assert np.abs(L - Le).max() <= LSE_ATOL, f"{label}: LSE"
    assert (e_blk <= bar_blk).all() and rms <= BLK_RMS, f"{label}: O vs the blocked FP8 algorithm"


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


def test_fp8_scale_tiny_closed_form():
    """scale -> 0: every 2^8 P is 256 (no rounding), so O is the mean of the
    visible V rows and LSE = ln(count), up to the bf16 output."""
    q8, k8, v8, ds = make_inputs_fp8(75, 1, 2, 200, 200, 128)
    O, L = run_fp8(q8, k8, v8, ds, True, 1e-30)
    v = widen_fp8(v8, ds[2])
    want = np.cumsum(v, axis=2) / np.arange(1, 201)[None, None, :, None]
    assert np.abs(O - want).max() <= 2.0 ** -8 * np.abs(want).max() + 1e-4
    assert np.abs(L - np.log(np.arange(1, 201))[None, None, :]).max() <= 1e-5
