"""GPU parity of the backward (fa_bwd) against the fp64 backward oracle.

The GPU forward (fa_fwd) supplies O and LSE, as the backward expects; the
oracle differentiates the exact definition on the same bf16 inputs.  Bar
per gradient tensor: max|g - g_ref| <= 2e-2 * max|g_ref|.  It allows about
ten bf16 unit roundoffs (2^-9): P or dS rounded to bf16 before the second
product, Delta computed from the bf16 O, and the bf16 output.
"""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from oracle import attention_bwd_ref
from seeded_inputs import WORKLOADS, make_grad, make_inputs, widen
from tests.gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu

GRAD_REL = 2e-2
GUARD = 4096


def f32_scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def run_bwd(q, k, v, do, causal, scale):
    """fa_fwd then fa_bwd on the GPU; gradients as bf16 bit arrays.  The
    gradient buffers carry canaries on both sides."""
    import torch
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qd, kd, vd, dod = (to_device(x) for x in (q, k, v, do))
    o = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    fa.fa_fwd(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale, s)
    bufs = []
    for L in (Lq, Lk, Lk):
        n = B * H * L * d
        bufs.append(torch.full((n + 2 * GUARD,), 0x7FC1, dtype=torch.int16, device="cuda"))
    dq, dk, dv = (b[GUARD:-GUARD] for b in bufs)
    nbytes = fa.bwd_workspace_size(B, H, Lq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fa.fa_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, B, H, Lq, Lk, d, int(causal), scale,
              ws, nbytes, s)
    torch.cuda.synchronize()
    out = []
    for b, L in zip(bufs, (Lq, Lk, Lk)):
        a = b.cpu().numpy().view(np.uint16)
        assert (a[:GUARD] == 0x7FC1).all() and (a[-GUARD:] == 0x7FC1).all(), "canary overwritten"
        out.append(a[GUARD:-GUARD].reshape(B, H, L, d))
    return out


def check_grads(got, ref, label):
    for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
        gw = widen(g)
        assert np.isfinite(gw).all(), f"{label}: non-finite {name}"
        # an exactly zero gradient (a single visible key gives dS = 0) is held
        # to the bar of a unit-sized one: the GPU's dP - Delta is rounding
        # noise there
        scale = max(float(np.abs(r).max()), 1.0 if not np.abs(r).max() else 0.0)
        err = float(np.abs(gw - r).max())
        say(f"{label}: {name} max|err| {err:.3e} = {err / scale:.2e} x max|ref| (bar {GRAD_REL})")
        assert err <= GRAD_REL * scale, f"{label}: {name} error {err} vs max {scale}"


def bwd_case(seed, B, H, Lq, Lk, d, causal, sigma_qk=1.0):
    q, k, v = make_inputs(seed, B, H, Lq, Lk, d, "bf16", sigma_qk=sigma_qk)
    do = make_grad(seed, B, H, Lq, d)
    s = f32_scale(d)
    label = f"bwd B={B} H={H} Lq={Lq} Lk={Lk} d={d} causal={causal}"
    say(f"case {label}")
    got = run_bwd(q, k, v, do, causal, s)
    ref = attention_bwd_ref(widen(q), widen(k), widen(v), widen(do), causal, s)
    check_grads(got, ref, label)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk,d", [(128, 128, 64), (300, 300, 128), (257, 500, 128),
                                     (500, 257, 64), (130, 70, 128), (64, 1000, 128),
                                     (20, 45, 128), (1, 33, 64)])
def test_bwd_small(causal, Lq, Lk, d):
    bwd_case(61, 1, 2, Lq, Lk, d, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_multihead_and_peaky(causal):
    bwd_case(62, 2, 4, 384, 384, 128, causal)
    bwd_case(63, 1, 2, 256, 320, 64, causal, sigma_qk=2.0)


def test_bwd_4k_causal_d128():
    """A longer causal case: B=1, H=4, L=4096, d=128 (every tile kind, many
    query and key blocks per workgroup), all rows."""
    bwd_case(64, 1, 4, 4096, 4096, 128, True)


def test_bwd_16k_workload_two_heads_full():
    """The backward bench workload (B=1, H=16, L=16384, d=128, causal) in the
    bench's launch configuration; dQ, dK, dV of two whole heads (every row)
    against the fp64 backward oracle."""
    w = WORKLOADS["bf16_causal_16k_d128"]
    q, k, v = make_inputs(w.seed, w.B, w.H, w.Lq, w.Lk, w.d, "bf16")
    do = make_grad(w.seed, w.B, w.H, w.Lq, w.d)
    say(f"case bwd 16k workload B={w.B} H={w.H} L={w.Lq} d={w.d} causal")
    dq, dk, dv = run_bwd(q, k, v, do, True, w.scale)
    for h in (0, w.H - 1):
        sl = (slice(0, 1), slice(h, h + 1))
        ref = attention_bwd_ref(widen(q[sl]), widen(k[sl]), widen(v[sl]), widen(do[sl]),
                                True, w.scale)
        check_grads((dq[sl], dk[sl], dv[sl]), ref, f"bwd 16k head {h}")


def test_bwd_scale_tiny_gives_zero_dq_dk():
    """Scale -> 0: P uniform over the visible keys, dS -> 0, so dQ and dK
    vanish (below bf16 resolution of their scale-free size) and dV_j is the
    mean of dO over the rows that see key j."""
    q, k, v = make_inputs(65, 1, 2, 200, 200, 64, "bf16")
    do = make_grad(65, 1, 2, 200, 64)
    dq, dk, dv = run_bwd(q, k, v, do, True, 1e-30)
    assert np.abs(widen(dq)).max() < 1e-20 and np.abs(widen(dk)).max() < 1e-20
    dow = widen(do)[0]
    want = np.zeros_like(dow)
    for i in range(200):
        want[:, :i + 1] += dow[:, i:i + 1] / (i + 1)
    assert np.abs(widen(dv)[0] - want).max() <= GRAD_REL * np.abs(want).max()
