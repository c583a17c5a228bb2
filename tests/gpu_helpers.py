"""Helpers for the GPU tests: move seeded inputs to the device, call the C
ABI through the binding, bring results back, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import exact_io_aware_08_amd as fa
from seeded_inputs import widen

GUARD = 4096            # elements of canary before and after each output
SENTINEL_BF16 = 0x7FC1  # a NaN pattern the kernel never writes
SENTINEL_F32 = np.float32(np.nan)

# parity bars (stated per tensor, see the design notes)
BF16_O_ATOL = 2e-2
BF16_LSE_ATOL = 1e-3
F32_REL = 1e-5


def say(msg: str):
    print(msg, file=sys.stderr, flush=True)


def to_device(x: np.ndarray):
    import torch
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def run_fa(q, k, v, causal: bool, scale: float, stream=None, guard=True,
           window=None):
    """Run the HIP forward on storage arrays (uint16 bf16 bits or fp32).

    ``window``: (left, right) with -1 for no bound; calls fa_fwd_window
    (``causal`` is then ignored).  Outputs are allocated with GUARD canary
    elements on both sides; the canaries are checked after the call.
    Returns (O storage array, LSE float32 array)."""
    import torch
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    bf16 = q.dtype == np.uint16
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    n_o = B * H * Lq * d
    n_l = B * H * Lq
    g = GUARD if guard else 0
    if bf16:
        obuf = torch.full((n_o + 2 * g,), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda")
    else:
        obuf = torch.full((n_o + 2 * g,), float("nan"), dtype=torch.float32,
                          device="cuda")
    lbuf = torch.full((n_l + 2 * g,), float("nan"), dtype=torch.float32,
                      device="cuda")
    o = obuf[g:g + n_o]
    lse = lbuf[g:g + n_l]
    if stream is None:
        stream = torch.cuda.current_stream()
    if window is not None:
        fa.fa_fwd_window(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(window[0]),
                         int(window[1]), scale, stream)
    else:
        fn = fa.fa_fwd if bf16 else fa.fa_fwd_f32
        fn(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale, stream)
    torch.cuda.synchronize()
    ob = obuf.cpu().numpy()
    lb = lbuf.cpu().numpy()
    if g:
        if bf16:
            assert (ob[:g] == SENTINEL_BF16).all() and (ob[-g:] == SENTINEL_BF16).all(), \
                "O canary overwritten"
        else:
            assert np.isnan(ob[:g]).all() and np.isnan(ob[-g:]).all(), "O canary overwritten"
        assert np.isnan(lb[:g]).all() and np.isnan(lb[-g:]).all(), "LSE canary overwritten"
    O = ob[g:g + n_o].reshape(B, H, Lq, d)
    if bf16:
        O = O.view(np.uint16)
    LSE = lb[g:g + n_l].reshape(B, H, Lq)
    return O, LSE


def check_parity(O, LSE, O_ref, LSE_ref, dtype: str, label: str = ""):
    """Assert the stated bar; return the measured errors.  Rows the oracle
    leaves empty (LSE = -inf, O = 0: only sliding windows make them) must
    be exactly that on the GPU too; the bar applies to the other rows."""
    Og = widen(O)
    assert np.isfinite(Og).all(), f"{label}: non-finite O"
    empty = np.isneginf(LSE_ref)
    assert (np.isneginf(LSE) == empty).all(), f"{label}: empty rows differ"
    assert not Og[empty].any(), f"{label}: O of an empty row is not 0"
    LSE, LSE_ref = LSE[~empty], LSE_ref[~empty]
    assert np.isfinite(LSE).all(), f"{label}: non-finite LSE"
    eo = float(np.abs(Og - O_ref).max())
    el = float(np.abs(LSE.astype(np.float64) - LSE_ref).max()) if LSE.size else 0.0
    if dtype == "bf16":
        say(f"{label}: max|dO|={eo:.3e} (bar {BF16_O_ATOL}) "
            f"max|dLSE|={el:.3e} (bar {BF16_LSE_ATOL})")
        assert eo <= BF16_O_ATOL, f"{label}: O error {eo}"
        assert el <= BF16_LSE_ATOL, f"{label}: LSE error {el}"
        return eo, el
    ro = eo / float(np.abs(O_ref).max())
    rl = el / float(np.abs(LSE_ref).max())
    say(f"{label}: rel O {ro:.3e} rel LSE {rl:.3e} (bar {F32_REL})")
    assert ro <= F32_REL, f"{label}: O rel error {ro}"
    assert rl <= F32_REL, f"{label}: LSE rel error {rl}"
    return ro, rl
