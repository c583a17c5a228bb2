"""Maximum-size case: a key range whose K and V tensors exceed 2^31 bytes
per head, so the last tiles sit past any 32-bit byte offset.

Lk = 2^24 + 37 keys at d = 64 (2.1 GB each for K and V).  K is zero except
one key near the end (the "needle", a multiple of query 0), so every score
is 0 except s_i = scale q_i . k_needle, and the definition of attention
(softmax over the keys, then the weighted mean of V) has a closed form per
row:

    O_i   = (e^{s_i} v_needle + sum_{j != needle} v_j) / (e^{s_i} + Lk - 1)
    LSE_i = ln(e^{s_i} + Lk - 1)

computed here in float64 from the same bf16 values the GPU sees (V drawn on
the CPU in chunks, its sum taken there).  Checked through fa_fwd and through
fa_fwd_splitkv, to the bf16 bars (2e-2 on O, 1e-3 on LSE).
"""
import math

import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from seeded_inputs import round_to_bf16_bits, widen
from tests.gpu_helpers import BF16_LSE_ATOL, BF16_O_ATOL, say

pytestmark = pytest.mark.gpu

D = 64
LQ = 40
LK = (1 << 24) + 37
NEEDLE = LK - 5
SCALE = 0.125            # 1/sqrt(64), exact
CHUNK = 1 << 20


@pytest.fixture(scope="module")
def long_inputs():
    import torch
    assert LK * D * 2 > (1 << 31)
    rng = np.random.default_rng(91)
    q = round_to_bf16_bits(rng.standard_normal((LQ, D), dtype=np.float32))
    k_needle = round_to_bf16_bits(widen(q[0]).astype(np.float32) * np.float32(4.0))
    v_dev = torch.empty((LK, D), dtype=torch.int16, device="cuda")
    v_sum = np.zeros(D)
    v_needle = None
    for r0 in range(0, LK, CHUNK):
        r1 = min(LK, r0 + CHUNK)
        vb = round_to_bf16_bits(rng.standard_normal((r1 - r0, D), dtype=np.float32))
        v_sum += widen(vb).sum(axis=0)
        if r0 <= NEEDLE < r1:
            v_needle = widen(vb[NEEDLE - r0])
        v_dev[r0:r1] = torch.from_numpy(vb.view(np.int16)).cuda()
    k_dev = torch.zeros((LK, D), dtype=torch.int16, device="cuda")
    k_dev[NEEDLE] = torch.from_numpy(k_needle.view(np.int16)).cuda()
    q_dev = torch.from_numpy(q.view(np.int16)).cuda()
    # closed form per row, in float64
    s = SCALE * (widen(q) @ widen(k_needle))                 # [LQ]
    m = np.maximum(s, 0.0)
    w = np.exp(s - m)
    rest = (LK - 1) * np.exp(-m)
    z = w + rest
    o_exact = (w[:, None] * v_needle + np.exp(-m)[:, None] * (v_sum - v_needle)) / z[:, None]
    lse_exact = m + np.log(z)
    say(f"long keys: Lk={LK}, {LK * D * 2 / 2**30:.2f} GiB per tensor; needle scores "
        f"{s.min():.2f}..{s.max():.2f}")
    yield q_dev, k_dev, v_dev, o_exact, lse_exact
    del q_dev, k_dev, v_dev
    torch.cuda.empty_cache()


def _check(o, lse, o_exact, lse_exact, label):
    import torch
    torch.cuda.synchronize()
    O = widen(o.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(LQ, D)
    L = lse.cpu().numpy().astype(np.float64).reshape(LQ)
    eo, el = np.abs(O - o_exact).max(), np.abs(L - lse_exact).max()
    say(f"{label}: max|O-O_exact| {eo:.3e}, max|LSE-LSE_exact| {el:.3e} "
        f"(ln Lk = {math.log(LK):.4f})")
    assert np.isfinite(O).all() and np.isfinite(L).all()
    assert eo <= BF16_O_ATOL and el <= BF16_LSE_ATOL, label


def test_long_keys_past_2gib_fa_fwd(long_inputs):
    import torch
    q, k, v, o_exact, lse_exact = long_inputs
    o = torch.empty((LQ, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((LQ,), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, 1, 1, LQ, LK, D, 0, SCALE, torch.cuda.current_stream())
    _check(o, lse, o_exact, lse_exact, "fa_fwd")


def test_long_keys_past_2gib_splitkv(long_inputs):
    import torch
    q, k, v, o_exact, lse_exact = long_inputs
    o = torch.empty((LQ, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((LQ,), dtype=torch.float32, device="cuda")
    splits = 64
    nbytes = fa.splitkv_workspace_size(1, 1, LQ, D, splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fa.fa_fwd_splitkv(q, k, v, o, lse, 1, 1, LQ, LK, D, 0, SCALE, splits, ws, nbytes,
                      torch.cuda.current_stream())
    _check(o, lse, o_exact, lse_exact, "fa_fwd_splitkv, 64 splits")
