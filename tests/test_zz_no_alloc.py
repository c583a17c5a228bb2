"""GPU check of fa_fwd_splitkv_noalloc, the key-split forward on the
library's fixed per-GPU scratch, through the C ABI: on two calls in a row
(the second on a smaller problem, over the scratch the first left behind)
its O and LSE equal those of fa_fwd_splitkv with a caller workspace bit for
bit, and match the fp64 oracle within the bf16 bars (O 2e-2, LSE 1e-3)."""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from oracle import attention_ref
from seeded_inputs import make_inputs, widen
from tests.gpu_helpers import GUARD, SENTINEL_BF16, say, to_device

pytestmark = pytest.mark.gpu


def f32_scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def _run(q, k, v, causal, scale, num_splits, noalloc):
    import torch
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    n_o, n_l = B * H * Lq * d, B * H * Lq
    obuf = torch.full((n_o + 2 * GUARD,), SENTINEL_BF16, dtype=torch.int16, device="cuda")
    lbuf = torch.full((n_l + 2 * GUARD,), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = obuf[GUARD:GUARD + n_o], lbuf[GUARD:GUARD + n_l]
    stream = torch.cuda.current_stream()
    if noalloc:
        fa.fa_fwd_splitkv_noalloc(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale,
                                  num_splits, stream)
    else:
        nbytes = fa.splitkv_workspace_size(B, H, Lq, d, num_splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        fa.fa_fwd_splitkv(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale,
                          num_splits, ws, nbytes, stream)
    torch.cuda.synchronize()
    ob = obuf.cpu().numpy().view(np.uint16)
    lb = lbuf.cpu().numpy()
    assert (ob[:GUARD] == SENTINEL_BF16).all() and (ob[-GUARD:] == SENTINEL_BF16).all()
    assert np.isnan(lb[:GUARD]).all() and np.isnan(lb[-GUARD:]).all()
    return ob[GUARD:-GUARD].reshape(B, H, Lq, d), lb[GUARD:-GUARD].reshape(B, H, Lq)


# (seed, B, H, Lq, Lk, d, causal, num_splits): the second is smaller than the
# first, so it runs over partials the first left in the scratch
CASES = [(81, 1, 4, 300, 5000, 128, False, 8), (82, 1, 2, 100, 700, 64, True, 3)]


def test_noalloc_matches_workspace_entry_point_twice():
    for seed, B, H, Lq, Lk, d, causal, ns in CASES:
        say(f"case noalloc seed={seed} B={B} H={H} Lq={Lq} Lk={Lk} d={d} causal={causal} "
            f"splits={ns}")
        assert fa.splitkv_workspace_size(B, H, Lq, d, ns) <= fa.noalloc_scratch_bytes()
        q, k, v = make_inputs(seed, B, H, Lq, Lk, d, "bf16")
        scale = f32_scale(d)
        O1, L1 = _run(q, k, v, causal, scale, ns, noalloc=True)
        O2, L2 = _run(q, k, v, causal, scale, ns, noalloc=False)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(L1, L2)
        O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), causal, scale)
        eo = float(np.abs(widen(O1) - O_ref).max())
        el = float(np.abs(L1.astype(np.float64) - L_ref).max())
        say(f"  max|dO| {eo:.3e} max|dLSE| {el:.3e}")
        assert eo <= 2e-2 and el <= 1e-3
