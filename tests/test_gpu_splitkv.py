"""GPU parity of the key-split forward (fa_fwd_splitkv) against the fp64
oracle on identical seeded bf16 inputs.

The keys a query block visits are split among num_splits workgroups; each
writes its normalised fp32 partial (O_s, LSE_s) into the caller's
workspace, and a merge kernel combines them with the block-merge step of
"Flash Attention 原理与实现详解" (tbr8.org), section 2.1.  Checked: the final O
and LSE against the oracle (bf16 bars: 2e-2 on O, 1e-3 on LSE); each
partial against the oracle over that split's key range (fp32 partials, so
a tighter bar: 1e-2 on O, 1e-4 on LSE, where the only error left is the
bf16 rounding of P); untouched memory past the workspace size.
"""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from oracle import attention_ref
from seeded_inputs import WORKLOADS, make_inputs, widen, workload_inputs
from tests.gpu_helpers import check_parity, say, to_device

pytestmark = pytest.mark.gpu

GUARD_BYTES = 1 << 16


def f32_scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def run_split(q, k, v, causal, scale, splits):
    """Returns O (bf16 bits), LSE, opart [S,B*H,Lq,d], lpart [S,B*H,Lq]."""
    import torch
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device="cuda")
    need = fa.splitkv_workspace_size(B, H, Lq, d, splits)
    ws = torch.full((need + GUARD_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
    fa.fa_fwd_splitkv(qd, kd, vd, o, lse, B, H, Lq, Lk, d, int(causal), scale, splits,
                      ws, need, torch.cuda.current_stream())
    torch.cuda.synchronize()
    wb = ws.cpu().numpy()
    assert (wb[need:] == 0xA5).all(), "write past the workspace size"
    n_o = splits * B * H * Lq * d
    o_bytes = (n_o * 4 + 255) // 256 * 256
    opart = wb[:n_o * 4].view(np.float32).reshape(splits, B * H, Lq, d)
    lpart = wb[o_bytes:o_bytes + splits * B * H * Lq * 4].view(np.float32).reshape(splits, B * H, Lq)
    O = o.view(torch.int16).cpu().numpy().view(np.uint16)
    return O, lse.cpu().numpy(), opart, lpart


def split_ranges(Lq, Lk, causal, splits, d):
    """Key range [k0, k1) of split s for each query block (the library's
    division of a block's tiles: ceil(tiles / splits) tiles per split)."""
    BM, BN, _ = fa.tile_config("bf16", d)
    out = []
    for qb in range((Lq + BM - 1) // BM):
        q0 = qb * BM
        kv_end = min(Lk, q0 + BM) if causal else Lk
        nt = max((kv_end + BN - 1) // BN, 1)
        per = (nt + splits - 1) // splits
        rows = np.arange(q0, min(Lq, q0 + BM))
        for s in range(splits):
            js, je = s * per, min(nt, s * per + per)
            out.append((rows, s, (js * BN, min(Lk, je * BN)) if js < je else None))
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,Lq,Lk,splits", [(128, 300, 2000, 3), (128, 130, 1000, 8),
                                            (64, 257, 3000, 5), (256, 100, 900, 4),
                                            (128, 64, 700, 64), (128, 513, 513, 1)])
def test_splitkv_parity_and_partials(causal, d, Lq, Lk, splits):
    q, k, v = make_inputs(41, 1, 2, Lq, Lk, d, "bf16")
    s = f32_scale(d)
    label = f"splitkv S={splits} Lq={Lq} Lk={Lk} d={d} causal={causal}"
    say(f"case {label}")
    O, LSE, opart, lpart = run_split(q, k, v, causal, s, splits)
    qw, kw, vw = widen(q), widen(k), widen(v)
    O_ref, L_ref = attention_ref(qw, kw, vw, causal, s, workers=8)
    check_parity(O, LSE, O_ref, L_ref, "bf16", label)
    for rows, sp, keys in split_ranges(Lq, Lk, causal, splits, d):
        part_o = opart[sp].reshape(2, Lq, d)[:, rows]
        part_l = lpart[sp].reshape(2, Lq)[:, rows]
        if keys is None:
            assert np.isneginf(part_l).all() and not part_o.any(), (sp, "empty split")
            continue
        Po, Pl = attention_ref(qw, kw, vw, causal, s, rows=rows, keys=keys, workers=8)
        Po, Pl = Po[0], Pl[0]
        empty = np.isneginf(Pl)
        assert (np.isneginf(part_l) == empty).all(), (sp, keys)
        assert not part_o[empty].any()
        assert np.abs(part_o - Po).max() <= 1e-2, (sp, keys, np.abs(part_o - Po).max())
        assert np.abs(part_l[~empty] - Pl[~empty]).max(initial=0) <= 1e-4, (sp, keys)


def test_splitkv_matches_unsplit_kernel():
    """Same inputs through fa_fwd and fa_fwd_splitkv: both within the bars of
    the oracle, and within bf16 rounding of each other."""
    import torch
    q, k, v = make_inputs(42, 1, 4, 256, 4096, 128, "bf16")
    s = f32_scale(128)
    O1, L1, _, _ = run_split(q, k, v, False, s, 8)
    qd, kd, vd = to_device(q), to_device(k), to_device(v)
    o = torch.empty((1, 4, 256, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 4, 256), dtype=torch.float32, device="cuda")
    fa.fa_fwd(qd, kd, vd, o, lse, 1, 4, 256, 4096, 128, 0, s)
    torch.cuda.synchronize()
    O0 = o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.abs(widen(O1) - widen(O0)).max() <= 2e-2
    assert np.abs(L1 - lse.cpu().numpy()).max() <= 1e-4


def test_longkv_workload_full():
    """The bench's long-key workload (B=1, H=16, Lq=512, Lk=65536, d=128,
    8 splits) at full size, every row against the oracle."""
    w = WORKLOADS["bf16_longkv_512x64k_d128"]
    q, k, v = workload_inputs(w)
    say(f"case {w.name} (full size, all rows)")
    O, LSE, _, _ = run_split(q, k, v, False, w.scale, w.splits)
    O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), False, w.scale)
    check_parity(O, LSE, O_ref, L_ref, "bf16", w.name)


def test_causal_share_workload_full():
    """One GPU's share of the 16K causal workload (B=1, H=2, L=16384,
    d=128), split 4 ways as the bench runs it, every row against the
    oracle; on a 256-CU device fa_splitkv_suggest picks those 4 splits."""
    import torch
    w = WORKLOADS["bf16_causal_16k_d128_2h"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        assert fa.splitkv_suggest(w.B, w.H, w.Lq, w.Lk, w.d, True) == w.splits
    q, k, v = workload_inputs(w)
    say(f"case {w.name} (full size, all rows, {w.splits} causal splits)")
    O, LSE, _, _ = run_split(q, k, v, True, w.scale, w.splits)
    O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), True, w.scale)
    check_parity(O, LSE, O_ref, L_ref, "bf16", w.name)


def test_suggested_split_on_this_device():
    """fa_splitkv_suggest with the device's own CU count (num_cus = 0), then
    fa_fwd_splitkv with that many splits, against the oracle."""
    import torch
    B, H, Lq, Lk, d = 1, 2, 200, 6000, 128
    n = fa.splitkv_suggest(B, H, Lq, Lk, d, False)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"suggested splits {n} for {cus} CUs")
    assert n == fa.splitkv_suggest(B, H, Lq, Lk, d, False, cus) and 1 < n <= 64
    q, k, v = make_inputs(44, B, H, Lq, Lk, d, "bf16")
    s = f32_scale(d)
    O, L, _, _ = run_split(q, k, v, False, s, n)
    O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), False, s)
    check_parity(O, L, O_ref, L_ref, "bf16", f"suggested {n} splits")
