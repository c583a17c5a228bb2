"""GPU parity of the sliding-window forward (fa_fwd_window) against the fp64
oracle with the same (left, right) window, on identical seeded bf16 inputs.

The window is the (left, right) window-size pair of "Flash Attention 原理与
实现详解" (tbr8.org), section 6.3 "滑动窗口注意力": key j is visible to query i
iff i - left <= j <= i + right; -1 in the ABI (None in the oracle) leaves a
side unbounded.  Bars as for the other bf16 tests: max-abs error <= 2e-2 on
O and <= 1e-3 on LSE; rows with no visible key must read O = 0, LSE = -inf.
"""
import numpy as np
import pytest

from oracle import attention_ref
from seeded_inputs import WORKLOADS, make_inputs, widen, workload_inputs
from tests.gpu_helpers import check_parity, run_fa, say

pytestmark = pytest.mark.gpu


def f32_scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def oracle_window(left, right):
    return (None if left < 0 else left, None if right < 0 else right)


def window_case(seed, B, H, Lq, Lk, d, left, right, sigma_qk=1.0):
    q, k, v = make_inputs(seed, B, H, Lq, Lk, d, "bf16", sigma_qk=sigma_qk)
    scale = f32_scale(d)
    label = f"bf16 window ({left}, {right}) B={B} H={H} Lq={Lq} Lk={Lk} d={d}"
    say(f"case {label}")
    O, LSE = run_fa(q, k, v, False, scale, window=(left, right))
    O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), False, scale,
                                 window=oracle_window(left, right), workers=8)
    return check_parity(O, LSE, O_ref, L_ref, "bf16", label)


# causal windows (left, 0): left below, at and just past tile and block
# edges (tiles of 64 or 128 keys, blocks of 128 or 256 queries)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("left", [0, 1, 31, 63, 127, 128, 129, 300])
def test_causal_window(d, left):
    window_case(31, 1, 2, 600, 600, d, left, 0)


# two-sided bands and one-sided right windows
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("left,right", [(50, 70), (0, 200), (200, 0), (-1, 5),
                                        (7, -1), (0, 0), (1000, 1000)])
def test_band(d, left, right):
    window_case(32, 1, 2, 530, 530, d, left, right)


# Lq != Lk, including rows with no visible key (Lq > Lk - 1 + left)
@pytest.mark.parametrize("Lq,Lk,left,right", [(700, 400, 100, 0), (700, 400, 33, 50),
                                              (300, 900, 64, 0), (300, 900, 10, 400),
                                              (1000, 70, 5, -1)])
def test_ragged_and_empty_rows(Lq, Lk, left, right):
    window_case(33, 1, 2, Lq, Lk, 128, left, right)


def test_peaky_d256_window():
    window_case(34, 1, 2, 400, 460, 256, 90, 20, sigma_qk=3.0)


def test_window_zero_gives_v_rows_bitwise():
    """(0, 0): each query sees only its own key, P = 1 exactly, so O is the
    row of V bit for bit."""
    q, k, v = make_inputs(35, 1, 2, 300, 300, 128, "bf16")
    O, LSE = run_fa(q, k, v, False, f32_scale(128), window=(0, 0))
    np.testing.assert_array_equal(O, v)


def test_unbounded_windows_equal_causal_and_full_bitwise():
    """(-1, 0) and (-1, -1) take the causal and full kernels; a left bound
    past every key takes the window kernel and gives the same bits."""
    q, k, v = make_inputs(36, 1, 2, 333, 333, 128, "bf16")
    s = f32_scale(128)
    Oc, Lc = run_fa(q, k, v, True, s)
    for win in ((-1, 0), (400, 0), (5000, 0)):
        Ow, Lw = run_fa(q, k, v, False, s, window=win)
        np.testing.assert_array_equal(Ow, Oc)
        np.testing.assert_array_equal(Lw, Lc)
    Of, Lf = run_fa(q, k, v, False, s)
    Ow, Lw = run_fa(q, k, v, False, s, window=(-1, -1))
    np.testing.assert_array_equal(Ow, Of)
    np.testing.assert_array_equal(Lw, Lf)


def test_window_1k_16k_workload_full():
    """The bench's window workload at full size (B=1, H=16, L=16384, d=128,
    causal window of 1024 keys), every row against the oracle."""
    w = WORKLOADS["bf16_window1k_16k_d128"]
    q, k, v = workload_inputs(w)
    say(f"case {w.name} (full size, all rows)")
    O, LSE = run_fa(q, k, v, False, w.scale, window=w.window_abi)
    O_ref, L_ref = attention_ref(widen(q), widen(k), widen(v), False, w.scale,
                                 window=w.window, chunk=256)
    check_parity(O, LSE, O_ref, L_ref, "bf16", w.name)
