"""GPU parity over seeded sweeps of shapes for the other entry points: the
key-split forward (fa_fwd_splitkv, with its fp32 partials), the backward
(fa_bwd) and the FP8 forward (fa_fwd_fp8), each under the bars of its own
test file (the same comparison helpers), against the oracles.

Shapes are drawn once from fixed seeds (listed in the test ids): ragged
Lq and Lk, one or several heads, both masks, and for the key split any
count from 1 to 16 (more splits than a block has tiles included).
"""
import numpy as np
import pytest

from tests.test_gpu_bwd import bwd_case
from tests.test_gpu_fp8 import fp8_case
from tests.test_gpu_splitkv import test_splitkv_parity_and_partials as splitkv_case

pytestmark = pytest.mark.gpu


def _draw(seed, n, dims, budget):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(rng.choice(dims))
        causal = bool(rng.integers(2))
        Lq = int(rng.integers(1, 900))
        Lk = Lq if (causal and rng.random() < 0.5) else int(rng.integers(1, 2500))
        if 2 * Lq * Lk * d > budget:
            continue
        out.append((Lq, Lk, d, causal, int(rng.integers(1, 17))))
    return out


SPLIT_CASES = _draw(71, 12, [64, 128, 256], 6e8)
BWD_CASES = _draw(72, 10, [64, 128], 2e8)
FP8_CASES = _draw(73, 10, [128], 6e8)


def _id(c, with_splits=False):
    Lq, Lk, d, causal, s = c
    return f"{Lq}x{Lk}-d{d}-{'c' if causal else 'nc'}" + (f"-s{s}" if with_splits else "")


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[_id(c, True) for c in SPLIT_CASES])
def test_splitkv_sweep(case):
    Lq, Lk, d, causal, splits = case
    splitkv_case(causal, d, Lq, Lk, splits)


@pytest.mark.parametrize("case", BWD_CASES, ids=[_id(c) for c in BWD_CASES])
def test_bwd_sweep(case):
    Lq, Lk, d, causal, _ = case
    bwd_case(200 + BWD_CASES.index(case), 1, 2, Lq, Lk, d, causal)


@pytest.mark.parametrize("case", FP8_CASES, ids=[_id(c) for c in FP8_CASES])
def test_fp8_sweep(case):
    Lq, Lk, d, causal, _ = case
    fp8_case(300 + FP8_CASES.index(case), 1, 2, Lq, Lk, d, causal)
