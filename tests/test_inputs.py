"""The seeded input generator: bf16 rounding and reproducibility."""
import numpy as np
import torch

from seeded_inputs import (WORKLOADS, bf16_bits_to_f32, draw, make_inputs,
                           round_to_bf16_bits, widen)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # ties and near-ties: values exactly halfway between bf16 neighbours
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
    ])
    ours = round_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours.view(np.int16), theirs)
    # widening is exact
    back = bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(
        back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draw_is_reproducible_and_ordered():
    q1, k1, v1 = draw(7, 1, 2, 5, 6, 4)
    q2, k2, v2 = draw(7, 1, 2, 5, 6, 4)
    np.testing.assert_array_equal(q1, q2)
    rng = np.random.default_rng(7)
    np.testing.assert_array_equal(q1, rng.standard_normal((1, 2, 5, 4), dtype=np.float32))
    np.testing.assert_array_equal(k1, rng.standard_normal((1, 2, 6, 4), dtype=np.float32))
    np.testing.assert_array_equal(v1, rng.standard_normal((1, 2, 6, 4), dtype=np.float32))


def test_sigma_and_widen():
    q, k, v = make_inputs(5, 1, 1, 64, 64, 8, "bf16", sigma_qk=3.0)
    qf, kf, vf = draw(5, 1, 1, 64, 64, 8, sigma_qk=3.0)
    np.testing.assert_array_equal(widen(q), torch.from_numpy(qf).to(torch.bfloat16).double().numpy())
    assert widen(v).dtype == np.float64
    assert abs(np.std(qf) - 3.0) < 0.5 and abs(np.std(vf) - 1.0) < 0.2


def test_workload_table():
    assert sorted(w.seed for w in WORKLOADS.values()) == list(range(1, 10))
    w = WORKLOADS["fp8_causal_16k_d128"]
    assert (w.dtype, w.B, w.H, w.Lq, w.Lk, w.d, w.modes) == ("fp8", 1, 16, 16384, 16384, 128, ("causal",))
    assert WORKLOADS["bf16_longkv_512x64k_d128"].splits == 8
    w = WORKLOADS["bf16_window1k_16k_d128"]
    assert w.window == (1024, 0) and w.window_abi == (1024, 0) and w.modes == ("window",)
    w = WORKLOADS["bf16_peaky_d256_ragged"]
    assert (w.Lq, w.Lk, w.d, w.sigma_qk) == (8000, 8192, 256, 3.0)
    assert np.float32(WORKLOADS["bf16_4k_d128"].scale) == np.float32(1 / np.sqrt(np.float32(128)))


def test_fp8_inputs_follow_the_bf16_draw():
    """The FP8 inputs quantise the same Gaussian draw, per tensor."""
    from seeded_inputs import make_inputs_fp8, widen_fp8
    q8, k8, v8, (qd, kd, vd) = make_inputs_fp8(9, 1, 2, 50, 60, 16)
    qf, kf, vf = draw(9, 1, 2, 50, 60, 16)
    for c, ds, x in ((q8, qd, qf), (k8, kd, kf), (v8, vd, vf)):
        assert c.dtype == np.uint8 and c.shape == x.shape
        assert ds == np.float32(np.abs(x).max() / 448.0)
        y = widen_fp8(c, ds)
        assert np.abs(y - x).max() <= 2.0 ** -4 * np.abs(x).max()
