"""Host-side arithmetic of bench.py (no GPU): algorithmic flops and bytes
against the measurement table's figures, the roofline bound each workload
gets, and the one-GPU guard."""
import math
import os

import pytest

import bench
from seeded_inputs import WORKLOADS


def test_flops_match_the_formula():
    # 4 B H Lq Lk d, halved for causal: 1.0995e12 for the 16K causal workload
    w = WORKLOADS["bf16_causal_16k_d128"]
    assert bench.flops_of(w, True) == 4.0 * 16 * 16384 * 16384 * 128 / 2
    assert math.isclose(bench.flops_of(w, True), 1.0995e12, rel_tol=1e-4)
    w = WORKLOADS["bf16_4k_d128"]
    assert bench.flops_of(w, False) == 2 * bench.flops_of(w, True)


def test_share_workload_is_an_eighth_of_the_bench_one():
    # one GPU's 2 of the bench workload's 16 heads; causal, split 4 ways
    w8, w = WORKLOADS["bf16_causal_16k_d128"], WORKLOADS["bf16_causal_16k_d128_2h"]
    assert bench.flops_of(w, True) * 8 == bench.flops_of(w8, True)
    assert (w.modes, w.splits) == (("splitkv", "causal"), 4)


@pytest.mark.parametrize("name,mb", [("bf16_causal_1k_d64", 33.8), ("bf16_4k_d128", 269.5),
                                     ("bf16_causal_16k_d128", 269.5),
                                     ("bf16_peaky_d256_ragged", 132.9)])
def test_compulsory_bytes(name, mb):
    # (2 B H Lq d + 2 B H Lk d) esize + 4 B H Lq
    w = WORKLOADS[name]
    want = (2 * w.B * w.H * w.Lq * w.d + 2 * w.B * w.H * w.Lk * w.d) * 2 + 4 * w.B * w.H * w.Lq
    assert bench.compulsory_bytes(w) == want
    assert round(want / 1e6, 1) == mb


def test_compulsory_bytes_fp8_and_backward():
    w = WORKLOADS["fp8_causal_16k_d128"]
    n = w.B * w.H * w.Lq * w.d
    # one-byte q, k, v in; bf16 o and fp32 LSE out
    assert bench.compulsory_bytes(w, fp8=True) == 3 * n + 2 * n + 4 * w.B * w.H * w.Lq
    w = WORKLOADS["bf16_causal_16k_d128"]
    # q, k, v, o, dO, LSE in; dq, dk, dv out
    assert bench.compulsory_bytes(w, backward=True) == 8 * n * 2 + 4 * w.B * w.H * w.Lq


def test_bound_by_intensity():
    # ridge = 2500 TFLOP/s / 8 TB/s = 312.5 flop/B: the 1K d=64 causal
    # workload (254 flop/B) is HBM-side, the others MFMA-side
    ridge = bench.PEAK_TFLOPS["bf16"] * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    w = WORKLOADS["bf16_causal_1k_d64"]
    assert bench.flops_of(w, True) / bench.compulsory_bytes(w) < ridge
    w = WORKLOADS["bf16_causal_16k_d128"]
    assert bench.flops_of(w, True) / bench.compulsory_bytes(w) > ridge


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _profile(tmp_path, name, fwd, bwd, fp8, nbytes=1.5e8):
    (tmp_path / name).write_text(
        f"# kernel_source_sha256_16: {fwd}\n# bwd_kernel_source_sha256_16: {bwd}\n"
        f"# fp8_kernel_source_sha256_16: {fp8}\nhbm_bytes_per_launch: {nbytes:.6e}\n")


def test_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """Committed counters count only while the hash of the kernel they were
    taken on matches the source; the backward's own hash alone decides for
    the backward, the FP8 kernel's for FP8."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    fwd = bench.kernel_source_hash()
    bwd = bench.kernel_source_hash(bench.BWD_KERNEL_SOURCE)
    fp8 = bench.kernel_source_hash(bench.FP8_KERNEL_SOURCE)
    stale = "0" * 16
    _profile(tmp_path, "fa_fwd_w_hbm_counters.txt", fwd, stale, stale)
    assert bench.traffic_from_profiles("w") == 1.5e8
    _profile(tmp_path, "fa_fwd_w_hbm_counters.txt", stale, bwd, fp8)
    assert bench.traffic_from_profiles("w") is None
    _profile(tmp_path, "fa_bwd_w_hbm_counters.txt", stale, bwd, stale)
    assert bench.traffic_from_profiles("w", backward=True) == 1.5e8
    _profile(tmp_path, "fa_bwd_w_hbm_counters.txt", fwd, stale, fp8)
    assert bench.traffic_from_profiles("w", backward=True) is None
    _profile(tmp_path, "fa_fwd_w8_hbm_counters.txt", stale, stale, fp8)
    assert bench.traffic_from_profiles("w8", fp8=True) == 1.5e8
    _profile(tmp_path, "fa_fwd_w8_hbm_counters.txt", fwd, bwd, stale)
    assert bench.traffic_from_profiles("w8", fp8=True) is None
    assert bench.traffic_from_profiles("absent") is None


def test_profile_lookup_prefers_the_mode(tmp_path, monkeypatch):
    """A summary named for the workload and mode is used for that mode; the
    one named for the workload alone serves the other modes.  The MFMA busy
    figure follows the same lookup and the same source hash."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    fwd = bench.kernel_source_hash()
    stale = "0" * 16
    _profile(tmp_path, "fa_fwd_w_hbm_counters.txt", fwd, stale, stale, nbytes=1.0e8)
    _profile(tmp_path, "fa_fwd_w_noncausal_hbm_counters.txt", fwd, stale, stale, nbytes=2.0e8)
    assert bench.traffic_from_profiles("w", mode="noncausal") == 2.0e8
    assert bench.traffic_from_profiles("w", mode="causal") == 1.0e8
    assert bench.traffic_from_profiles("w") == 1.0e8
    (tmp_path / "fa_fwd_w_causal_sq_counters.txt").write_text(
        f"# kernel_source_sha256_16: {fwd}\n"
        "MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles) = 0.611\n")
    assert bench.mfma_busy_from_profiles("w", mode="causal") == 0.611
    assert bench.mfma_busy_from_profiles("w", mode="noncausal") is None
    (tmp_path / "fa_fwd_w_causal_sq_counters.txt").write_text(
        f"# kernel_source_sha256_16: {stale}\n"
        "MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles) = 0.611\n")
    assert bench.mfma_busy_from_profiles("w", mode="causal") is None


def test_counters_in_run_sums_the_kernels_of_a_call(monkeypatch):
    """The in-run counter passes average each counter over each named
    kernel's dispatches and sum the averages over the kernels of one call;
    MFMA busy is busy cycles over 1024 SIMDs x kernel cycles (GRBM_GUI_ACTIVE
    summed over the 8 XCDs), HBM bytes are FETCH_SIZE and WRITE_SIZE KiB
    scaled by what they read for the copy of known size in the same call
    (here half and all of its bytes: factors 2 and 1).  rocprofv3 is
    replaced by a writer of its CSV."""
    import csv as _csv
    known = bench.CALIBRATION_MIB * 1024.0
    copy_reads = {"FETCH_SIZE": [known / 2, known / 2], "WRITE_SIZE": [known, known]}
    values = {  # per kernel: counter -> per-dispatch values
        "fa_a_kernel<1>": {"SQ_VALU_MFMA_BUSY_CYCLES": [1024 * 800.0, 1024 * 600.0],
                           "GRBM_GUI_ACTIVE": [8 * 1000.0, 8 * 1000.0],
                           "FETCH_SIZE": [100.0, 300.0], "WRITE_SIZE": [50.0, 50.0]},
        "fa_b_kernel<1>": {"SQ_VALU_MFMA_BUSY_CYCLES": [0.0],
                           "GRBM_GUI_ACTIVE": [8 * 1000.0],
                           "FETCH_SIZE": [10.0], "WRITE_SIZE": [5.0]},
        "other_kernel": {"SQ_VALU_MFMA_BUSY_CYCLES": [1e12], "GRBM_GUI_ACTIVE": [1.0],
                         "FETCH_SIZE": [1e9], "WRITE_SIZE": [1e9]},
    }

    def fake_run(cmd, **kw):
        d = cmd[cmd.index("-d") + 1]
        pmc = cmd[cmd.index("--pmc") + 1:cmd.index("--output-format")]
        with open(os.path.join(d, "c_counter_collection.csv"), "w", newline="") as f:
            wr = _csv.writer(f)
            wr.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            if "--copy-calibration" in cmd:
                for c in pmc:
                    # the fill that creates the copy's source is not counted
                    wr.writerow(["vectorized_elementwise_kernel<FillFunctor>", c, 3.0])
                    for x in copy_reads[c]:
                        wr.writerow(["__amd_rocclr_copyBuffer", c, x])
                return
            for kn, cv in values.items():
                for c in pmc:
                    for x in cv[c]:
                        wr.writerow([kn, c, x])

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/usr/bin/rocprofv3")
    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    r = bench.counters_in_run(["--workload", "w"], ["fa_a_kernel", "fa_b_kernel"])
    # busy: (700 + 0) x 1024 / (1024 x (1000 + 1000)) = 0.35
    assert r["mfma_busy"] == 0.35
    # bytes: ((200 + 10) x 2 + (50 + 5)) KiB
    assert r["hbm_bytes_per_launch"] == (210 * 2 + 55) * 1024
    assert r["kernels"] == ["fa_a_kernel", "fa_b_kernel"]
    # "&" joins substrings that must all occur: fa_a_kernel<2> is not <1>
    values["fa_a_kernel<2>"] = {k: [x * 9 for x in v] for k, v in values["fa_a_kernel<1>"].items()}
    r2 = bench.counters_in_run(["--workload", "w"], ["fa_a_kernel&<1>", "fa_b_kernel"])
    assert r2["mfma_busy"] == 0.35 and r2["hbm_bytes_per_launch"] == r["hbm_bytes_per_launch"]
    # a counter that reads 2/5 of the copied bytes is scaled by 2.5
    copy_reads["FETCH_SIZE"] = [known * 0.4]
    r3 = bench.counters_in_run(["--workload", "w"], ["fa_a_kernel&<1>", "fa_b_kernel"])
    assert r3["hbm_bytes_per_launch"] == pytest.approx((210 * 2.5 + 55) * 1024)
    assert r3["copy_calibration"]["fetch_scale"] == 2.5
    monkeypatch.setattr(bench.shutil, "which", lambda name: None)
    assert bench.counters_in_run(["--workload", "w"], ["fa_a_kernel"]) is None


def test_warm_up_counts(monkeypatch):
    """The warm-up runs exactly the launches asked for; by default at least
    MIN_WARMUP of them and at least WARMUP_S seconds' worth."""
    import time as _time
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []

    def launch():
        calls.append(1)
        _time.sleep(0.002)

    for n in (0, 1, 3, 7):
        calls.clear()
        done, per = bench.warm_up(launch, (), n)
        assert done == n == len(calls)
        assert (per is None) == (n <= 1)
    monkeypatch.setattr(bench, "WARMUP_S", 0.05)
    calls.clear()
    t0 = _time.perf_counter()
    done, per = bench.warm_up(launch, ())
    assert done == len(calls) >= bench.MIN_WARMUP
    assert _time.perf_counter() - t0 >= 0.05
    assert 0.0015 < per < 0.02

