"""Benchmark of the MI355X FlashAttention-2 forward (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward pass (one ``fa_fwd`` launch) over the whole workload
with Q, K, V already resident in HBM.  W untimed steps, then exactly K timed
steps bracketed by device synchronisation; rank 0 prints one JSON line.
Without the flags, W covers at least 0.2 s and K at least 0.1 s of launches
(and at least 5 and 50 of them): the shader clock settles under a
continuous load only after some tens of milliseconds.

Throughput counts the two matmuls only: 4*B*H*Lq*Lk*d flops, halved for
causal ("第 08 章: Flash Attention——分块注意力" (chuoer47.github.io), its
benchmark harness).  The roofline object prices that against MI355X's dense
bf16 MFMA peak (2.5 PFLOP/s).  The CPU baseline times the fp64 oracle on a
bounded sample of the same workload (whole heads) on this host's cores; it
is a reported baseline only.

``--workload fp8_causal_16k_d128`` runs the FP8 (E4M3) forward, fa_fwd_fp8,
priced against the dense FP8 MFMA peak (5.0 PFLOP/s); its CPU baseline is
the fp64 oracle on the dequantised inputs.

The roofline object also carries the peak derived from this device (compute
units x 4096 bf16 flops per clock x the maximum shader clock), the MFMA
utilisation and HBM bytes of the committed rocprofv3 summaries (while their
kernel-source hash matches), and, with ``--counters``, the same two figures
from rocprofv3 passes over this bench in child processes.  The exit status
is 1 when the result on the CPU sample is outside the parity bars.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import re
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, causal & non-causal) and % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3, "fp8": 5000.0}   # MI355X dense MFMA / fp32
DEFAULT_WORKLOAD = "bf16_causal_16k_d128"
KERNEL_SOURCE = os.path.join(ROOT, "exact_io_aware_08_amd", "csrc",
                             "fa_fwd_kernel.hip")
BWD_KERNEL_SOURCE = os.path.join(ROOT, "exact_io_aware_08_amd", "csrc",
                                 "fa_bwd_kernel.hip")
FP8_KERNEL_SOURCE = os.path.join(ROOT, "exact_io_aware_08_amd", "csrc",
                                 "fa_fp8_kernel.hip")
SHARED_DEVICE_HEADER = os.path.join(ROOT, "exact_io_aware_08_amd", "csrc", "fa_device.h")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(path: str = None) -> str:
    """Hash of a kernel source (default: the forward's) and the device
    header every kernel source includes (fa_device.h), with comments and
    whitespace removed, so that counters stay attached to the code they
    were taken on and survive edits that cannot change it."""
    text = open(path or KERNEL_SOURCE).read() + open(SHARED_DEVICE_HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def profile_path(kind: str, workload: str, mode: str | None, backward: bool):
    """The committed summary of `kind` (hbm_counters, sq_counters) for this
    workload: the one named for the workload and mode if present, else the
    one named for the workload; None if neither exists."""
    pre = os.path.join(PROFILES, f"fa_{'bwd' if backward else 'fwd'}_{workload}")
    for path in ([f"{pre}_{mode}_{kind}.txt"] if mode else []) + [f"{pre}_{kind}.txt"]:
        if os.path.exists(path):
            return path
    return None


def traffic_from_profiles(workload: str, backward: bool = False, fp8: bool = False,
                          mode: str | None = None):
    """HBM bytes per call from the committed rocprofv3 counter summary for
    this workload and pass, or None if absent or taken on a different
    kernel source."""
    path = profile_path("hbm_counters", workload, mode, backward)
    if path is None:
        return None
    text = open(path).read()
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if fp8:
        h3 = re.search(r"fp8_kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        if not t or not h3 or h3.group(1) != kernel_source_hash(FP8_KERNEL_SOURCE):
            return None
        return float(t.group(1))
    if backward:
        # the counters cover the backward's own kernels only (the forward
        # that supplies O and LSE runs outside the timed region)
        h2 = re.search(r"bwd_kernel_source_sha256_16:\s*([0-9a-f]+)", text)
        if not t or not h2 or h2.group(1) != kernel_source_hash(BWD_KERNEL_SOURCE):
            return None
        return float(t.group(1))
    h = re.search(r"(?<![a-z0-9_])kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def mfma_busy_from_profiles(workload: str, backward: bool = False, fp8: bool = False,
                            mode: str | None = None):
    """MFMA busy per SIMD (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x kernel
    cycles) from the committed rocprofv3 SQ summary of this workload and
    pass, or None if absent or taken on a different kernel source."""
    path = profile_path("sq_counters", workload, mode, backward)
    if path is None:
        return None
    text = open(path).read()
    b = re.search(r"MFMA busy per SIMD:[^=]*=\s*([0-9.]+)", text)
    src = FP8_KERNEL_SOURCE if fp8 else BWD_KERNEL_SOURCE if backward else None
    key = "fp8_kernel_source_sha256_16" if fp8 else \
        "bwd_kernel_source_sha256_16" if backward else "kernel_source_sha256_16"
    h = re.search(r"(?<![a-z0-9_])" + key + r":\s*([0-9a-f]+)", text)
    if not b or not h or h.group(1) != kernel_source_hash(src):
        return None
    return float(b.group(1))


def device_peak(cus: int):
    """The bf16 dense MFMA peak derived from this device: compute units x
    4096 flops per clock x the maximum shader clock (hipDeviceGetAttribute,
    hipDeviceAttributeClockRate, in kHz)."""
    khz = None
    for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
        try:
            hip = ctypes.CDLL(name)
        except OSError:
            continue
        v = ctypes.c_int(0)
        HIP_ATTR_CLOCK_RATE = 5   # hipDeviceAttributeClockRate
        if hip.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_CLOCK_RATE, 0) == 0 and v.value > 0:
            khz = v.value
        break
    out = {"cus": cus, "bf16_flops_per_clk_per_cu": 4096,
           "max_sclk_mhz": None if khz is None else khz / 1e3}
    out["derived_bf16_tflops"] = None if khz is None else round(cus * 4096 * khz * 1e3 / 1e12, 1)
    return out


# counters of the in-run pass (one rocprofv3 run each).  The byte counters
# are scaled by what they read for a plain copy of known size, measured in
# the same call (FETCH_SIZE has read half the copied bytes, WRITE_SIZE all
# of them).
COUNTER_PASSES = (("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"), ("FETCH_SIZE",),
                  ("WRITE_SIZE",))
CALIBRATION_MIB = 256


def counters_in_run(argv, kernels):
    """rocprofv3 counter passes over this bench (child processes, the same
    workload and mode, 3 steps): MFMA busy per SIMD and HBM bytes per call
    of the timed pass.  ``kernels``: the kernels that make up one call, each
    given by name substrings joined with "&" (all must occur in the name);
    each counter is averaged over each kernel's dispatches and the averages
    summed.  None when rocprofv3 is not available."""
    rp = shutil.which("rocprofv3")
    if rp is None:
        return None

    def passes(child, counter_sets):
        found = []   # (kernel name, counter name, value) of every dispatch
        for counters in counter_sets:
            with tempfile.TemporaryDirectory() as d:
                cmd = [rp, "--pmc", *counters, "--output-format", "csv", "-d", d, "-o", "c",
                       "--", *child]
                subprocess.run(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL,
                               timeout=300, cwd=tempfile.gettempdir())
                for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                   recursive=True):
                    for r in csv.DictReader(open(f)):
                        found.append((r["Kernel_Name"], r["Counter_Name"],
                                      float(r["Counter_Value"])))
        return found

    me = [sys.executable, os.path.abspath(__file__)]
    vals = {}   # (kernel, counter) -> values
    for name, counter, value in passes(me + [*argv, "--steps", "3", "--warmup", "1",
                                             "--no-cpu-baseline", "--no-counters"],
                              COUNTER_PASSES):
        for kn in kernels:
            if all(part in name for part in kn.split("&")):
                vals.setdefault((kn, counter), []).append(value)
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "FETCH_SIZE", "WRITE_SIZE")
    if not all(vals.get((kn, n)) for kn in kernels for n in need):
        return None
    # the copy of known size: CALIBRATION_MIB MiB read and written per
    # dispatch of the copy kernel (the fill that creates its source is not
    # counted)
    cal = {}
    for name, counter, value in passes(me + ["--copy-calibration", str(CALIBRATION_MIB),
                                             "--steps", "3", "--warmup", "1"],
                                       (("FETCH_SIZE",), ("WRITE_SIZE",))):
        if "copy" in name.lower():
            cal.setdefault(counter, []).append(value)
    if not (cal.get("FETCH_SIZE") and cal.get("WRITE_SIZE")):
        return None
    known_kib = CALIBRATION_MIB * 1024.0
    fetch_scale = known_kib / float(np.mean(cal["FETCH_SIZE"]))
    write_scale = known_kib / float(np.mean(cal["WRITE_SIZE"]))
    tot = {n: sum(float(np.mean(vals[(kn, n)])) for kn in kernels) for n in need}
    cycles = tot["GRBM_GUI_ACTIVE"] / 8          # summed over the 8 XCDs
    return {"mfma_busy": round(tot["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cycles), 4),
            "hbm_bytes_per_launch": (fetch_scale * tot["FETCH_SIZE"] +
                                     write_scale * tot["WRITE_SIZE"]) * 1024,
            "copy_calibration": {"mib": CALIBRATION_MIB, "fetch_scale": round(fetch_scale, 4),
                                 "write_scale": round(write_scale, 4)},
            "kernels": list(kernels),
            "passes": [" ".join(c) for c in COUNTER_PASSES]}


def to_device(x: np.ndarray):
    """Host storage array (bf16 bits as uint16, or fp32) -> GPU tensor."""
    import torch
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        return t.view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def flops_of(w, causal: bool, window=None) -> float:
    """4*d flops per visible (query, key) pair: exactly half the dense count
    for the causal square workloads (the pages' benchmark convention), the
    counted pairs for a sliding window (left, right; None = no bound)."""
    f = 4.0 * w.B * w.H * w.Lq * w.Lk * w.d
    if window is None:
        return f / 2 if causal else f
    i = np.arange(w.Lq, dtype=np.int64)
    hi = np.minimum(w.Lk - 1, i + window[1]) if window[1] is not None else np.full_like(i, w.Lk - 1)
    lo = np.maximum(0, i - window[0]) if window[0] is not None else np.zeros_like(i)
    pairs = int(np.maximum(hi - lo + 1, 0).sum())
    return 4.0 * w.B * w.H * w.d * pairs


HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def compulsory_bytes(w, backward: bool = False, fp8: bool = False) -> float:
    """Algorithmic HBM bytes of one call: every input read once and every
    output written once.  Forward: q, k, v in, o and the fp32 LSE out (FP8:
    one-byte inputs, bf16 o).  Backward: q, k, v, o, dO and LSE in, dq, dk,
    dv out."""
    esize = {"bf16": 2, "fp32": 4, "fp8": 1}[w.dtype]
    nq, nk = w.B * w.H * w.Lq * w.d, w.B * w.H * w.Lk * w.d
    rows = 4.0 * w.B * w.H * w.Lq
    if backward:
        return (3 * nq + 2 * nk) * esize + rows + (nq + 2 * nk) * esize
    osize = 2 if fp8 else esize
    return (nq + 2 * nk) * esize + nq * osize + rows


def cpu_baseline(w, causal, q, k, v, gpu_out, budget_s=15.0, max_heads=None,
                 window=None):
    """Time the oracle on whole (batch, head) slices of the workload, one
    after another, until ``budget_s`` of host time is spent or all slices
    are done.  Also reports the GPU result's error on that sample."""
    from oracle import algorithmic_flops, attention_ref, default_workers
    from seeded_inputs import widen
    cores = default_workers()
    O_gpu, L_gpu = gpu_out
    slices = [(b, h) for b in range(w.B) for h in range(w.H)]
    if max_heads:
        slices = slices[:max_heads]
    per_slice = algorithmic_flops(np.arange(w.Lq), w.Lk, w.d, causal, window)
    spent, done, eo, el, omax, lmax = 0.0, 0, 0.0, 0.0, 0.0, 0.0
    for b, h in slices:
        qs, ks, vs = (widen(x[b:b + 1, h:h + 1]) for x in (q, k, v))
        t0 = time.perf_counter()
        O_ref, L_ref = attention_ref(qs, ks, vs, causal, w.scale,
                                     workers=cores, chunk=256, window=window)
        spent += time.perf_counter() - t0
        done += 1
        eo = max(eo, float(np.abs(widen(O_gpu[b:b + 1, h:h + 1]) - O_ref).max()))
        fin = np.isfinite(L_ref)
        el = max(el, float(np.abs(L_gpu[b:b + 1, h:h + 1].astype(np.float64)[fin]
                                  - L_ref[fin]).max()))
        omax = max(omax, float(np.abs(O_ref).max()))
        lmax = max(lmax, float(np.abs(L_ref[fin]).max()))
        if spent >= budget_s:
            break
    fl = done * per_slice
    return {
        "value": fl / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{done} of {w.B * w.H} (batch, head) slices, all "
                   f"{w.Lq} query rows each, fp64 numpy oracle, "
                   f"{spent:.2f} s wall"),
        "seconds": spent,
        "sample_flops": fl,
    }, {"max_abs_err_O": eo, "max_abs_err_LSE": el, "max_abs_O_ref": omax,
        "max_abs_LSE_ref": lmax, "slices": done}


def cpu_baseline_fp8(w, causal, q8, k8, v8, ds, gpu_out, budget_s=15.0, max_heads=None):
    """Time the fp64 oracle (the exact definition on the dequantised E4M3
    inputs) on whole (batch, head) slices until budget_s of host time is
    spent; report the GPU result's error on that sample and its worst ratio
    to the derived FP8 bar (<= 1: within it): the E4M3 rounding of 2^8 P and
    an S error of at most gamma_{d-1} sum_t |q_t k_t| (fp32 additions in any
    order and rounding direction), plus 2^-8 |O| + 1e-4 for the bf16 output."""
    from oracle import attention_ref, default_workers, fp8_error_bound, fp8_flops
    from oracle.attention_fp8 import fp32_sum_error_factor
    from seeded_inputs import widen, widen_fp8
    cores = default_workers()
    s_err = fp32_sum_error_factor(w.d)
    O_gpu, L_gpu = gpu_out
    slices = [(b, h) for b in range(w.B) for h in range(w.H)]
    if max_heads:
        slices = slices[:max_heads]
    spent, done, ee, el, rx = 0.0, 0, 0.0, 0.0, 0.0
    for b, h in slices:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs = (widen_fp8(x[sl], s) for x, s in zip((q8, k8, v8), ds))
        t0 = time.perf_counter()
        O_ex, L_ex = attention_ref(qs, ks, vs, causal, w.scale, workers=cores, chunk=256)
        spent += time.perf_counter() - t0
        done += 1
        og = widen(O_gpu[sl])
        ee = max(ee, float(np.abs(og - O_ex).max()))
        el = max(el, float(np.abs(L_gpu[sl].astype(np.float64) - L_ex).max()))
        if done == 1:
            rows = np.arange(0, w.Lq, max(1, w.Lq // 256))
            bound = fp8_error_bound(qs, ks, vs, causal, w.scale, rows=rows, s_err=s_err)
            o_r, e_r = og[:, :, rows], O_ex[:, :, rows]
            rx = float((np.abs(o_r - e_r) / (bound + 2.0 ** -8 * np.abs(e_r) + 1e-4)).max())
        if spent >= budget_s:
            break
    fl = done * fp8_flops(w.Lq, w.Lk, w.d, causal)
    return {
        "value": fl / spent / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": (f"{done} of {w.B * w.H} (batch, head) slices, all {w.Lq} rows each, "
                   f"fp64 numpy oracle on the dequantised inputs, {spent:.2f} s wall"),
        "seconds": spent,
    }, {"max_abs_err_O": ee, "max_abs_err_LSE": el,
        "worst_ratio_to_fp8_bound_sampled_rows": rx, "slices": done}


def cpu_baseline_bwd(w, causal, q, k, v, do, grads, budget_s=15.0, max_heads=None):
    """Time the fp64 backward oracle on whole (batch, head) slices until
    ``budget_s`` of host time is spent; report the GPU gradients' error on
    that sample relative to each tensor's largest magnitude."""
    from oracle import attention_bwd_ref, backward_flops, default_workers
    from seeded_inputs import widen
    cores = default_workers()
    slices = [(b, h) for b in range(w.B) for h in range(w.H)]
    if max_heads:
        slices = slices[:max_heads]
    spent, done, rel = 0.0, 0, [0.0, 0.0, 0.0]
    for b, h in slices:
        xs = [widen(x[b:b + 1, h:h + 1]) for x in (q, k, v, do)]
        t0 = time.perf_counter()
        ref = attention_bwd_ref(*xs, causal, w.scale)
        spent += time.perf_counter() - t0
        done += 1
        for n, (g, r) in enumerate(zip(grads, ref)):
            gr = widen(g[b:b + 1, h:h + 1])
            rel[n] = max(rel[n], float(np.abs(gr - r).max() / np.abs(r).max()))
        if spent >= budget_s:
            break
    fl = done * backward_flops(w.Lq, w.Lk, w.d, causal)
    return {
        "value": fl / spent / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": (f"{done} of {w.B * w.H} (batch, head) slices, full backward each, "
                   f"fp64 numpy oracle (BLAS threads per numpy default), {spent:.2f} s wall"),
        "seconds": spent,
    }, {"max_rel_err_dQ": rel[0], "max_rel_err_dK": rel[1], "max_rel_err_dV": rel[2],
        "slices": done}


# Default launch counts.  Under a continuous load the GPU's clock takes
# tens of milliseconds to settle: launch durations first rise, then fall to
# a steady value (bench workload: ≈ 1.2 ms at the fourth launch, steady
# from about the thirtieth).  The default warm-up therefore runs for a
# fixed time rather than a fixed count, and the timed launches cover a
# fixed minimum time as well.
MIN_WARMUP, WARMUP_S = 5, 0.2
MIN_STEPS, TIMED_S = 50, 0.1


def warm_up(fn, args, n=None):
    """Untimed launches of fn(*args): exactly n if given, else at least
    MIN_WARMUP and at least WARMUP_S seconds of them.  Returns (launches,
    seconds per launch measured after the first one)."""
    import torch
    if n == 0:
        return 0, None
    fn(*args)                       # first launch: loads code, faults in pages
    torch.cuda.synchronize()
    t0, done, target = time.perf_counter(), 1, n
    batch = 1
    while True:
        if target is not None and done >= target:
            break
        k = batch if target is None else min(batch, target - done)
        for _ in range(k):
            fn(*args)
        torch.cuda.synchronize()
        done += k
        spent = time.perf_counter() - t0
        per = spent / (done - 1)
        if target is None and done >= MIN_WARMUP and spent >= WARMUP_S:
            break
        batch = max(1, min(4 * batch, math.ceil((WARMUP_S - spent) / per)))
    per = (time.perf_counter() - t0) / (done - 1) if done > 1 else None
    return done, per


def copy_calibration(mib: int, steps: int, warmup: int) -> int:
    """Plain copy of a known byte count: reads and writes mib MiB per step."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read_per_step": n * 4,
                      "copy_bytes_written_per_step": n * 4,
                      "ms_per_step": dt * 1e3,
                      "GB_per_s": 2 * n * 4 / dt / 1e9}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed launches (default: at least %d, and at least %.1f s of "
                         "them)" % (MIN_STEPS, TIMED_S))
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches before them (default: at least %d, and at "
                         "least %.1f s of them)" % (MIN_WARMUP, WARMUP_S))
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=["causal", "noncausal", "window", "splitkv", "bwd"],
                    default=None,
                    help="default: the workload's first mode")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="host seconds for the CPU-baseline sample")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="cap on (batch, head) slices in the CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="also run rocprofv3 counter passes (MFMA busy, HBM bytes) over "
                         "this bench in child processes")
    ap.add_argument("--no-counters", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device-to-device "
                         "copy of MIB MiB per step (the known-size reference "
                         "that HBM byte counters are scaled by)")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not "
              "supported (the forward shards over batch*head with no "
              "communication; see the design notes)", file=sys.stderr)
        return 2

    import torch
    if a.copy_calibration:
        return copy_calibration(a.copy_calibration, a.steps or MIN_STEPS,
                                MIN_WARMUP if a.warmup is None else a.warmup)
    import exact_io_aware_08_amd as fa
    from seeded_inputs import WORKLOADS, workload_inputs

    props = torch.cuda.get_device_properties(0)
    sclk = getattr(props, "clock_rate", 0) / 1e3   # kHz -> MHz, where torch reports it
    cus = props.multi_processor_count
    derived = device_peak(cus)
    log(f"bench: {props.name}: {cus} CUs" + (
        f", max sclk {derived['max_sclk_mhz']:.0f} MHz -> {cus} x 4096 bf16 flops/clk x sclk = "
        f"{derived['derived_bf16_tflops']:.1f} TFLOP/s dense bf16"
        if derived["derived_bf16_tflops"] else "") +
        "; the roofline uses the published peaks (bf16 2500, FP8 5000 TFLOP/s, HBM 8 TB/s)")

    w = WORKLOADS[a.workload]
    mode = a.mode or w.modes[0]
    causal = mode == "causal" or (mode in ("bwd", "splitkv") and "causal" in w.modes)
    window = w.window if mode == "window" else None
    fp8 = w.dtype == "fp8"
    if fp8 and mode not in ("causal", "noncausal"):
        raise SystemExit("the FP8 forward has causal and non-causal modes only")
    log(f"bench: workload {w.name} mode {mode}")
    if fp8:
        q, k, v, descales = workload_inputs(w)
        qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v))
    else:
        q, k, v = workload_inputs(w)
        qd, kd, vd = to_device(q), to_device(k), to_device(v)
    tdt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    od = torch.empty((w.B, w.H, w.Lq, w.d), dtype=tdt, device="cuda")
    ld = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    splits = w.splits if mode == "splitkv" else 0
    backward = mode == "bwd"
    if backward:
        if w.dtype != "bf16":
            raise SystemExit("the backward is bf16 only")
        from seeded_inputs import make_grad
        do = make_grad(w.seed, w.B, w.H, w.Lq, w.d)
        dod = to_device(do)
        # the forward's O and LSE, computed once outside the timed region
        fa.fa_fwd(qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, int(causal), w.scale, stream)
        dqd = torch.empty_like(od)
        dkd = torch.empty((w.B, w.H, w.Lk, w.d), dtype=torch.bfloat16, device="cuda")
        dvd = torch.empty_like(dkd)
        nbytes = fa.bwd_workspace_size(w.B, w.H, w.Lq)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")   # caller-owned scratch
        fn = fa.fa_bwd
        args = (qd, kd, vd, od, ld, dod, dqd, dkd, dvd, w.B, w.H, w.Lq, w.Lk, w.d,
                int(causal), w.scale, ws, nbytes, stream)
    elif fp8:
        fn = fa.fa_fwd_fp8
        args = (qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, int(causal), w.scale,
                *descales, stream)
    elif window is not None:
        fn = fa.fa_fwd_window
        args = (qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, *w.window_abi,
                w.scale, stream)
    elif splits:
        nbytes = fa.splitkv_workspace_size(w.B, w.H, w.Lq, w.d, splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")   # caller-owned scratch
        fn = fa.fa_fwd_splitkv
        args = (qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, int(causal), w.scale, splits,
                ws, nbytes, stream)
    else:
        fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32
        args = (qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, int(causal),
                w.scale, stream)

    a.warmup, per_launch = warm_up(fn, args, a.warmup)
    if a.steps is None:
        a.steps = MIN_STEPS if per_launch is None else max(MIN_STEPS,
                                                           math.ceil(TIMED_S / per_launch))
    log(f"bench: warm-up {a.warmup} launches, timing {a.steps}")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        starts[i].record(stream)
        fn(*args)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]   # ms
    ms_kernel = float(np.mean(per))
    ms_step = wall * 1e3 / a.steps
    flops = flops_of(w, causal, window)
    if backward:
        flops *= 2.5   # the pages' count: 2.0 (backward) + 0.5 (recomputed S, P)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"bench: kernel {ms_kernel:.4f} ms (min {min(per):.4f}, median "
        f"{float(np.median(per)):.4f}), step {ms_step:.4f} ms, "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.2f}% of {peak} peak")

    unsplit_ms = None
    if splits:
        # the same inputs through the unsplit kernel, for reference
        ref_args = (qd, kd, vd, od, ld, w.B, w.H, w.Lq, w.Lk, w.d, int(causal), w.scale, stream)
        for _ in range(2):
            fa.fa_fwd(*ref_args)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fa.fa_fwd(*ref_args)
        e1.record(stream)
        torch.cuda.synchronize()
        unsplit_ms = e0.elapsed_time(e1) / 10
        log(f"bench: unsplit fa_fwd on the same inputs {unsplit_ms:.4f} ms")
        fn(*args)   # leave the split result in od / ld for the CPU check
        torch.cuda.synchronize()

    gpu_out = None
    cpu = None
    parity = None
    if not a.no_cpu_baseline and backward:
        grads = [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (dqd, dkd, dvd)]
        log("bench: CPU oracle baseline (backward) ...")
        cpu, parity = cpu_baseline_bwd(w, causal, q, k, v, do, grads, a.cpu_budget, a.cpu_heads)
        log(f"bench: oracle {cpu['seconds']:.2f} s on {cpu['cores']} cores "
            f"-> {cpu['value'] * 1e3:.2f} GFLOP/s; parity on sample {parity}")
    elif not a.no_cpu_baseline and fp8:
        gpu_out = (od.view(torch.int16).cpu().numpy().view(np.uint16), ld.cpu().numpy())
        log("bench: CPU oracle baseline (FP8) ...")
        cpu, parity = cpu_baseline_fp8(w, causal, q, k, v, descales, gpu_out, a.cpu_budget,
                                       a.cpu_heads)
        log(f"bench: oracle {cpu['seconds']:.2f} s -> {cpu['value'] * 1e3:.2f} GFLOP/s; "
            f"parity on sample {parity}")
    elif not a.no_cpu_baseline:
        o_np = od.view(torch.int16).cpu().numpy().view(np.uint16) \
            if w.dtype == "bf16" else od.cpu().numpy()
        gpu_out = (o_np, ld.cpu().numpy())
        log("bench: CPU oracle baseline ...")
        cpu, parity = cpu_baseline(w, causal, q, k, v, gpu_out, a.cpu_budget,
                                   a.cpu_heads, window)
        log(f"bench: oracle {cpu['seconds']:.2f} s on {cpu['cores']} cores "
            f"-> {cpu['value'] * 1e3:.2f} GFLOP/s; parity on sample {parity}")

    # the kernel's bound: MFMA unless its arithmetic intensity (algorithmic
    # flops per compulsory byte) is below the ridge point peak / 8 TB/s
    cbytes = compulsory_bytes(w, backward, fp8)
    hbm_bound = flops / cbytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = traffic_from_profiles(w.name, backward, fp8, mode)
    if hbm_bound:
        gbs = cbytes / (ms_kernel * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 5), "traffic": traffic}
    roofline.update({
        "kernel_ms": round(ms_kernel, 5),
        "kernel_ms_median": round(float(np.median(per)), 5),
        "kernel_ms_min": round(float(min(per)), 5),
        "algorithmic_flops_per_launch": flops,
        "algorithmic_bytes_per_launch": cbytes,
        "arithmetic_intensity": round(flops / cbytes, 2),
        # achieved HBM rates: compulsory bytes, and measured bytes (rocprofv3
        # FETCH_SIZE + WRITE_SIZE of the committed profile) over the mean launch
        "hbm_gbs_algorithmic": round(cbytes / (ms_kernel * 1e-3) / 1e9, 2),
        "hbm_gbs_measured": None if traffic is None
        else round(traffic / (ms_kernel * 1e-3) / 1e9, 2),
    })
    if hbm_bound:
        roofline["tflops_achieved"] = round(achieved, 3)
    roofline["peak_derived_from_device"] = derived
    roofline["mfma_busy"] = mfma_busy_from_profiles(w.name, backward, fp8, mode)
    if a.counters and not a.no_counters:
        log("bench: rocprofv3 counter passes ...")
        if backward:
            knames = ["fa_bwd_pre", "fa_bwd_dkdv", "fa_bwd_dq"]
        elif fp8:
            knames = ["fa_fwd_fp8_kernel"]
        elif w.dtype != "bf16":
            knames = ["fa_fwd_kernel"]
        elif mode == "splitkv":
            # the split instantiation only (the unsplit comparison run
            # launches the same kernel name with SPLIT = false)
            knames = ["fa_fwd_direct_kernel&, true,", "fa_merge_kernel"]
        else:
            knames = ["fa_fwd_direct_kernel"]
        fwd_args = ["--workload", w.name, "--mode", mode]
        cr = counters_in_run(fwd_args, knames)
        if cr is not None:
            cr["hbm_gbs"] = round(cr["hbm_bytes_per_launch"] / (ms_kernel * 1e-3) / 1e9, 2)
        roofline["counters_in_run"] = cr

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else w.dtype,
        "data": "synthetic",
        "pct_of_mfma_peak": round(100 * value / peak, 3),
        "config": {"workload": f"{w.name} ({mode})", "B": w.B, "H": w.H,
                   "Lq": w.Lq, "Lk": w.Lk, "d": w.d, "causal": causal,
                   "window": None if window is None else list(w.window_abi),
                   "num_splits": splits or None, "pass": "backward" if backward else "forward",
                   "scale": w.scale, "seed": w.seed,
                   "sigma_qk": w.sigma_qk, "sigma_v": w.sigma_v},
        "roofline": roofline,
        "cpu_baseline": None if cpu is None else {
            k2: cpu[k2] for k2 in ("value", "unit", "cores", "kind", "sample")},
    }
    ok = True
    if parity is not None:
        line["parity_on_cpu_sample"] = parity
        ok = parity_ok(parity, w, backward, fp8)
        line["parity_ok"] = ok
    if unsplit_ms is not None:
        line["unsplit_kernel_ms"] = round(unsplit_ms, 5)
    print(json.dumps(line), flush=True)
    if not ok:
        log("bench: the result on the CPU sample is outside the parity bars")
        return 1
    return 0


def parity_ok(parity: dict, w, backward: bool, fp8: bool) -> bool:
    """The parity bars on the CPU sample: bf16 O 2e-2 and LSE 1e-3 absolute;
    fp32 1e-5 of each tensor's largest magnitude; FP8 within the derived
    bound and LSE 1e-3; backward 2e-2 of each gradient's largest
    magnitude."""
    if backward:
        return all(parity[k] <= 2e-2 for k in ("max_rel_err_dQ", "max_rel_err_dK",
                                               "max_rel_err_dV"))
    if fp8:
        return (parity["worst_ratio_to_fp8_bound_sampled_rows"] <= 1.0 and
                parity["max_abs_err_LSE"] <= 1e-3)
    if w.dtype == "fp32":
        return (parity["max_abs_err_O"] <= 1e-5 * parity["max_abs_O_ref"] and
                parity["max_abs_err_LSE"] <= 1e-5 * parity["max_abs_LSE_ref"])
    return parity["max_abs_err_O"] <= 2e-2 and parity["max_abs_err_LSE"] <= 1e-3


if __name__ == "__main__":
    sys.exit(main())
