"""Seeded synthetic inputs for the attention forward pass.

This module is the only code that both the CPU oracle side (tests, the
bench's CPU baseline) and the HIP side (tests, bench, smoke) use.  It draws
i.i.d. Gaussian Q, K, V from a numpy ``default_rng(seed)`` and, for the bf16
workloads, rounds them to bfloat16 with round-to-nearest-even.  It contains
no attention arithmetic: no products, no softmax, no masking.

The value distributions follow the pages' own test and benchmark inputs
(standard normal Q, K, V: "第 08 章: Flash Attention——分块注意力",
chuoer47.github.io, the test and benchmark harness of its listing), with the
per-workload sigma and sizes listed in ``WORKLOADS``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str            # "bf16", "fp32" or "fp8" (E4M3 codes + descales)
    modes: tuple          # subset of ("noncausal", "causal", "window", "splitkv")
    seed: int
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    window: tuple | None = None   # (left, right), None for no bound
    splits: int = 0               # key splits for the "splitkv" mode

    @property
    def window_abi(self) -> tuple:
        """The window as fa_fwd_window takes it: -1 for no bound."""
        return tuple(-1 if w is None else int(w) for w in self.window)

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to fp32: the value both sides receive.
        return float(np.float32(1.0) / np.sqrt(np.float32(self.d)))


# The synthetic workloads (one seed each, drawn in the order Q, K, V).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 128, 128, 64, "fp32",
                          ("noncausal", "causal"), 1),
    "bf16_causal_1k_d64": Workload("bf16_causal_1k_d64", 4, 16, 1024, 1024, 64,
                                   "bf16", ("causal",), 2),
    "bf16_4k_d128": Workload("bf16_4k_d128", 2, 32, 4096, 4096, 128, "bf16",
                             ("noncausal", "causal"), 3),
    "bf16_causal_16k_d128": Workload("bf16_causal_16k_d128", 1, 16, 16384,
                                     16384, 128, "bf16", ("causal",), 4),
    "bf16_peaky_d256_ragged": Workload("bf16_peaky_d256_ragged", 1, 8, 8000,
                                       8192, 256, "bf16", ("noncausal",), 5,
                                       sigma_qk=3.0),
    # sliding window of 1024 keys to the left and none to the right, the
    # pages' example window ("Flash Attention 原理与实现详解" (tbr8.org),
    # section 6.3), at the 16K causal shape
    "bf16_window1k_16k_d128": Workload("bf16_window1k_16k_d128", 1, 16, 16384,
                                       16384, 128, "bf16", ("window",), 6,
                                       window=(1024, 0)),
    # short queries against a long key sequence: 2 query blocks per head,
    # too few workgroups for 256 CUs unless the keys are split (8 splits:
    # 256 workgroups, the fastest of 1..64 measured)
    "bf16_longkv_512x64k_d128": Workload("bf16_longkv_512x64k_d128", 1, 16, 512,
                                         65536, 128, "bf16", ("splitkv",), 7,
                                         splits=8),
    # one GPU's share of the 16K causal workload when its 16 heads are split
    # over 8 GPUs: 128 query blocks for 256 CUs, so the keys are split (4
    # splits, the fastest of 1..8 measured, and fa_splitkv_suggest's choice)
    "bf16_causal_16k_d128_2h": Workload("bf16_causal_16k_d128_2h", 1, 2, 16384, 16384, 128,
                                        "bf16", ("splitkv", "causal"), 9, splits=4),
    # FP8 E4M3 inputs (per-tensor descale) at the 16K causal shape, the
    # pages' FP8 variant ("Flash Attention 原理与实现详解" (tbr8.org), section
    # 4.3 "FP8 支持")
    "fp8_causal_16k_d128": Workload("fp8_causal_16k_d128", 1, 16, 16384, 16384, 128,
                                    "fp8", ("causal",), 8),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite Gaussian draws, so NaN handling is not needed; an
    assertion guards that assumption.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.isfinite(x).all()
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw(seed: int, B: int, H: int, Lq: int, Lk: int, d: int,
         sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Draw fp32 Q [B,H,Lq,d], K [B,H,Lk,d], V [B,H,Lk,d] in that order."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Lq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Lk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Lk, d), dtype=np.float32)
    if sigma_qk != 1.0:
        q *= np.float32(sigma_qk)
        k *= np.float32(sigma_qk)
    if sigma_v != 1.0:
        v *= np.float32(sigma_v)
    return q, k, v


def make_inputs(seed: int, B: int, H: int, Lq: int, Lk: int, d: int,
                dtype: str = "bf16", sigma_qk: float = 1.0,
                sigma_v: float = 1.0):
    """Return (q, k, v) as the device-side storage arrays.

    dtype "bf16": uint16 arrays holding bfloat16 bits (RNE from the fp32
    draw).  dtype "fp32": float32 arrays.  The oracle side widens these with
    ``widen`` so both sides see identical values.
    """
    q, k, v = draw(seed, B, H, Lq, Lk, d, sigma_qk, sigma_v)
    if dtype == "bf16":
        return round_to_bf16_bits(q), round_to_bf16_bits(k), round_to_bf16_bits(v)
    if dtype == "fp32":
        return q, k, v
    raise ValueError(f"unknown dtype {dtype!r}")


def make_grad(seed: int, B: int, H: int, Lq: int, d: int) -> np.ndarray:
    """Upstream gradient dO [B,H,Lq,d] for the backward pass: standard
    normal (the pages' benchmark draws it with randn_like), from its own
    generator (seed + 1000), rounded to bfloat16 bits."""
    rng = np.random.default_rng(seed + 1000)
    return round_to_bf16_bits(rng.standard_normal((B, H, Lq, d), dtype=np.float32))


# ---- FP8 inputs (OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa
# bits; no infinities; S.1111.111 is NaN; largest finite 448) ------------------
def _e4m3_positive_table() -> np.ndarray:
    """Values of the codes 0..126 (all finite non-negative ones), ascending."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3_POS = _e4m3_positive_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> exact float64 values (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    val = np.where(mag == 0x7F, np.nan, _E4M3_POS[np.minimum(mag, 126)])
    return np.where(c & 0x80, -val, val)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes, round to nearest, ties to even; |x| <= 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.isfinite(a).all() and (a <= 448.0).all()
    hi = np.minimum(np.searchsorted(_E4M3_POS, a, side="left"), 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(_E4M3_POS[hi] == a, hi, pick)
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor quantisation: descale = max|x| / 448 (fp32), codes =
    e4m3(x / descale).  The value a code stands for is decode(code) *
    descale."""
    amax = float(np.abs(x).max())
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    y = np.asarray(x, dtype=np.float64) / descale
    return e4m3_encode(np.clip(y, -448.0, 448.0)), descale


def make_inputs_fp8(seed: int, B: int, H: int, Lq: int, Lk: int, d: int,
                    sigma_qk: float = 1.0, sigma_v: float = 1.0):
    """Return (q8, k8, v8, (q_descale, k_descale, v_descale)): the same fp32
    Gaussian draw as make_inputs, each tensor quantised to E4M3 codes with its
    own per-tensor descale factor."""
    q, k, v = draw(seed, B, H, Lq, Lk, d, sigma_qk, sigma_v)
    (q8, qd), (k8, kd), (v8, vd) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    return q8, k8, v8, (qd, kd, vd)


def widen_fp8(codes: np.ndarray, descale: float) -> np.ndarray:
    """E4M3 codes and their descale -> the exact float64 values they stand
    for (decode(code) * descale, exact in float64)."""
    return e4m3_decode(codes) * float(descale)


def widen(x: np.ndarray) -> np.ndarray:
    """Storage array (bf16 bits or fp32) -> exact float64 values."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def workload_inputs(w: Workload):
    """(q, k, v) storage arrays; fp8 workloads also return the descales as a
    fourth element."""
    if w.dtype == "fp8":
        return make_inputs_fp8(w.seed, w.B, w.H, w.Lq, w.Lk, w.d, w.sigma_qk, w.sigma_v)
    return make_inputs(w.seed, w.B, w.H, w.Lq, w.Lk, w.d, w.dtype,
                       w.sigma_qk, w.sigma_v)
