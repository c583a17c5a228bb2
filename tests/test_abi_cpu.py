"""The C-ABI library loads on a CPU-only host, exports every symbol that
include/fa.h declares, and rejects bad arguments on the host before any HIP
call (these calls never reach a launch, so no GPU is needed)."""
import math
import os
import re
import subprocess

import pytest

import exact_io_aware_08_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# distinct, 16-byte aligned fake device addresses: never dereferenced,
# because every call below fails validation first
Q, K, V, O, L = (0x10000000 * i for i in range(1, 6))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_header_declares_expected_symbols():
    assert declared_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+FA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert fa.abi_version() == int(m.group(1))


def test_status_strings(lib):
    for st in range(10):
        assert fa.status_string(st) != "unknown status"
    assert fa.status_string(99) == "unknown status"


def test_tile_config():
    for dt in ("bf16", "fp32"):
        for d in (64, 128, 256):
            bm, bn, th = fa.tile_config(dt, d)
            assert bm % 32 == 0 and bn % 32 == 0
            assert th in (128, 256, 512) and bm % (th // 64 * 32) == 0
    with pytest.raises(fa.FAError):
        fa.tile_config("bf16", 96)
    bm, bn, th = fa.tile_config("fp8", 128)
    # the FP8 kernel's key tile is the block the blocked FP8 diagnostic uses
    from oracle.attention_fp8 import FP8_DIAG_BLOCK
    assert bn == FP8_DIAG_BLOCK
    assert bm % 32 == 0 and bn % 64 == 0 and bm % (th // 64 * 32) == 0
    for d in (64, 256):
        with pytest.raises(fa.FAError):
            fa.tile_config("fp8", d)


def _st(fn, **kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Lq=128, Lk=128, d=64,
                causal=0, scale=0.125)
    args.update(kw)
    try:
        fn(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32])
def test_validation_errors(fn):
    assert _st(fn, q=0) == 1
    assert _st(fn, lse=0) == 1
    for bad in ({"B": 0}, {"H": -1}, {"Lq": 0}, {"Lk": 0}):
        assert _st(fn, **bad) == 2
    for d in (0, 32, 96, 512):
        assert _st(fn, d=d) == 3
    assert _st(fn, k=K + 8) == 4
    assert _st(fn, o=O + 2) == 4
    for s in (-0.5, -0.0 - 1e-30, math.inf, math.nan):
        assert _st(fn, scale=s) == 5
    # scale * log2(e) past fp32's range (the exponent factor would be inf)
    assert _st(fn, scale=3e38) == 5
    assert _st(fn, scale=2e38, causal=2) == 6
    # scale = 0 is accepted (the check after it fails instead)
    assert _st(fn, scale=0.0, causal=2) == 6
    assert _st(fn, causal=2) == 6
    assert _st(fn, causal=-1) == 6
    # outputs overlapping an input or each other
    assert _st(fn, o=Q + 256) == 6
    assert _st(fn, lse=V + 1024) == 6
    assert _st(fn, lse=O + 16) == 6
    # a grid too large for one dimension
    assert _st(fn, B=1 << 16, H=1 << 15, Lq=1 << 20) == 2


def _st_window(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Lq=128, Lk=128, d=64,
                window_left=16, window_right=0, scale=0.125)
    args.update(kw)
    try:
        fa.fa_fwd_window(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


def test_window_validation_errors():
    assert _st_window(q=0) == 1
    assert _st_window(Lk=0) == 2
    assert _st_window(d=96) == 3
    assert _st_window(v=V + 4) == 4
    assert _st_window(scale=math.nan) == 5
    for wl, wr in ((-2, 0), (0, -2), (-5, -5)):
        assert _st_window(window_left=wl, window_right=wr) == 6
    assert _st_window(o=K + 64) == 6


W = 0x10000000 * 7   # fake workspace address, disjoint from the others


def _st_split(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Lq=128, Lk=128, d=64,
                causal=0, scale=0.125, num_splits=4, workspace=W,
                workspace_bytes=1 << 30)
    args.update(kw)
    try:
        fa.fa_fwd_splitkv(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


def test_splitkv_workspace_size():
    # fp32 partial O then fp32 partial LSE, each rounded up to 256 bytes
    def r(n):
        return (n + 255) // 256 * 256
    for (B, H, Lq, d, S) in ((1, 2, 128, 64, 4), (2, 3, 77, 128, 7), (1, 1, 1, 256, 1)):
        assert fa.splitkv_workspace_size(B, H, Lq, d, S) == \
            r(S * B * H * Lq * d * 4) + r(S * B * H * Lq * 4)
    for bad in ((0, 1, 8, 64, 2), (1, 1, 8, 96, 2), (1, 1, 8, 64, 0), (1, 1, 8, 64, 65)):
        assert fa.splitkv_workspace_size(*bad) == 0


def test_splitkv_validation_errors():
    assert _st_split(workspace=0) == 1
    assert _st_split(workspace=W + 8) == 4
    assert _st_split(causal=3) == 6
    for n in (0, -1, 65):
        assert _st_split(num_splits=n) == 6
    need = fa.splitkv_workspace_size(1, 2, 128, 64, 4)
    assert _st_split(workspace_bytes=need - 1) == 8
    assert _st_split(workspace=Q + 256) == 6         # overlaps q
    assert _st_split(d=32) == 3


def _st_noalloc(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Lq=128, Lk=128, d=64,
                causal=0, scale=0.125, num_splits=4)
    args.update(kw)
    try:
        fa.fa_fwd_splitkv_noalloc(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


def test_noalloc_validation_errors():
    # the ordinary key-split checks run first, on the host
    assert fa.noalloc_scratch_bytes() == 40 << 20
    assert _st_noalloc(q=0) == 1
    assert _st_noalloc(B=0) == 2
    assert _st_noalloc(d=96) == 3
    assert _st_noalloc(o=O + 2) == 4
    assert _st_noalloc(scale=-1.0) == 5
    assert _st_noalloc(causal=2) == 6
    for n in (0, 65):
        assert _st_noalloc(num_splits=n) == 6
    assert _st_noalloc(o=Q + 256) == 6
    # partials beyond the fixed scratch: a clear error, before any HIP call
    cap = fa.noalloc_scratch_bytes()
    big = dict(B=1, H=16, Lq=4096, Lk=65536, d=128, num_splits=8)
    assert fa.splitkv_workspace_size(1, 16, 4096, 128, 8) > cap
    assert _st_noalloc(**big) == 9
    assert "scratch" in fa.status_string(9)


DO, DQ, DK, DV, WB = (0x10000000 * i for i in range(8, 13))


def _st_bwd(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, B=1, H=2,
                Lq=128, Lk=128, d=64, causal=1, scale=0.125, workspace=WB,
                workspace_bytes=1 << 20)
    args.update(kw)
    try:
        fa.fa_bwd(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


def test_bwd_workspace_size():
    assert fa.bwd_workspace_size(1, 2, 128) == 2 * ((2 * 128 * 4 + 255) // 256 * 256)
    assert fa.bwd_workspace_size(2, 3, 77) == 2 * ((6 * 77 * 4 + 255) // 256 * 256)
    assert fa.bwd_workspace_size(0, 2, 128) == 0


def test_bwd_validation_errors():
    assert _st_bwd(dout=0) == 1
    assert _st_bwd(workspace=0) == 1
    assert _st_bwd(Lk=0) == 2
    assert _st_bwd(d=256) == 3 and _st_bwd(d=96) == 3
    assert _st_bwd(dq=DQ + 8) == 4
    assert _st_bwd(scale=0.0) == 5
    assert _st_bwd(scale=3e38) == 5
    assert _st_bwd(causal=2) == 6
    assert _st_bwd(workspace_bytes=fa.bwd_workspace_size(1, 2, 128) - 1) == 8
    assert _st_bwd(dk=Q + 64) == 6         # an output overlapping an input
    assert _st_bwd(dv=DK + 16) == 6        # two outputs overlapping


def _st_fp8(**kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Lq=128, Lk=128, d=128,
                causal=0, scale=0.125, q_descale=0.01, k_descale=0.02, v_descale=0.03)
    args.update(kw)
    try:
        fa.fa_fwd_fp8(**args)
    except fa.FAError as e:
        return e.status
    raise AssertionError("call was expected to fail validation")


def test_fp8_validation_errors():
    assert _st_fp8(v=0) == 1
    for bad in ({"B": 0}, {"Lq": 0}, {"Lk": -3}):
        assert _st_fp8(**bad) == 2
    for d in (64, 96, 256):
        assert _st_fp8(d=d) == 3
    assert _st_fp8(q=Q + 8) == 4
    for name in ("scale", "q_descale", "k_descale", "v_descale"):
        for x in (-1.0, math.inf, math.nan):
            assert _st_fp8(**{name: x}) == 5
    for name in ("q_descale", "k_descale", "v_descale"):
        assert _st_fp8(**{name: 0.0}) == 5
    # scale = 0 is accepted (the check after it fails instead)
    assert _st_fp8(scale=0.0, causal=3) == 6
    # the combined exponent factor overflows fp32; one that underflows
    # weighs every key the same, as scale = 0 does
    assert _st_fp8(q_descale=1e30, k_descale=1e30) == 5
    assert _st_fp8(q_descale=1e-30, k_descale=1e-30, causal=3) == 6
    assert _st_fp8(causal=3) == 6
    # o is bf16 (2 bytes per element) over 1-byte inputs: o = [Q, Q + 2 |q|)
    assert _st_fp8(k=Q + 2 * 2 * 128 * 128 - 16, o=Q, q=O) == 6
    assert _st_fp8(lse=V + 2 * 128 * 128 - 16) == 6


@pytest.mark.parametrize("shape,want", [
    ((1, 16, 512, 65536, 128, 0), 8),      # 32 query blocks: 8 splits cover 256 CUs
    ((1, 8, 256, 32768, 128, 0), 32),
    ((2, 16, 1024, 16384, 128, 0), 2),
    ((1, 4, 64, 131072, 64, 0), 64),       # capped at 64
    ((1, 2, 512, 8000, 256, 0), 31),       # capped at 8 tiles per split (250 tiles of 32)
    ((1, 4, 4096, 4096, 128, 1), 4),       # causal: capped at 8 of the longest block's 32 tiles
    ((1, 2, 16384, 16384, 128, 1), 4),     # causal: 128 longest / (8320 tiles / 256 CUs)
    ((1, 4, 16384, 16384, 128, 1), 2),     # causal: 256 blocks, the longest twice the mean
    ((1, 16, 16384, 16384, 128, 1), 1),    # causal: 1024 blocks balance on their own
    ((4, 16, 2048, 8192, 128, 0), 1),      # 512 query blocks already fill 256 CUs
    ((1, 1, 100, 100, 128, 0), 1),         # too few tiles to split
    ((4, 16, 1024, 1024, 64, 1), 1),       # causal d = 64: 512 blocks, 16 tiles at most
    ((2, 16, 1024, 1024, 64, 1), 1),       # 2 by the causal rule; key halves already
    ((1, 4, 4096, 4096, 64, 1), 4),        # 64 longest / (4224 tiles / 256 CUs)
    ((1, 8, 128, 8192, 64, 0), 16),        # 32 by the CU rule, capped at 8 of 128 tiles
    ((1, 16, 1024, 2048, 64, 0), 1),       # 128 blocks: 2 by the CU rule; key halves already
    ((1, 16, 1024, 2048, 128, 0), 2),      # d = 128: 64 blocks, 4 by the CU rule, capped at 16 / 8
])
def test_splitkv_suggest(shape, want):
    assert fa.splitkv_suggest(*shape, num_cus=256) == want


def test_splitkv_suggest_invalid():
    assert fa.splitkv_suggest(0, 1, 8, 8, 128, 0, 256) == 0
    assert fa.splitkv_suggest(1, 1, 8, 8, 96, 0, 256) == 0
    assert fa.splitkv_suggest(1, 1, 8, 8, 128, 2, 256) == 0


def test_attention_rejects_unknown_split_mode():
    """num_splits takes an int, None or 'auto'; any other string is refused
    before any GPU work."""
    import torch
    x = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="num_splits"):
        fa.attention(x, x, x, num_splits="fastest")
