"""MI355X (gfx950) FlashAttention-2 forward: thin Python binding.

The compute lives entirely in ``libfa_fwd.so`` (HIP kernels behind the C ABI
declared in ``include/fa.h``).  This module only marshals arguments: raw
device pointers, sizes and a stream handle.  PyTorch is used, when the
caller passes tensors, for device memory and streams only.

There is no fallback: if the library is missing, importing the binding's
entry points raises ``FABuildError``.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_fwd.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED_D",
    4: "FA_ERR_ALIGN", 5: "FA_ERR_SCALE", 6: "FA_ERR_ARG", 7: "FA_ERR_LAUNCH",
    8: "FA_ERR_WORKSPACE",
}
# every function the C header declares
EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_fwd_window", "fa_fwd_splitkv",
           "fa_fwd_splitkv_noalloc", "fa_noalloc_scratch_bytes", "fa_splitkv_workspace_size", "fa_splitkv_suggest", "fa_bwd", "fa_bwd_workspace_size",
           "fa_status_string", "fa_abi_version", "fa_tile_config")


class FABuildError(RuntimeError):
    pass


class FAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa_fwd.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FABuildError(
            f"{path} is missing: build it with `python -m "
            "exact_io_aware_08_amd.build` (or __graft_entry__.build())")
    # torch ships its own HIP runtime under the same soname as ROCm's.  If
    # this library were loaded first it would bring in the system runtime,
    # torch would then run on that one or on its own, and launches on torch's
    # streams fail ("invalid device function").  Loading torch first makes
    # the library bind to the runtime that owns the caller's tensors and
    # streams.  Without torch (raw device pointers) nothing changes.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd.argtypes = sig
    lib.fa_fwd.restype = i
    lib.fa_fwd_f32.argtypes = sig
    lib.fa_fwd_f32.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_window.restype = i
    sz = ctypes.c_size_t
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_noalloc_scratch_bytes.argtypes = []
    lib.fa_noalloc_scratch_bytes.restype = sz
    lib.fa_splitkv_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_splitkv_workspace_size.restype = sz
    lib.fa_splitkv_suggest.argtypes = [i, i, i, i, i, i, i]
    lib.fa_splitkv_suggest.restype = i
    lib.fa_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, f, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    lib.fa_tile_config.argtypes = [i, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                   ctypes.POINTER(i)]
    lib.fa_tile_config.restype = i
    _lib = lib
    return lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"expected a device pointer or tensor, got {type(x)!r}")


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"expected a stream handle, got {type(s)!r}")


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def abi_version() -> int:
    return int(load_library().fa_abi_version())


def tile_config(dtype: str, d: int):
    """(block_m, block_n, threads) the library uses for dtype 'bf16', 'fp32'
    or 'fp8'."""
    lib = load_library()
    bm, bn, th = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    st = lib.fa_tile_config({"bf16": 0, "fp32": 1, "fp8": 2}[dtype], int(d),
                            ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(th))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return bm.value, bn.value, th.value


def _call(fn, q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, stream):
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
            int(Lq), int(Lk), int(d), int(causal), float(scale), _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def fa_fwd(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, stream=None):
    """bf16 forward through the C ABI (``fa_fwd`` in include/fa.h).

    q, k, v, o, lse: device pointers (ints) or tensors; stream: hipStream_t
    handle, a torch stream, or None for the null stream.  Raises FAError on
    a nonzero status."""
    return _call(load_library().fa_fwd, q, k, v, o, lse, B, H, Lq, Lk, d,
                 causal, scale, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, stream=None):
    """fp32 forward through the C ABI (``fa_fwd_f32``)."""
    return _call(load_library().fa_fwd_f32, q, k, v, o, lse, B, H, Lq, Lk, d,
                 causal, scale, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, q_descale, k_descale,
               v_descale, stream=None):
    """FP8 (E4M3) forward through the C ABI (``fa_fwd_fp8``): q, k, v hold
    E4M3 codes (one byte each) standing for code * descale; o is bf16."""
    st = load_library().fa_fwd_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Lq), int(Lk),
        int(d), int(causal), float(scale), float(q_descale), float(k_descale),
        float(v_descale), _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def fa_fwd_window(q, k, v, o, lse, B, H, Lq, Lk, d, window_left, window_right,
                  scale, stream=None):
    """bf16 sliding-window forward through the C ABI (``fa_fwd_window``):
    key j visible to query i iff i - window_left <= j <= i + window_right;
    -1 leaves that side unbounded."""
    st = load_library().fa_fwd_window(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Lq),
        int(Lk), int(d), int(window_left), int(window_right), float(scale),
        _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def splitkv_workspace_size(B, H, Lq, d, num_splits) -> int:
    """Bytes of workspace fa_fwd_splitkv needs (0: invalid arguments)."""
    return int(load_library().fa_splitkv_workspace_size(int(B), int(H), int(Lq),
                                                         int(d), int(num_splits)))


def splitkv_suggest(B, H, Lq, Lk, d, causal=False, num_cus=0) -> int:
    """num_splits the library suggests for fa_fwd_splitkv on this shape
    (``fa_splitkv_suggest``; 1: no split needed, 0: invalid arguments)."""
    return int(load_library().fa_splitkv_suggest(int(B), int(H), int(Lq), int(Lk), int(d),
                                                 int(causal), int(num_cus)))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, num_splits,
                   workspace, workspace_bytes, stream=None):
    """bf16 key-split forward through the C ABI (``fa_fwd_splitkv``):
    ``num_splits`` partial results in the caller's ``workspace`` (device
    pointer or tensor of at least ``splitkv_workspace_size`` bytes), then
    their merge into o and lse."""
    st = load_library().fa_fwd_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Lq),
        int(Lk), int(d), int(causal), float(scale), int(num_splits), _ptr(workspace),
        int(workspace_bytes), _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Lq, Lk, d, causal, scale, num_splits,
                           stream=None):
    """bf16 key-split forward through the C ABI (``fa_fwd_splitkv_noalloc``):
    the partials go to the library's fixed per-GPU scratch, so nothing is
    allocated; calls that overlap on one GPU race."""
    st = load_library().fa_fwd_splitkv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Lq),
        int(Lk), int(d), int(causal), float(scale), int(num_splits), _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed scratch ``fa_fwd_splitkv_noalloc`` uses per GPU."""
    return int(load_library().fa_noalloc_scratch_bytes())


def bwd_workspace_size(B, H, Lq) -> int:
    """Bytes of workspace fa_bwd needs (0: invalid arguments)."""
    return int(load_library().fa_bwd_workspace_size(int(B), int(H), int(Lq)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, causal, scale,
           workspace, workspace_bytes, stream=None):
    """bf16 backward through the C ABI (``fa_bwd``): dq, dk, dv from q, k,
    v, the forward's o and lse, and the upstream gradient dout."""
    st = load_library().fa_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), int(B), int(H), int(Lq), int(Lk), int(d), int(causal), float(scale),
        _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != FA_OK:
        raise FAError(st, status_string(st))
    return st


def attention(q, k, v, causal: bool = False, scale: float | None = None,
              stream=None, window=None, num_splits: int | None = None):
    """Convenience wrapper on torch tensors [B,H,L,d] (bf16 or fp32, on the
    GPU, contiguous): allocates O and LSE with torch and calls the C ABI on
    ``stream`` (a torch stream or a raw handle; default: torch's current
    stream).  On another stream than the current one, the launch stream
    first waits for the current stream's work, O, LSE and the workspace are
    allocated on the launch stream (so torch never hands their memory to
    other work while the kernels run), and q, k, v are recorded as used
    there; the caller synchronises before reading O and LSE on another
    stream, as with any torch side stream.  ``window``: optional (left,
    right) sliding window, None on a side for no bound (bf16 only; combined
    with ``causal`` the right bound is 0).  ``num_splits``: split the keys
    among that many workgroups per query block and merge (bf16 only; the
    workspace is allocated with torch); ``"auto"``: the count
    ``splitkv_suggest`` gives for this shape on this device, no split when it
    gives 1 (or for fp32 inputs or a window).  Returns (O, LSE)."""
    import torch
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, L, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, d) or tuple(v.shape) != (B, H, Lk, d):
        raise ValueError("k and v must be [B, H, Lk, d] matching q")
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if isinstance(num_splits, str):
        if num_splits != "auto":
            raise ValueError(f"num_splits must be an int, None or 'auto', not {num_splits!r}")
        num_splits = None
        if q.dtype == torch.bfloat16 and window is None:
            n = splitkv_suggest(B, H, Lq, Lk, d, causal)
            if n > 1:
                num_splits = n
    current = torch.cuda.current_stream(q.device)
    if stream is None:
        stream = current
    elif isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=q.device)
    if stream != current:
        stream.wait_stream(current)
        for t in (q, k, v):
            t.record_stream(stream)
    with torch.cuda.stream(stream):
        return _attention_on(q, k, v, causal, scale, stream, window, num_splits, B, H, Lq,
                             Lk, d)


def _attention_on(q, k, v, causal, scale, stream, window, num_splits, B, H, Lq, Lk, d):
    # body of attention(): runs with `stream` as torch's current stream, so
    # every allocation below belongs to it
    import torch
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if num_splits is not None:
        if q.dtype != torch.bfloat16 or window is not None:
            raise ValueError("key splits are implemented for bf16 without a window")
        nbytes = splitkv_workspace_size(B, H, Lq, d, num_splits)
        if nbytes == 0:
            raise ValueError(f"unsupported num_splits {num_splits}")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        fa_fwd_splitkv(q, k, v, o, lse, B, H, Lq, Lk, d, int(causal), scale,
                       num_splits, ws, nbytes, stream)
    elif window is not None:
        if q.dtype != torch.bfloat16:
            raise ValueError("sliding windows are implemented for bf16 only")
        left = -1 if window[0] is None else int(window[0])
        right = -1 if window[1] is None else int(window[1])
        if causal:
            right = 0 if right < 0 else min(right, 0)
        fa_fwd_window(q, k, v, o, lse, B, H, Lq, Lk, d, left, right, scale, stream)
    elif q.dtype == torch.bfloat16:
        fa_fwd(q, k, v, o, lse, B, H, Lq, Lk, d, int(causal), scale, stream)
    elif q.dtype == torch.float32:
        fa_fwd_f32(q, k, v, o, lse, B, H, Lq, Lk, d, int(causal), scale, stream)
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return o, lse


__all__ = ["fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_fwd_window", "fa_fwd_splitkv",
           "fa_fwd_splitkv_noalloc", "noalloc_scratch_bytes",
           "splitkv_workspace_size", "splitkv_suggest", "fa_bwd", "bwd_workspace_size",
           "attention",
           "status_string",
           "abi_version", "tile_config", "load_library", "FAError",
           "FABuildError", "EXPORTS", "LIB_PATH"]
