"""The entry points under HIP graph capture (torch.cuda.CUDAGraph on ROCm):
fa_fwd, fa_fwd_splitkv, fa_bwd and fa_fwd_fp8 each enqueue kernels only (no
allocation, no memset), so a captured call replays.  Each replay runs with
other eager work and a synchronisation between replays and must match the
eager result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest

import exact_io_aware_08_amd as fa
from seeded_inputs import make_grad, make_inputs, make_inputs_fp8
from tests.gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu

B, H, L, D = 1, 4, 1000, 128
SCALE = float(np.float32(1.0) / np.sqrt(np.float32(D)))


def _replays_match(make_outputs, call, n=3):
    """Eager call into one output set, captured call into another, then n
    replays with eager work in between; every replay must equal eager."""
    import torch
    eager = make_outputs()
    call(eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in eager]
    graphed = make_outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capture stream
        call(graphed, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(graphed, torch.cuda.current_stream())
    for r in range(n):
        for t in graphed:
            t.fill_(float("nan")) if t.is_floating_point() else t.fill_(0x7FC1)
        junk = torch.randn(1 << 20, device="cuda").sum()   # other eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for a, b in zip(graphed, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"replay {r} differs from the eager result"
    say(f"{n} replays equal the eager result")


def test_graph_fa_fwd():
    import torch
    q, k, v = (to_device(x) for x in make_inputs(81, B, H, L, L, D, "bf16"))

    def outs():
        return [torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, H, L), dtype=torch.float32, device="cuda")]

    def call(o, s):
        fa.fa_fwd(q, k, v, o[0], o[1], B, H, L, L, D, 1, SCALE, s)

    _replays_match(outs, call)


def test_graph_fa_fwd_splitkv():
    import torch
    q, k, v = (to_device(x) for x in make_inputs(82, B, H, 200, 3000, D, "bf16"))
    nbytes = fa.splitkv_workspace_size(B, H, 200, D, 6)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def outs():
        return [torch.empty((B, H, 200, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, H, 200), dtype=torch.float32, device="cuda")]

    def call(o, s):
        fa.fa_fwd_splitkv(q, k, v, o[0], o[1], B, H, 200, 3000, D, 0, SCALE, 6, ws, nbytes, s)

    _replays_match(outs, call)


def test_graph_fa_bwd():
    import torch
    qn, kn, vn = make_inputs(83, B, H, L, L, D, "bf16")
    q, k, v = (to_device(x) for x in (qn, kn, vn))
    do = to_device(make_grad(83, B, H, L, D))
    o = torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, B, H, L, L, D, 1, SCALE, torch.cuda.current_stream())
    nbytes = fa.bwd_workspace_size(B, H, L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def outs():
        return [torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]

    def call(g, s):
        fa.fa_bwd(q, k, v, o, lse, do, g[0], g[1], g[2], B, H, L, L, D, 1, SCALE, ws, nbytes, s)

    _replays_match(outs, call)


def test_graph_fa_fwd_fp8():
    import torch
    q8, k8, v8, ds = make_inputs_fp8(84, B, H, L, L, D)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q8, k8, v8))

    def outs():
        return [torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((B, H, L), dtype=torch.float32, device="cuda")]

    def call(o, s):
        fa.fa_fwd_fp8(q, k, v, o[0], o[1], B, H, L, L, D, 1, SCALE, *ds, s)

    _replays_match(outs, call)
