"""The library works when it is loaded before torch is imported (a fresh
process loads the package, then torch, then launches on torch's stream)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import exact_io_aware_08_amd as fa
fa.load_library()
import numpy as np
import torch
from seeded_inputs import make_inputs
q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
           for x in make_inputs(3, 1, 2, 200, 200, 64, "bf16"))
o = torch.empty_like(q)
lse = torch.empty((1, 2, 200), device="cuda")
fa.fa_fwd(q, k, v, o, lse, 1, 2, 200, 200, 64, 1, 0.125, torch.cuda.current_stream())
torch.cuda.synchronize()
assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
print("load-order ok")
"""


def test_library_loaded_before_torch():
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "load-order ok" in r.stdout, r.stderr[-2000:]
