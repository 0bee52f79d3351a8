"""The library loaded before anything in the process touches the GPU still
launches its kernels (load_library brings the device runtime up first).  Runs
in a fresh interpreter: the test process itself has already used the GPU."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = r"""
import sys
sys.path.insert(0, sys.argv[1])
import causal_attention_amd as ca
ca.load_library()                      # first: before any torch GPU work
import torch
q = torch.randn(1, 2, 300, 64, device="cuda").to(torch.bfloat16)
o, lse = ca.forward(q, q, q, 0.125)
dq, dk, dv, _ = ca.backward(q, q, q, o, q, lse, 0.125)
torch.cuda.synchronize()
assert all(bool(torch.isfinite(t).all()) for t in (o, lse, dq, dk, dv))
print("load order ok", flush=True)
"""


def test_library_loaded_before_the_device_runtime():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, "-c", CODE, ROOT], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and "load order ok" in r.stdout, r.stdout + r.stderr
