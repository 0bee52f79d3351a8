"""The README's Python example runs as written and its outputs agree with the
fp64 oracle on sampled heads (the example is part of the package's surface:
this catches drift between the binding and what the README shows)."""
import os
import re

import numpy as np
import pytest

from tests.gpu_util import compare, log, oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def _readme_python():
    with open(os.path.join(ROOT, "README.md")) as f:
        text = f.read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "the README holds one Python example"
    return blocks[0]


def test_readme_example_runs_and_matches_the_oracle():
    import torch
    env = {}
    torch.manual_seed(0)
    exec(compile(_readme_python(), "README.md", "exec"), env)
    torch.cuda.synchronize()
    q, k, v, do = env["q"], env["k"], env["v"], env["do"]
    x = {n: t.float().cpu().numpy() for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    x.update(scale=env["scale"], mask_mode=0)
    heads = [(0, 0), (7, 15), (3, 5)]
    log("[readme] example: forward / backward against the oracle on sampled heads")
    got = {"o": env["o"], "lse": env["lse"], "dq": env["dq"], "dk": env["dk"], "dv": env["dv"],
           "delta": env["delta"]}
    compare(got, oracle(x, heads=heads), "bf16", heads=heads, tag="readme")
    # the options call (grouped heads, RoPE, 16-bit O in a [B, S, H, D] view)
    # on sampled heads: the oracle's RoPE path, K/V heads of each group cut out
    from oracle import attention_rope_ref
    xq = env["xq"].transpose(1, 2).float().cpu().numpy()
    xkv = env["xkv"].transpose(1, 2).float().cpu().numpy()
    G = xq.shape[1] // xkv.shape[1]
    for b, h in heads:
        ref = attention_rope_ref(xq[b:b + 1, h:h + 1], xkv[b:b + 1, h // G:h // G + 1],
                                 xkv[b:b + 1, h // G:h // G + 1], np.zeros_like(xq[b:b + 1, h:h + 1]),
                                 env["scale"], 0, None, dtype="bf16")
        got = {"o": env["o16"][b:b + 1, h:h + 1], "lse": env["lse16"][b:b + 1, h:h + 1]}
        compare(got, ref, "bf16", names=("o", "lse"), out16="bf16", tag=f"readme options ({b},{h})")
