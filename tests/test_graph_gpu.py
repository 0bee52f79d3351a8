"""The entry points inside a captured HIP graph: the forward and backward of
several shapes (causal, packed documents, grouped heads, RoPE, 16-bit
outputs) are captured once and replayed three times, with other eager work
and synchronisations between the replays; every replay must reproduce the
eager results bit for bit (the kernels use no atomics, and the entry points
launch kernels only: no allocation, copy or memset is recorded)."""
import numpy as np
import pytest

from tests.gpu_util import log, to_device
from workload import AttnConfig, make_cu_seqlens, make_inputs

pytestmark = pytest.mark.gpu

NAMES = ("o", "lse", "dq", "dk", "dv", "delta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def _setup(B, H, H_kv, S, D, dtype, seed, docs, rope, out16):
    import torch
    import causal_attention_amd as ca
    x = make_inputs(AttnConfig("graph", B=B, H=H, S=S, D=D, dtype=dtype), seed, shape=(B, H, S, D))
    x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
    x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    dev = to_device(x)
    odt = dev["q"].dtype if out16 else torch.float32
    out = {"o": torch.empty((B, H, S, D), dtype=odt, device="cuda"),
           "dq": torch.empty((B, H, S, D), dtype=odt, device="cuda"),
           "dk": torch.empty((B, H_kv, S, D), dtype=odt, device="cuda"),
           "dv": torch.empty((B, H_kv, S, D), dtype=odt, device="cuda"),
           "lse": torch.empty((B, H, S), device="cuda"), "delta": torch.empty((B, H, S), device="cuda")}
    kw = {}
    if docs:
        cu = make_cu_seqlens(S, 1, 200, seed)
        kw.update(mask_mode=1, cu_seqlens=torch.from_numpy(cu).cuda(), max_seqlen=int(np.diff(cu).max()))
    if rope:
        kw["rope_table"] = ca.rope_table(kw.get("max_seqlen", S), D)
        kw["q_rot"] = torch.empty_like(dev["q"])
        kw["k_rot"] = torch.empty_like(dev["k"])
    scale = D ** -0.5

    def step(stream):
        ca.attn_fwd_ex(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], scale, stream=stream, **kw)
        ca.attn_bwd_ex(dev["q"], dev["k"], dev["v"], out["o"], dev["do"], out["lse"], out["dq"], out["dk"],
                       out["dv"], out["delta"], scale, stream=stream, **kw)
    return out, step


@pytest.mark.parametrize("B,H,H_kv,S,D,dtype,docs,rope,out16", [
    (2, 4, 4, 300, 64, "bf16", False, False, False),
    (1, 4, 4, 700, 128, "bf16", True, False, False),
    (1, 8, 2, 257, 64, "bf16", False, False, False),
    (1, 6, 2, 333, 128, "bf16", False, True, False),
    (2, 4, 4, 190, 64, "bf16", False, False, True),
    (1, 2, 2, 129, 64, "f32", False, False, False),
])
def test_graph_replays_match_eager(B, H, H_kv, S, D, dtype, docs, rope, out16):
    import torch
    log(f"[graph] B{B} H{H}/{H_kv} S{S} D{D} {dtype} docs={docs} rope={rope} out16={out16}")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    out, step = _setup(B, H, H_kv, S, D, dtype, 70 + S, docs, rope, out16)
    step(s)
    torch.cuda.synchronize()
    ref = {n: out[n].clone() for n in NAMES}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    other_out, other_step = _setup(1, 2, 2, 200, 64, "bf16", 5, False, False, False)
    for rep in range(3):
        for n in NAMES:  # poison outside the graph, then unrelated eager work
            out[n].fill_(float("nan"))
        other_step(None)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for n in NAMES:
            assert bool((out[n] == ref[n]).all()), f"replay {rep}: {n} differs from the eager result"
    log("[graph] three replays bitwise equal to eager")


def test_graph_replays_with_the_grouped_workspace():
    """attn_bwd_gqa_ws inside a graph: the parts kernels and their sum (B1
    H8/2 S600 D128, four parts) captured once, replayed three times with the
    outputs and the workspace poisoned in between; every replay equals the
    eager step."""
    import torch
    import causal_attention_amd as ca
    B, H, H_kv, S, D = 1, 8, 2, 600, 128
    log(f"[graph] workspace path B{B} H{H}/{H_kv} S{S} D{D}")
    x = make_inputs(AttnConfig("graph", B=B, H=H, S=S, D=D, dtype="bf16"), 81, shape=(B, H, S, D))
    x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
    x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    dev = to_device(x)
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"o": torch.empty((B, H, S, D), **f32), "dq": torch.empty((B, H, S, D), **f32),
           "dk": torch.empty((B, H_kv, S, D), **f32), "dv": torch.empty((B, H_kv, S, D), **f32),
           "lse": torch.empty((B, H, S), **f32), "delta": torch.empty((B, H, S), **f32)}
    n = ca.bwd_workspace_bytes(B, H, H_kv, S, D, torch.bfloat16)
    assert n == 2 * 4 * B * H_kv * S * D * 4
    ws = torch.empty(n // 4, **f32)
    scale = D ** -0.5

    def step(stream):
        ca.attn_fwd(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], scale, stream=stream)
        ca.attn_bwd(dev["q"], dev["k"], dev["v"], out["o"], dev["do"], out["lse"], out["dq"], out["dk"], out["dv"],
                    out["delta"], scale, stream=stream, workspace=ws)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    step(s)
    torch.cuda.synchronize()
    ref = {k: out[k].clone() for k in NAMES}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    other_out, other_step = _setup(1, 2, 2, 200, 64, "bf16", 5, False, False, False)
    for rep in range(3):
        for k in NAMES:
            out[k].fill_(float("nan"))
        ws.fill_(float("nan"))
        other_step(None)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for k in NAMES:
            assert bool((out[k] == ref[k]).all()), f"replay {rep}: {k} differs from the eager result"
    log("[graph] three replays of the workspace path bitwise equal to eager")
