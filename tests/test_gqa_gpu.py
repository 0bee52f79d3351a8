"""GPU parity for grouped-query attention (attn_fwd_gqa / attn_bwd_gqa through the
C ABI) against the fp64 oracle: query head h uses K/V head h // (H / H_kv), and
dK, dV sum over each K/V head's query heads.  Same tolerances as the other parity
tests (tests/gpu_util.py)."""
import ctypes

import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL
from tests.gpu_util import compare, log, oracle, run_hip, to_device
from workload import AttnConfig, make_cu_seqlens, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def gqa_inputs(dtype, B, H, H_kv, S, D, seed, qkv_scale=1.0):
    """Seeded inputs with K and V cut to their first H_kv heads."""
    cfg = AttnConfig("gqa", B=B, H=H, S=S, D=D, dtype=dtype, qkv_scale=qkv_scale)
    x = make_inputs(cfg, seed, shape=(B, H, S, D))
    x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
    x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    return x


CASES = [
    ("bf16", 2, 8, 2, 300, 64),
    ("bf16", 1, 4, 1, 257, 64),    # multi-query: one K/V head
    ("bf16", 1, 6, 3, 130, 128),
    ("bf16", 2, 4, 4, 200, 32),    # H_kv = H through the grouped entry points' binding
    ("bf16", 1, 16, 4, 1024, 64),  # the 237M-class shape with 4 K/V heads
    ("f32", 2, 4, 2, 100, 32),
    ("f32", 1, 4, 1, 129, 128),
    ("bf16", 1, 6, 2, 300, 128),   # odd group (G = 3): dK/dV by wave pairs, three heads per key
    ("f16", 1, 9, 3, 257, 128),
    ("bf16", 2, 6, 2, 190, 64),    # odd group at D = 64: one wave per 32 keys
    # dK/dV split four ways per key group: G a multiple of four at D = 128,
    # of eight at D <= 64
    ("bf16", 1, 8, 2, 300, 128),
    ("bf16", 1, 16, 1, 200, 128),  # multi-query, 16 query heads
    ("f16", 1, 8, 1, 257, 32),
    ("bf16", 2, 16, 2, 130, 64),
]


@pytest.mark.parametrize("dtype,B,H,H_kv,S,D", CASES)
def test_gqa_parity(dtype, B, H, H_kv, S, D):
    log(f"[gqa] {dtype} B{B} H{H} H_kv{H_kv} S{S} D{D}")
    x = gqa_inputs(dtype, B, H, H_kv, S, D, 500 + H + 7 * H_kv + S)
    compare(run_hip(x), oracle(x), dtype, tag=f"gqa {dtype} B{B} H{H}/{H_kv} S{S} D{D}")


@pytest.mark.parametrize("B,H,H_kv,S", [(4, 16, 8, 2048), (16, 16, 4, 1024), (15, 4, 2, 2048), (16, 4, 2, 2048),
                                         (1, 16, 4, 2048), (1, 16, 1, 1024)])
def test_gqa_even_group_wave_pairs_sampled(B, H, H_kv, S):
    """Even groups at D = 128 with B * H_kv * ceil(S / 64) >= 1024 64-key units
    take dK/dV by wave pairs, smaller grids split the group, two ways or (G a
    multiple of four, the last two cases) four ways (the third and fourth
    cases sit on either side: 960 and 1024 units).  The oracle checks sampled
    (batch, K/V head) slices: batch entries and K/V heads are independent
    problems with G query heads each."""
    import torch
    D, G = 128, H // H_kv
    units = B * H_kv * ((S + 63) // 64)
    assert G % 2 == 0
    log(f"[gqa] even group: B{B} H{H} H_kv{H_kv} S{S} D{D}, {units} units "
        f"({'wave pairs' if units >= 1024 else 'group split'})")
    x = gqa_inputs("bf16", B, H, H_kv, S, D, 900 + B + S)
    out = run_hip(x)
    rng = np.random.default_rng(901)
    for b, j in [(0, 0), (B - 1, H_kv - 1), (int(rng.integers(B)), int(rng.integers(H_kv)))]:
        hs = slice(j * G, (j + 1) * G)
        xs = dict(x, B=1, H=G)
        for n in ("q", "do"):
            xs[n] = np.ascontiguousarray(x[n][b:b + 1, hs])
        for n in ("k", "v"):
            xs[n] = np.ascontiguousarray(x[n][b:b + 1, j:j + 1])
        got = {n: out[n][b:b + 1, hs] for n in ("o", "lse", "dq", "delta")}
        got.update({n: out[n][b:b + 1, j:j + 1] for n in ("dk", "dv")})
        assert all(bool(torch.isfinite(t).all()) for t in out.values())
        compare(got, oracle(xs), "bf16", tag=f"gqa pairs B{B} H{H}/{H_kv} S{S} slice ({b},{j})")


@pytest.mark.parametrize("D,H", [(64, 8), (64, 16), (128, 8), (128, 6)])
def test_gqa_packed_documents(D, H):
    cu = make_cu_seqlens(700, 1, 260, 41 + D)
    log(f"[gqa] packed ({len(cu) - 1} docs) D{D} H{H}/2")
    x = gqa_inputs("bf16", 1, H, 2, int(cu[-1]), D, 42 + D + H)
    x["cu_seqlens"] = cu
    x["mask_mode"] = MASK_DOC_CAUSAL
    compare(run_hip(x), oracle(x), "bf16", tag=f"gqa packed D{D} H{H}/2")


def test_gqa_bitwise_reproducible():
    x = gqa_inputs("bf16", 1, 8, 2, 513, 64, 77)
    log("[gqa] reproducibility")
    a = run_hip(x)
    b = run_hip(x)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((a[n] == b[n]).all()), n


def test_gqa_entry_points_with_equal_heads_match_plain_calls():
    """attn_fwd_gqa / attn_bwd_gqa with H_kv = H give bitwise the results of attn_fwd / attn_bwd."""
    import torch
    import causal_attention_amd as ca
    lib = ca.load_library()
    x = gqa_inputs("bf16", 1, 4, 4, 200, 64, 78)
    log("[gqa] H_kv = H through the grouped entry points")
    dev = to_device(x)
    ref = run_hip(x, dev=dev)
    B, H, S, D = 1, 4, 200, 64
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.full((B, H, S, D), float("nan"), **f32)
    lse = torch.full((B, H, S), float("nan"), **f32)
    dq, dk, dv = (torch.full((B, H, S, D), float("nan"), **f32) for _ in range(3))
    delta = torch.full((B, H, S), float("nan"), **f32)
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    assert lib.attn_fwd_gqa(p(dev["q"]), p(dev["k"]), p(dev["v"]), p(o), p(lse), B, H, H, S, D, x["scale"], 0,
                            None, 0, 0, 1, stream) == 0
    assert lib.attn_bwd_gqa(p(dev["q"]), p(dev["k"]), p(dev["v"]), p(o), p(dev["do"]), p(lse), p(dq), p(dk),
                            p(dv), p(delta), B, H, H, S, D, x["scale"], 0, None, 0, 0, 1, stream) == 0
    torch.cuda.synchronize()
    for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool((t == ref[n]).all()), n


@pytest.mark.parametrize("seed", [6, 11])
def test_gqa_full_workload(seed):
    """The 237M-class context-1024 layer with 4 K/V heads (B8 H16 S1024 D64), every output element."""
    from workload import CONFIGS
    c = CONFIGS["lm237m_ctx1024_gqa4"]
    log(f"[gqa] {c.name} seed={seed}")
    x = make_inputs(c, seed)
    compare(run_hip(x), oracle(x), "bf16", tag=f"{c.name}/{seed}")
