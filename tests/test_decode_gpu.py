"""GPU parity for the decode step against a K/V cache (attn_decode through the C ABI)
against the fp64 oracle (attention_decode_ref): one query per (batch entry, head)
attending the first cache_lens[b] keys of its K/V head.  Covers grouped heads
(up to 32 query heads per K/V head), per-entry lengths from 1 to S_max, lengths
that are not a multiple of the 32-key tile, the single-chunk path (no workspace)
and the split path with its exact merge.  Tolerances as tests/gpu_util.py."""
import numpy as np
import pytest

from oracle import attention_decode_ref
from tests.gpu_util import TOL, errors, log
from workload import round_to

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def decode_inputs(dtype, B, H, H_kv, S_max, D, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S_max, D))
    v = rng.standard_normal((B, H_kv, S_max, D))
    return dict(q=round_to(q, dtype), k=round_to(k, dtype), v=round_to(v, dtype), lens=np.asarray(lens, dtype=np.int32), dtype=dtype,
                scale=1.0 / np.sqrt(D))


def run_decode(x):
    import torch
    import causal_attention_amd as ca
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x["dtype"]]
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(dt) for n in ("q", "k", "v"))
    lens = torch.from_numpy(x["lens"]).cuda()
    B, H, D = q.shape
    o = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    n = ca.decode_workspace_bytes(B, H, k.shape[1], D, int(x["lens"].max()))
    ws = torch.full((max(n, 4),), 255, dtype=torch.uint8, device="cuda") if n else None
    ca.attn_decode(q, k, v, lens, o, lse, ws, x["scale"], int(x["lens"].max()))
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy(), n


def check(x, tag):
    o, lse, n = run_decode(x)
    ro, rlse = attention_decode_ref(x["q"], x["k"], x["v"], x["lens"], x["scale"])
    tol = TOL[x["dtype"]]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{tag}: unwritten or non-finite outputs"
    ma, rf = errors(o, ro)
    ml, _ = errors(lse, rlse)
    log(f"[decode] {tag} workspace={n} o:{ma:.2e}/{rf:.1e} lse:{ml:.2e}")
    assert ma <= tol["max_abs"], f"{tag}: O max-abs {ma:.3e}"
    if tol["rel_fro"] is not None:
        assert rf <= tol["rel_fro"], f"{tag}: O rel-Frobenius {rf:.3e}"
    assert ml <= tol["lse"], f"{tag}: LSE max-abs {ml:.3e}"
    return n


CASES = [
    ("bf16", 2, 8, 2, 1000, 64, [1000, 37]),
    ("bf16", 3, 16, 16, 300, 128, [1, 300, 33]),
    ("bf16", 1, 32, 1, 4096, 64, [4095]),               # 32 query heads on one K/V head
    ("bf16", 4, 16, 4, 8192, 128, [8192, 5000, 1, 8191]),
    ("bf16", 2, 4, 4, 777, 32, [777, 400]),
    ("f32", 2, 4, 1, 257, 64, [257, 256]),
    ("f32", 1, 8, 2, 100, 128, [65]),
    ("f16", 2, 8, 2, 1500, 128, [1500, 700]),
    ("f16", 1, 4, 4, 300, 64, [300]),
]


@pytest.mark.parametrize("dtype,B,H,H_kv,S_max,D,lens", CASES)
def test_decode_parity(dtype, B, H, H_kv, S_max, D, lens):
    x = decode_inputs(dtype, B, H, H_kv, S_max, D, lens, 900 + H + S_max)
    check(x, f"{dtype} B{B} H{H}/{H_kv} S{S_max} D{D}")


def test_decode_single_chunk_path():
    """1024 (batch entry, K/V head) pairs and a short cache: one chunk each, no workspace."""
    x = decode_inputs("bf16", 64, 16, 16, 64, 64, list(range(1, 65)), 950)
    assert check(x, "single chunk") == 0


def test_decode_split_path_uses_workspace():
    x = decode_inputs("bf16", 1, 8, 8, 2048, 64, [2048], 951)
    assert check(x, "split") > 0


def test_decode_bitwise_reproducible():
    x = decode_inputs("bf16", 2, 16, 4, 3000, 128, [3000, 1234], 952)
    log("[decode] reproducibility")
    a = run_decode(x)
    b = run_decode(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
