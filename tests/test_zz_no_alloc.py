"""attn_decode_noalloc through the C ABI: the decode step whose chunk partials
live in the library's static per-GPU scratch instead of a caller workspace
(for callers that cannot allocate).  Its results are attn_decode's, bit for
bit (same kernels, same split), and the oracle's within the 16-bit bounds;
two calls in a row, the second smaller, show that what the first left in the
shared scratch does not leak into the second; a split larger than the
scratch is refused before anything runs."""
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


def _inputs(dtype, B, H, H_kv, S_max, D, lens, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S_max, D))
    v = rng.standard_normal((B, H_kv, S_max, D))
    return dict(q=round_to(q, dtype), k=round_to(k, dtype), v=round_to(v, dtype),
                lens=np.asarray(lens, dtype=np.int32), dtype=dtype, scale=1.0 / np.sqrt(D))


def _both(x):
    """(attn_decode with a workspace, attn_decode_noalloc) outputs, NaN-poisoned first."""
    import torch
    import causal_attention_amd as ca
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x["dtype"]]
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(dt) for n in ("q", "k", "v"))
    lens = torch.from_numpy(x["lens"]).cuda()
    B, H, D = q.shape
    max_len = int(x["lens"].max())
    nbytes = ca.decode_workspace_bytes(B, H, k.shape[1], D, max_len)
    ws = torch.full((max(nbytes, 4),), 255, dtype=torch.uint8, device="cuda")
    res = []
    for noalloc in (False, True):
        o = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            ca.attn_decode_noalloc(q, k, v, lens, o, lse, x["scale"], max_len)
        else:
            ca.attn_decode(q, k, v, lens, o, lse, ws, x["scale"], max_len)
        torch.cuda.synchronize()
        res.append((o.cpu().numpy(), lse.cpu().numpy()))
    return res, nbytes


# The first call's split fills much of the scratch; the second, smaller call
# reads only what it wrote itself.
CALLS = [("bf16", 4, 32, 8, 6000, 128, [6000, 17, 4999, 3333], 1201),
         ("bf16", 2, 8, 2, 900, 64, [900, 450], 1202)]


def test_noalloc_equals_decode_on_two_calls_in_a_row():
    import causal_attention_amd as ca
    for dtype, B, H, H_kv, S_max, D, lens, seed in CALLS:
        x = _inputs(dtype, B, H, H_kv, S_max, D, lens, seed)
        log(f"[noalloc] {dtype} B{B} H{H}/{H_kv} S{S_max} D{D} lens {lens}")
        (ref, got), nbytes = _both(x)
        (ref_o, ref_lse), (o, lse) = ref, got
        assert 0 < nbytes <= ca.ATTN_DECODE_SCRATCH_BYTES, nbytes  # the split path, inside the scratch
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        assert np.array_equal(o, ref_o) and np.array_equal(lse, ref_lse)
        ro, rl = attention_decode_ref(x["q"], x["k"], x["v"], x["lens"], x["scale"])
        ma, rf = errors(o, ro)
        ml, _ = errors(lse, rl)
        log(f"[noalloc] partials {nbytes} B; o:{ma:.2e}/{rf:.1e} lse:{ml:.2e}")
        tol = TOL[dtype]
        assert ma <= tol["max_abs"] and rf <= tol["rel_fro"] and ml <= tol["lse"]


def test_noalloc_refuses_a_split_larger_than_the_scratch():
    """32 query heads on one K/V head and a 65536-key cache: the split needs
    1024 chunks x 32 heads x 129 floats, more than the scratch; the call
    returns ATTN_ERR_SCRATCH and leaves the outputs untouched."""
    import torch
    import causal_attention_amd as ca
    B, H, H_kv, S_max, D = 1, 32, 1, 65536, 128
    assert ca.decode_workspace_bytes(B, H, H_kv, D, S_max) > ca.ATTN_DECODE_SCRATCH_BYTES
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, H_kv, S_max, D), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), S_max, dtype=torch.int32, device="cuda")
    o = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(ca.AttnError, match="ATTN_ERR_SCRATCH"):
        ca.attn_decode_noalloc(q, kv, kv, lens, o, lse, 1.0 / np.sqrt(D), S_max)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all()) and bool(torch.isnan(lse).all())
