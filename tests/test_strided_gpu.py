"""GPU tests for strided [B, H, S, D] views through attn_fwd_ex / attn_bwd_ex:
[B, S, H, D] tensors, q/k/v slices of a fused [B, S, 3, H, D] projection,
rows padded with NaN, and a key/value head broadcast by a zero head stride.
Only addressing changes, so every result must equal the contiguous call's
bit for bit; one case is also checked against the fp64 oracle."""
import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL
from tests.gpu_util import compare, log, oracle, to_device
from workload import AttnConfig, make_cu_seqlens, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def _inputs(B, H, S, D, dtype, seed, H_kv=None, cu=None):
    x = make_inputs(AttnConfig("strided", B=B, H=H, S=S, D=D, dtype=dtype), seed, shape=(B, H, S, D))
    if H_kv is not None:
        x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
        x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    if cu is not None:
        x["cu_seqlens"] = cu
        x["mask_mode"] = MASK_DOC_CAUSAL
    return x


def _bshd(t, pad=0):
    """The same values as a [B, H, S, D] view of a [B, S, H, D + pad] buffer
    (padding NaN)."""
    import torch
    B, H, S, D = t.shape
    buf = torch.full((B, S, H, D + pad), float("nan"), dtype=t.dtype, device=t.device)
    view = buf.transpose(1, 2)[..., :D]
    view.copy_(t)
    return view


def _out_view(shape, dtype, pad=0):
    import torch
    B, H, S, D = shape
    buf = torch.full((B, S, H, D + pad), float("nan"), dtype=dtype, device="cuda")
    return buf.transpose(1, 2)[..., :D]


def run(x, q, k, v, do, views_out=False, out16=False, pad=0, rope=False):
    """attn_fwd_ex + attn_bwd_ex on the given input tensors (any views); outputs
    contiguous, or [B, S, H, D] views (NaN-filled) when views_out."""
    import torch
    import causal_attention_amd as ca
    B, H, S, D = x["B"], x["H"], x["S"], x["D"]
    odt = q.dtype if out16 else torch.float32
    shp = {"o": (B, H, S, D), "dq": (B, H, S, D), "dk": tuple(k.shape), "dv": tuple(k.shape)}
    if views_out:
        out = {n: _out_view(s, odt, pad) for n, s in shp.items()}
    else:
        out = {n: torch.full(s, float("nan"), dtype=odt, device="cuda") for n, s in shp.items()}
    out["lse"] = torch.full((B, H, S), float("nan"), device="cuda")
    out["delta"] = torch.full((B, H, S), float("nan"), device="cuda")
    kw = dict(mask_mode=x["mask_mode"])
    if x.get("cu_seqlens") is not None:
        kw["cu_seqlens"] = torch.from_numpy(np.asarray(x["cu_seqlens"], dtype=np.int32)).cuda()
        kw["max_seqlen"] = int(np.diff(x["cu_seqlens"]).max())
    if rope:
        kw["rope_table"] = ca.rope_table(kw.get("max_seqlen", S), D)
        kw["q_rot"] = torch.empty((B, H, S, D), dtype=q.dtype, device="cuda")
        kw["k_rot"] = torch.empty(tuple(k.shape), dtype=q.dtype, device="cuda")
    ca.attn_fwd_ex(q, k, v, out["o"], out["lse"], x["scale"], **kw)
    ca.attn_bwd_ex(q, k, v, out["o"], do, out["lse"], out["dq"], out["dk"], out["dv"], out["delta"], x["scale"],
                   **kw)
    torch.cuda.synchronize()
    return out


def same(a, b, names=("o", "lse", "dq", "dk", "dv", "delta")):
    for n in names:
        assert a[n].shape == b[n].shape, n
        assert bool((a[n] == b[n]).all()), f"{n}: strided result differs from the contiguous one"


@pytest.mark.parametrize("B,H,S,D,dtype,out16", [
    (2, 4, 300, 64, "bf16", False), (1, 2, 700, 128, "bf16", False), (3, 2, 257, 32, "bf16", False),
    (2, 4, 300, 64, "bf16", True), (2, 2, 200, 64, "f16", True), (1, 2, 333, 64, "f32", False),
    (1, 2, 190, 128, "f32", False),
])
def test_bshd_equals_contiguous(B, H, S, D, dtype, out16):
    log(f"[strided] BSHD B{B} H{H} S{S} D{D} {dtype} out16={out16}")
    x = _inputs(B, H, S, D, dtype, 600 + S + D)
    dev = to_device(x)
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"], out16=out16)
    got = run(x, *(_bshd(dev[n]) for n in ("q", "k", "v", "do")), views_out=True, out16=out16)
    same(got, ref)


def test_padded_rows_are_never_read():
    """Rows D + 32 elements apart with NaN in the gaps (inputs and outputs):
    results equal the contiguous call's, so no padding was read or written."""
    x = _inputs(2, 4, 260, 64, "bf16", 91)
    dev = to_device(x)
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"])
    got = run(x, *(_bshd(dev[n], pad=32) for n in ("q", "k", "v", "do")), views_out=True, pad=32)
    same(got, ref)


def test_fused_qkv_projection_slices():
    """q, k, v as slices of one [B, S, 3, H, D] tensor (row stride 3*H*D)."""
    import torch
    x = _inputs(2, 4, 300, 64, "bf16", 92)
    dev = to_device(x)
    B, H, S, D = 2, 4, 300, 64
    qkv = torch.empty((B, S, 3, H, D), dtype=torch.bfloat16, device="cuda")
    for i, n in enumerate(("q", "k", "v")):
        qkv[:, :, i].copy_(dev[n].transpose(1, 2))
    views = [qkv[:, :, i].transpose(1, 2) for i in range(3)]
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"])
    got = run(x, *views, dev["do"])
    same(got, ref)
    log("[strided] fused qkv: bitwise equal")


@pytest.mark.parametrize("D", [64, 128])
def test_strided_packed_documents(D):
    cu = make_cu_seqlens(900, 1, 300, 93 + D)
    x = _inputs(1, 4, int(cu[-1]), D, "bf16", 94 + D, cu=cu)
    dev = to_device(x)
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"])
    got = run(x, *(_bshd(dev[n]) for n in ("q", "k", "v", "do")), views_out=True)
    same(got, ref)


def test_strided_grouped_heads():
    x = _inputs(2, 8, 400, 64, "bf16", 95, H_kv=2)
    dev = to_device(x)
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"])
    got = run(x, *(_bshd(dev[n]) for n in ("q", "k", "v", "do")), views_out=True)
    same(got, ref)


def test_strided_with_rope():
    """RoPE reads the strided q, k and writes contiguous q_rot, k_rot."""
    x = _inputs(2, 4, 300, 64, "bf16", 96)
    dev = to_device(x)
    ref = run(x, dev["q"], dev["k"], dev["v"], dev["do"], rope=True)
    got = run(x, *(_bshd(dev[n]) for n in ("q", "k", "v", "do")), views_out=True, rope=True)
    same(got, ref)


def test_head_broadcast_by_zero_stride():
    """One key/value head expanded over all query heads (head stride 0) gives
    the forward and dQ of multi-query attention (H_kv = 1) bit for bit."""
    x = _inputs(2, 4, 300, 64, "bf16", 97, H_kv=1)
    dev = to_device(x)
    mqa = run(x, dev["q"], dev["k"], dev["v"], dev["do"])
    kx, vx = dev["k"].expand(2, 4, 300, 64), dev["v"].expand(2, 4, 300, 64)
    got = run(x, dev["q"], kx, vx, dev["do"])
    same(got, mqa, names=("o", "lse", "dq", "delta"))
    # per-head dK, dV of the broadcast call sum to the shared head's gradient
    for n in ("dk", "dv"):
        err = float((got[n].sum(dim=1, keepdim=True) - mqa[n]).abs().max())
        assert err <= 1e-4, (n, err)


def test_strided_against_oracle():
    log("[strided] BSHD B2 H4 S300 D64 bf16 vs oracle")
    x = _inputs(2, 4, 300, 64, "bf16", 98)
    dev = to_device(x)
    got = run(x, *(_bshd(dev[n]) for n in ("q", "k", "v", "do")), views_out=True)
    compare(got, oracle(x), "bf16", tag="strided BSHD")
