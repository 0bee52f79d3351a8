"""GPU parity for 16-bit outputs (attn_fwd_ex / attn_bwd_ex with out_dtype =
the input dtype): O, dQ, dK, dV stored in bf16 (or fp16), rounded once at the
store.  Against the fp64 oracle each element may be off by the fp32-output
bound plus its own rounding (half a unit in the last place); against the
fp32-output kernels, O and dV (which do not depend on Delta) are those
results rounded, bit for bit, and LSE is unchanged.  dQ and dK see Delta
computed from the stored 16-bit O."""
import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL, attention_rope_ref
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
    x = make_inputs(AttnConfig("out16", B=B, H=H, S=S, D=D, dtype=dtype), seed, shape=(B, H, S, D))
    if H_kv is not None:
        x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
        x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    if cu is not None:
        x["cu_seqlens"] = cu
        x["mask_mode"] = MASK_DOC_CAUSAL
    return x


def run_ex(x, out_fp32=False, rope=False):
    """attn_fwd_ex + attn_bwd_ex; outputs in the input dtype unless out_fp32."""
    import torch
    import causal_attention_amd as ca
    dev = to_device(x)
    B, H, S, D = x["B"], x["H"], x["S"], x["D"]
    odt = torch.float32 if out_fp32 else dev["q"].dtype
    nan = float("nan")
    out = {n: torch.full((B, H, S, D), nan, dtype=odt, device="cuda") for n in ("o", "dq")}
    for n in ("dk", "dv"):
        out[n] = torch.full(tuple(x["k"].shape), nan, dtype=odt, device="cuda")
    out["lse"] = torch.full((B, H, S), nan, dtype=torch.float32, device="cuda")
    out["delta"] = torch.full((B, H, S), nan, dtype=torch.float32, device="cuda")
    kw = dict(mask_mode=x["mask_mode"], cu_seqlens=dev["cu"], max_seqlen=dev["max_seqlen"])
    if rope:
        kw["rope_table"] = ca.rope_table(dev["max_seqlen"] or S, D)
        kw["q_rot"], kw["k_rot"] = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
    ca.attn_fwd_ex(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], x["scale"], **kw)
    ca.attn_bwd_ex(dev["q"], dev["k"], dev["v"], out["o"], dev["do"], out["lse"], out["dq"], out["dk"], out["dv"],
                   out["delta"], x["scale"], **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,H,S,D,dtype", [
    (2, 4, 300, 64, "bf16"), (1, 2, 1000, 128, "bf16"), (3, 2, 257, 32, "bf16"), (1, 1, 1, 64, "bf16"),
    (2, 2, 257, 64, "f16"), (1, 2, 700, 128, "f16"),
])
def test_out16_parity(B, H, S, D, dtype):
    log(f"[out16] B{B} H{H} S{S} D{D} {dtype}")
    x = _inputs(B, H, S, D, dtype, 500 + S + D)
    compare(run_ex(x), oracle(x), dtype, out16=dtype, tag=f"out16 B{B} H{H} S{S} D{D} {dtype}")


@pytest.mark.parametrize("dtype,seed", [("bf16", 3), ("bf16", 11), ("f16", 3)])
def test_out16_full_ctx1024_shape(dtype, seed):
    """The 237M-class layer shape (B8 H16 S1024 D64), every output element."""
    log(f"[out16] B8 H16 S1024 D64 {dtype} seed {seed}")
    x = _inputs(8, 16, 1024, 64, dtype, seed)
    compare(run_ex(x), oracle(x), dtype, out16=dtype, tag=f"out16 ctx1024 {dtype} seed {seed}")


@pytest.mark.parametrize("D", [64, 128])
def test_out16_packed_documents(D):
    cu = make_cu_seqlens(900, 1, 300, 81 + D)
    log(f"[out16] packed ({len(cu) - 1} docs) D{D}")
    x = _inputs(1, 4, int(cu[-1]), D, "bf16", 82 + D, cu=cu)
    compare(run_ex(x), oracle(x), "bf16", out16="bf16", tag=f"out16 packed D{D}")


def test_out16_grouped_heads():
    log("[out16] B2 H8 H_kv2 S400 D64")
    x = _inputs(2, 8, 400, 64, "bf16", 83, H_kv=2)
    compare(run_ex(x), oracle(x), "bf16", out16="bf16", tag="out16 gqa")


def test_out16_with_rope():
    log("[out16] RoPE B2 H4 S300 D64")
    x = _inputs(2, 4, 300, 64, "bf16", 84)
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "do")]
    ref = attention_rope_ref(*args, x["scale"], dtype="bf16")
    compare(run_ex(x, rope=True), ref, "bf16", out16="bf16", tag="out16 rope")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_out16_is_fp32_output_rounded(dtype):
    """O and dV: the 16-bit outputs are the fp32-output kernels' values rounded
    to nearest even (same arithmetic, one rounding at the store); LSE equal."""
    import torch
    x = _inputs(2, 4, 333, 64, dtype, 85)
    a = run_ex(x)
    b = run_ex(x, out_fp32=True)
    for n in ("o", "dv"):
        assert torch.equal(a[n], b[n].to(a[n].dtype)), n
    assert torch.equal(a["lse"], b["lse"])


def test_out16_bitwise_reproducible():
    import torch
    x = _inputs(1, 4, 513, 64, "bf16", 86)
    a = run_ex(x)
    b = run_ex(x)
    for n in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert torch.equal(a[n], b[n]), n
