"""GPU parity for RoPE (attn_rope_table, attn_rope, attn_fwd_rope,
attn_bwd_rope) against the fp64 oracle (oracle/rope.py): the table, the
rotated q and k, and forward + backward with the gradients turned back to the
unrotated inputs, causal and packed documents, grouped K/V heads, every
input dtype.  Attention outputs use the same bounds as without RoPE."""
import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL, attention_rope_ref, rope_angles, rope_positions, rope_rotate, round_to_dtype
from tests.gpu_util import compare, log, to_device
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
    x = make_inputs(AttnConfig("rope", B=B, H=H, S=S, D=D, dtype=dtype), seed, shape=(B, H, S, D))
    if H_kv is not None:
        x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
        x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    if cu is not None:
        x["cu_seqlens"] = cu
        x["mask_mode"] = MASK_DOC_CAUSAL
    return x


def run_rope(x, base=10000.0, extra_pos=0):
    import torch
    import causal_attention_amd as ca
    dev = to_device(x)
    B, H, S, D = x["B"], x["H"], x["S"], x["D"]
    n_pos = (dev["max_seqlen"] or S) + extra_pos
    tab = ca.rope_table(n_pos, D, base)
    nan = float("nan")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {n: torch.full((B, H, S, D), nan, **f32) for n in ("o", "dq")}
    for n in ("dk", "dv"):
        out[n] = torch.full(tuple(x["k"].shape), nan, **f32)
    out["lse"] = torch.full((B, H, S), nan, **f32)
    out["delta"] = torch.full((B, H, S), nan, **f32)
    q_rot = torch.full_like(dev["q"], nan)
    k_rot = torch.full_like(dev["k"], nan)
    mode = x["mask_mode"]
    ca.attn_fwd_rope(dev["q"], dev["k"], dev["v"], q_rot, k_rot, out["o"], out["lse"], tab, x["scale"], mode,
                     dev["cu"], None, dev["max_seqlen"])
    ca.attn_bwd_rope(q_rot, k_rot, dev["v"], out["o"], dev["do"], out["lse"], out["dq"], out["dk"], out["dv"],
                     out["delta"], tab, x["scale"], mode, dev["cu"], None, dev["max_seqlen"])
    torch.cuda.synchronize()
    out["q_rot"], out["k_rot"], out["tab"], out["dev"] = q_rot, k_rot, tab, dev
    return out


def rope_oracle(x, base=10000.0):
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "do")]
    return attention_rope_ref(*args, x["scale"], x["mask_mode"], x.get("cu_seqlens"), base, dtype=x["dtype"])


# relative spacing of representable values (one unit in the last place, relative)
_REL_ULP = {"bf16": 2.0 ** -7, "f16": 2.0 ** -10, "f32": 2.0 ** -23}


def check_rotated(got, ref, x, dtype, tag):
    """The kernel rotates in fp32 and rounds once; the oracle rotates in fp64 and
    rounds once.  The fp32 rotation is off by a few fp32 rounding errors of the
    pair's magnitude |(x_2i, x_2i+1)| (not of the result, which can cancel to
    near zero), so a 16-bit result may land one unit in the last place away
    where the exact value sits that close to a rounding boundary; such
    elements must be rare: at most one in a thousand, plus two (a tiny input
    of a few hundred elements can hold one by chance)."""
    g = got.float().cpu().numpy().astype(np.float64)
    d = np.abs(g - ref)
    x = np.asarray(x, dtype=np.float64)
    pair = np.repeat(np.hypot(x[..., 0::2], x[..., 1::2]), 2, axis=-1)
    fp32_err = 6 * 2.0 ** -24 * pair  # table, two products, one sum, and the oracle's own fp32 rounding
    if dtype == "f32":
        assert np.all(d <= fp32_err), f"{tag}: max excess {float(np.max(d - fp32_err)):.2e}"
        return
    assert np.all(d <= _REL_ULP[dtype] * np.abs(ref) + 2 * fp32_err), f"{tag}: more than one unit in the last place"
    n_diff = int(np.count_nonzero(d > 0))
    frac = n_diff / max(d.size, 1)
    assert n_diff <= 1e-3 * d.size + 2, f"{tag}: {n_diff} of {d.size} elements differ"
    log(f"{tag}: {frac:.1e} of elements one ulp apart")


@pytest.mark.parametrize("D,base", [(32, 10000.0), (64, 10000.0), (128, 500000.0)])
def test_table(D, base):
    import causal_attention_amd as ca
    n_pos = 8192
    tab = ca.rope_table(n_pos, D, base).cpu().numpy().astype(np.float64)
    ang = rope_angles(n_pos, D, base)
    assert np.max(np.abs(tab[..., 0] - np.cos(ang))) <= 1e-7
    assert np.max(np.abs(tab[..., 1] - np.sin(ang))) <= 1e-7


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rotation_matches_oracle(dtype):
    import torch
    import causal_attention_amd as ca
    x = _inputs(2, 4, 333, 64, dtype, 70, H_kv=2)
    dev = to_device(x)
    tab = ca.rope_table(333, 64)
    q_rot, k_rot = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
    ca.attn_rope(dev["q"], dev["k"], q_rot, k_rot, tab)
    torch.cuda.synchronize()
    pos = np.arange(333)
    check_rotated(q_rot, round_to_dtype(rope_rotate(x["q"], pos), dtype), x["q"], dtype, f"q_rot {dtype}")
    check_rotated(k_rot, round_to_dtype(rope_rotate(x["k"], pos), dtype), x["k"], dtype, f"k_rot {dtype}")
    # in place gives the same values
    q2, k2 = dev["q"].clone(), dev["k"].clone()
    ca.attn_rope(q2, k2, q2, k2, tab)
    torch.cuda.synchronize()
    assert torch.equal(q2, q_rot) and torch.equal(k2, k_rot)


def test_rotation_positions_restart_per_document():
    import torch
    import causal_attention_amd as ca
    cu = make_cu_seqlens(700, 1, 300, 71)
    x = _inputs(1, 2, int(cu[-1]), 64, "bf16", 72, cu=cu)
    dev = to_device(x)
    tab = ca.rope_table(dev["max_seqlen"], 64)
    q_rot, k_rot = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
    ca.attn_rope(dev["q"], dev["k"], q_rot, k_rot, tab, MASK_DOC_CAUSAL, dev["cu"], None, dev["max_seqlen"])
    torch.cuda.synchronize()
    pos = rope_positions(x["S"], MASK_DOC_CAUSAL, cu)
    check_rotated(q_rot, round_to_dtype(rope_rotate(x["q"], pos), "bf16"), x["q"], "bf16", "q_rot docs")


def test_rope_empty_documents_change_nothing():
    """RoPE positions restart per document; empty documents (first, in between,
    last) own no rows and must not shift them: parity with the oracle, and
    bitwise the outputs of the same call without the empty documents."""
    cu = np.array([0, 1, 97, 98, 260, 300], dtype=np.int32)
    cu_e = np.array([0, 0, 1, 97, 97, 97, 98, 260, 300, 300], dtype=np.int32)
    log("[rope] empty documents bf16 D128 G=3")
    x = _inputs(1, 3, 300, 128, "bf16", 81, H_kv=1, cu=cu_e)
    out = run_rope(x)
    compare(out, rope_oracle(x), "bf16", tag="rope empty docs")
    y = dict(x)
    y["cu_seqlens"] = cu
    ref = run_rope(y)
    for n in ("o", "lse", "dq", "dk", "dv", "delta", "q_rot", "k_rot"):
        assert bool((out[n] == ref[n]).all()), n


@pytest.mark.parametrize("B,H,S,D,dtype", [
    (2, 4, 300, 64, "bf16"), (1, 2, 1000, 128, "bf16"), (3, 2, 257, 32, "bf16"), (1, 1, 1, 64, "bf16"),
    (2, 2, 257, 64, "f16"), (1, 3, 130, 32, "f32"), (1, 2, 333, 128, "f32"), (2, 2, 190, 64, "f32"),
])
def test_rope_parity(B, H, S, D, dtype):
    log(f"[rope] B{B} H{H} S{S} D{D} {dtype}")
    x = _inputs(B, H, S, D, dtype, 400 + S + D)
    out = run_rope(x, extra_pos=37)
    ref = rope_oracle(x)
    compare(out, ref, dtype, tag=f"rope B{B} H{H} S{S} D{D} {dtype}")
    check_rotated(out["q_rot"], ref["q_rot"], x["q"], dtype, "q_rot")


def test_rope_full_ctx1024_shape():
    """The 237M-class layer shape (B8 H16 S1024 D64, bf16) with RoPE, every output element."""
    log("[rope] B8 H16 S1024 D64 bf16")
    x = _inputs(8, 16, 1024, 64, "bf16", 3)
    compare(run_rope(x), rope_oracle(x), "bf16", tag="rope ctx1024")


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32")])
def test_rope_packed_documents(D, dtype):
    cu = make_cu_seqlens(900, 1, 300, 73 + D)
    log(f"[rope] packed ({len(cu) - 1} docs) D{D} {dtype}")
    x = _inputs(1, 4, int(cu[-1]), D, dtype, 74 + D, cu=cu)
    compare(run_rope(x), rope_oracle(x), dtype, tag=f"rope packed D{D} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_grouped_heads(dtype):
    log(f"[rope] B2 H8 H_kv2 S400 D64 {dtype}")
    x = _inputs(2, 8, 400, 64, dtype, 75, H_kv=2)
    compare(run_rope(x), rope_oracle(x), dtype, tag=f"rope gqa {dtype}")


def test_rope_backward_is_plain_backward_turned_back():
    """attn_bwd_rope = attn_bwd on the rotated inputs with dq, dk turned back:
    dv and delta bitwise equal, dq and dk equal to the host-side inverse
    rotation of the plain gradients (fp32 rounding)."""
    import torch
    import causal_attention_amd as ca
    x = _inputs(1, 4, 520, 64, "bf16", 76)
    out = run_rope(x)
    dev = out["dev"]
    plain = ca.backward(out["q_rot"], out["k_rot"], dev["v"], out["o"], dev["do"], out["lse"], x["scale"])
    torch.cuda.synchronize()
    assert torch.equal(plain[2], out["dv"]) and torch.equal(plain[3], out["delta"])
    pos = np.arange(520)
    for got, g in ((out["dq"], plain[0]), (out["dk"], plain[1])):
        want = rope_rotate(g.cpu().numpy().astype(np.float64), pos, inverse=True)
        err = np.max(np.abs(got.cpu().numpy() - want))
        assert err <= 1e-5 * max(1.0, float(np.max(np.abs(want)))), err


def test_rope_bitwise_reproducible():
    import torch
    x = _inputs(1, 4, 513, 64, "bf16", 77)
    log("[rope] reproducibility")
    a = run_rope(x)
    b = run_rope(x)
    for n in ("o", "lse", "dq", "dk", "dv", "q_rot", "k_rot"):
        assert torch.equal(a[n], b[n]), n
