"""Seeded random combinations of every option of attn_fwd_ex / attn_bwd_ex
(input dtype, D, causal or packed documents, grouped K/V heads, RoPE, 16-bit
outputs, [B, S, H, D] views, empty documents among packed ones) against
the fp64 oracle, at sizes the oracle finishes quickly.  The cases are drawn
once from a fixed seed, so a failure names a reproducible case.  16-bit
cases are bounded by the fixed bounds or by twice the 16-bit rounding
model's error on the same input, whichever is larger.  With RoPE the
rotated q, k are checked against the oracle's rotation (one rounding apart
at most, rarely) and attention against the oracle on those rotated values:
a last-bit difference in a rotated element moves the scores by up to
|k| scale ulp, which at unit-scale inputs can pass the fixed LSE bound on
its own."""
import numpy as np
import pytest

from oracle import MASK_CAUSAL, MASK_DOC_CAUSAL, attention_bwd_ref, attention_rope_ref
from oracle.rope import rope_positions, rope_rotate
from tests.bf16_model import attention_model
from tests.gpu_util import TOL, compare, half_ulp, log
from tests.test_rope_gpu import check_rotated

pytestmark = pytest.mark.gpu


def _draw_cases(n=96, seed=2026, groups=(1, 2, 4), kv_heads=(1, 2, 3), first_id=0):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(first_id, first_id + n):
        dtype = str(rng.choice(["bf16", "bf16", "f16", "f32"]))
        D = int(rng.choice([32, 64, 128]))
        H_kv = int(rng.choice(list(kv_heads)))
        G = int(rng.choice(list(groups)))
        doc = bool(rng.random() < 0.35)
        B = 1 if doc else int(rng.integers(1, 4))
        if doc:
            lens = rng.integers(1, 160, size=int(rng.integers(1, 5)))
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            S = int(cu[-1])
            if i % 3 == 0:  # empty documents (repeated boundaries), from a stream of their own
                er = np.random.default_rng(seed + i)
                for _ in range(int(er.integers(1, 4))):
                    j = int(er.integers(0, len(cu)))
                    cu = np.insert(cu, j, cu[j])
        else:
            cu = None
            S = int(rng.integers(1, 330))
        cases.append(dict(id=i, dtype=dtype, D=D, H_kv=H_kv, H=H_kv * G, B=B, S=S, cu=cu,
                          rope=bool(rng.random() < 0.4), out16=dtype != "f32" and bool(rng.random() < 0.4),
                          strided=bool(rng.random() < 0.5), seed=int(rng.integers(1 << 30))))
    return cases


# 96 mixes of every option, plus 32 with groups of 8 and 16 query heads per
# K/V head (the four-way dK/dV split at every head dimension)
CASES = _draw_cases() + _draw_cases(32, 2027, groups=(8, 16), kv_heads=(1, 2), first_id=96)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def _round(x, dtype):
    import torch
    t = torch.from_numpy(x.astype(np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    return t.to(torch.float64).numpy()


def _view(t, strided):
    """t itself, or the same values as a [B, H, S, D] view of a [B, S, H, D + 8]
    buffer (padding NaN)."""
    import torch
    if not strided:
        return t
    B, H, S, D = t.shape
    buf = torch.full((B, S, H, D + 8), float("nan"), dtype=t.dtype, device=t.device)
    v = buf.transpose(1, 2)[..., :D]
    v.copy_(t)
    return v


def _parts(c):
    """The workspace split the library takes for this mix (0: none): 16-bit
    inputs, a group G even at D = 128 or >= 8 below, fewer than 1024 dK/dV
    workgroups (64 keys each at D = 128, 128 below); P the smallest divisor
    of G that brings them to 1024, else G."""
    G = c["H"] // c["H_kv"]
    if c["dtype"] == "f32" or (G % 2 if c["D"] == 128 else G < 8):
        return 0
    bn = 64 if c["D"] == 128 else 128
    if c["cu"] is not None:
        units = (len(c["cu"]) - 1) * c["H_kv"] * -(-int(np.diff(c["cu"]).max()) // bn)
    else:
        units = c["B"] * c["H_kv"] * -(-c["S"] // bn)
    if units >= 1024:
        return 0
    return next((p for p in range(2, G) if G % p == 0 and units * p >= 1024), G)


# the mixes whose grouped heads split their dK/dV step when given a workspace
WS_CASES = [c for c in CASES if _parts(c)]


@pytest.mark.parametrize("case", CASES, ids=[f"c{c['id']}" for c in CASES])
def test_random_option_mix(case):
    _run_case(case, with_ws=False)


@pytest.mark.parametrize("case", WS_CASES, ids=[f"c{c['id']}" for c in WS_CASES])
def test_random_option_mix_with_workspace(case):
    """The same mix through attn_bwd_ex with a (NaN-filled) workspace: the
    grouped heads' dK/dV in parts, summed in order, stored in the output type
    through the output strides, turned back by RoPE in each part."""
    _run_case(case, with_ws=True)


def _run_case(case, with_ws):
    import torch
    import causal_attention_amd as ca
    c = case
    log(f"[random{' ws' if with_ws else ''}] {c}")
    rng = np.random.default_rng(c["seed"])
    B, H, H_kv, S, D = c["B"], c["H"], c["H_kv"], c["S"], c["D"]
    # float32 draws rounded to the input dtype: the oracle sees exactly the kernel's inputs
    x = {n: _round(rng.standard_normal(shape), c["dtype"])
         for n, shape in (("q", (B, H, S, D)), ("k", (B, H_kv, S, D)), ("v", (B, H_kv, S, D)),
                          ("do", (B, H, S, D)))}
    scale = 1.0 / np.sqrt(D)
    mode = MASK_DOC_CAUSAL if c["cu"] is not None else MASK_CAUSAL
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[c["dtype"]]
    dev = {n: torch.from_numpy(x[n]).to("cuda").to(tdt) for n in x}
    odt = tdt if c["out16"] else torch.float32
    nan = float("nan")
    out = {"o": _view(torch.full((B, H, S, D), nan, dtype=odt, device="cuda"), c["strided"]),
           "dq": _view(torch.full((B, H, S, D), nan, dtype=odt, device="cuda"), c["strided"]),
           "dk": _view(torch.full((B, H_kv, S, D), nan, dtype=odt, device="cuda"), c["strided"]),
           "dv": _view(torch.full((B, H_kv, S, D), nan, dtype=odt, device="cuda"), c["strided"]),
           "lse": torch.full((B, H, S), nan, device="cuda"), "delta": torch.full((B, H, S), nan, device="cuda")}
    q, k, v, do = (_view(dev[n], c["strided"]) for n in ("q", "k", "v", "do"))
    kw = dict(mask_mode=mode)
    if c["cu"] is not None:
        kw["cu_seqlens"] = torch.from_numpy(c["cu"]).cuda()
        kw["max_seqlen"] = int(np.diff(c["cu"]).max())
    if c["rope"]:
        kw["rope_table"] = ca.rope_table(kw.get("max_seqlen", S), D)
        kw["q_rot"] = torch.empty((B, H, S, D), dtype=tdt, device="cuda")
        kw["k_rot"] = torch.empty((B, H_kv, S, D), dtype=tdt, device="cuda")
    ws = None
    if with_ws:
        n_seqs = len(c["cu"]) - 1 if c["cu"] is not None else 0
        n = ca.bwd_workspace_bytes(B, H, H_kv, S, D, tdt, mode, n_seqs, kw.get("max_seqlen", 0))
        assert n == 2 * _parts(c) * B * H_kv * S * D * 4, n
        ws = torch.full((n // 4,), nan, dtype=torch.float32, device="cuda")
    ca.attn_fwd_ex(q, k, v, out["o"], out["lse"], scale, **kw)
    ca.attn_bwd_ex(q, k, v, out["o"], do, out["lse"], out["dq"], out["dk"], out["dv"], out["delta"], scale,
                   workspace=ws, **kw)
    torch.cuda.synchronize()
    if c["rope"]:
        # the rotation against the oracle's (one rounding apart at most,
        # rarely), then attention against the oracle on the rotated values the
        # kernels consumed, with dQ, dK turned back to the unrotated inputs
        rot = attention_rope_ref(x["q"], x["k"], x["v"], x["do"], scale, mode, c["cu"], dtype=c["dtype"])
        check_rotated(kw["q_rot"], rot["q_rot"], x["q"], c["dtype"], f"random c{c['id']} q_rot")
        check_rotated(kw["k_rot"], rot["k_rot"], x["k"], c["dtype"], f"random c{c['id']} k_rot")
        q_in, k_in = (kw[n].float().cpu().numpy().astype(np.float64) for n in ("q_rot", "k_rot"))
        ref = attention_bwd_ref(q_in, k_in, x["v"], x["do"], scale, mode, c["cu"])
        pos = rope_positions(S, mode, c["cu"])
        ref["dq"] = rope_rotate(ref["dq"], pos, inverse=True)
        ref["dk"] = rope_rotate(ref["dk"], pos, inverse=True)
    else:
        q_in, k_in = x["q"], x["k"]
        ref = attention_bwd_ref(x["q"], x["k"], x["v"], x["do"], scale, mode, c["cu"])
    out16 = c["dtype"] if c["out16"] else None
    compare(out, ref, c["dtype"], out16=out16, tag=f"random c{c['id']}",
            bounds=None if c["dtype"] == "f32" else model_bounds(x, q_in, k_in, ref, c, scale, mode, out16))


def model_bounds(x, q, k, ref, c, scale, mode, out16):
    """Max-abs and relative-Frobenius bounds of O, dQ, dK, dV for a 16-bit
    case: the fixed bound, or twice the 16-bit rounding model's own error on
    this input where that is larger.  Unit-scale inputs with groups of 8-16
    query heads sum enough rounded weights into dK, dV to pass the fixed
    max-abs bound, and with two or three rows one row whose dP - Delta
    cancels sets the whole relative-Frobenius error.  The model computes the
    same rounding points on the same values (q and k the rotated values with
    RoPE)."""
    m = attention_model(q, k, x["v"], x["do"], scale, mode, c["cu"], fmt=c["dtype"], out16=out16 is not None)
    if c["rope"]:
        pos = rope_positions(q.shape[2], mode, c["cu"])
        m["dq"] = rope_rotate(m["dq"], pos, inverse=True)
        m["dk"] = rope_rotate(m["dk"], pos, inverse=True)
    bounds = {}
    for n in ("o", "dq", "dk", "dv"):
        d = np.abs(m[n] - ref[n])
        if out16 is not None:
            d = d - half_ulp(np.maximum(np.abs(m[n]), np.abs(ref[n])), out16)
        err = float(np.max(d)) if d.size else 0.0
        bounds[n] = max(TOL[c["dtype"]]["max_abs"], 2.0 * err)
        r_norm = float(np.linalg.norm(ref[n]))
        fro = float(np.linalg.norm(m[n] - ref[n])) / r_norm if r_norm > 0 else 0.0
        bounds[n + "_fro"] = max(TOL[c["dtype"]]["rel_fro"], 2.0 * fro)
    return bounds
