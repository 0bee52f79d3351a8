"""Seeded random combinations of every option of attn_fwd_ex / attn_bwd_ex
(input dtype, D, causal or packed documents, grouped K/V heads, RoPE, 16-bit
outputs, [B, S, H, D] views, empty documents among packed ones) against
the fp64 oracle, at sizes the oracle finishes quickly.  The cases are drawn
once from a fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest

from oracle import MASK_CAUSAL, MASK_DOC_CAUSAL, attention_bwd_ref, attention_rope_ref
from tests.gpu_util import compare, log

pytestmark = pytest.mark.gpu


def _draw_cases(n=96, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "bf16", "f16", "f32"]))
        D = int(rng.choice([32, 64, 128]))
        H_kv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4]))
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


CASES = _draw_cases()


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


@pytest.mark.parametrize("case", CASES, ids=[f"c{c['id']}" for c in CASES])
def test_random_option_mix(case):
    import torch
    import causal_attention_amd as ca
    c = case
    log(f"[random] {c}")
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
    ca.attn_fwd_ex(q, k, v, out["o"], out["lse"], scale, **kw)
    ca.attn_bwd_ex(q, k, v, out["o"], do, out["lse"], out["dq"], out["dk"], out["dv"], out["delta"], scale, **kw)
    torch.cuda.synchronize()
    if c["rope"]:
        ref = attention_rope_ref(x["q"], x["k"], x["v"], x["do"], scale, mode, c["cu"], dtype=c["dtype"])
    else:
        ref = attention_bwd_ref(x["q"], x["k"], x["v"], x["do"], scale, mode, c["cu"])
    compare(out, ref, c["dtype"], out16=c["dtype"] if c["out16"] else None, tag=f"random c{c['id']}")
