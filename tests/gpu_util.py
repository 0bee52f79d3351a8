"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI, compare against the fp64 oracle with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

import causal_attention_amd as ca
from oracle import attention_bwd_ref

# Tolerances: fp32 inputs, max-abs 1e-4 on every output; bf16 inputs, max-abs
# 2e-2 and relative Frobenius error 1e-2 per tensor (O, dQ, dK, dV), LSE 1e-3.
TOL = {
    "f32": dict(max_abs=1e-4, rel_fro=None, lse=1e-4),
    "bf16": dict(max_abs=2e-2, rel_fro=1e-2, lse=1e-3),
    "f16": dict(max_abs=2e-2, rel_fro=1e-2, lse=1e-3),  # 16-bit inputs: the bf16 bounds
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x):
    import torch
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[x["dtype"]]
    dev = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to("cuda").to(dt).contiguous()
           for n in ("q", "k", "v", "do")}
    cu = x.get("cu_seqlens")
    if cu is not None:
        dev["cu"] = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to("cuda")
        dev["max_seqlen"] = int(np.diff(cu).max())
    else:
        dev["cu"] = None
        dev["max_seqlen"] = None
    return dev


def run_hip(x, dev=None, poison=True, stream=None, workspace=None):
    """Forward + backward on the GPU.  Outputs are NaN-poisoned first, so an
    element the kernels fail to write shows up as NaN.  Returns torch tensors.
    workspace: passed to the backward (attn_bwd_gqa_ws), or None."""
    import torch
    if dev is None:
        dev = to_device(x)
    B, H, S, D = x["B"], x["H"], x["S"], x["D"]
    fill = float("nan") if poison else 0.0
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {n: torch.full((B, H, S, D), fill, **f32) for n in ("o", "dq")}
    for n in ("dk", "dv"):  # K/V may have fewer heads (grouped-query attention)
        out[n] = torch.full(tuple(x["k"].shape), fill, **f32)
    out["lse"] = torch.full((B, H, S), fill, **f32)
    out["delta"] = torch.full((B, H, S), fill, **f32)
    mode = x["mask_mode"]
    ca.attn_fwd(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], x["scale"], mode, dev["cu"], None,
                dev["max_seqlen"], stream)
    ca.attn_bwd(dev["q"], dev["k"], dev["v"], out["o"], dev["do"], out["lse"], out["dq"], out["dk"], out["dv"],
                out["delta"], x["scale"], mode, dev["cu"], None, dev["max_seqlen"], stream, workspace=workspace)
    torch.cuda.synchronize()
    return out


def oracle(x, heads=None):
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "do")]
    return attention_bwd_ref(*args, x["scale"], x["mask_mode"], x.get("cu_seqlens"), heads=heads)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel_fro = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got - ref))
    return max_abs, rel_fro


def check_delta(out, x):
    """Delta against fp64 rowsum(dO o O) of the O the GPU stored: both kernels
    that compute it add D products of an input-dtype dO and an fp32 O in fp32,
    so each row's error is at most D * 2^-24 * sum_d |dO_d O_d| (a chain of D
    rounded fused multiply-adds, or a tree of them: the same bound)."""
    o = out["o"].detach().float().cpu().numpy().astype(np.float64)
    do = np.asarray(x["do"], dtype=np.float64)
    if o.shape != do.shape:
        raise ValueError("Delta check needs O and dO of the same shape")
    got = out["delta"].detach().cpu().numpy().astype(np.float64)
    exact = np.sum(do * o, axis=-1)
    D = o.shape[-1]
    bound = D * 2.0 ** -24 * np.sum(np.abs(do * o), axis=-1) + 1e-30
    worst = float(np.max(np.abs(got - exact) / bound))
    assert worst <= 1.0, f"Delta off rowsum(dO o O_stored) by {worst:.2f}x its fp32 bound"
    return worst


# significant bits of the 16-bit output formats
_OUT_BITS = {"bf16": 8, "f16": 11}


def half_ulp(x, fmt):
    """Half the spacing of ``fmt`` ("bf16" or "f16") values at |x|: the error a
    correctly rounded store of the exact value may make."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))  # |x| = m 2^e, 1/2 <= m < 1
    return np.ldexp(1.0, e - _OUT_BITS[fmt] - 1)


def compare(out, ref, dtype, heads=None, names=("o", "lse", "dq", "dk", "dv", "delta"), tag="",
            rel_to_max=None, out16=None, bounds=None):
    """Assert the GPU outputs match the oracle on the given heads (all if None).

    rel_to_max: if given, the max-abs bound of O/dQ/dK/dV is rel_to_max * max|ref|
    instead of the fixed absolute bound (for inputs far outside the workloads'
    scale, where bf16 rounding error grows with the magnitudes).
    out16: "bf16" or "f16" when O, dQ, dK, dV are stored in that format; each
    element's bound then grows by its own rounding, half_ulp(ref).
    bounds: optional max-abs bound per output name (O, dQ, dK, dV), replacing
    the fixed one, and optional relative-Frobenius bound under the name plus
    "_fro" (both derived by the caller from the 16-bit rounding model)."""
    tol = TOL[dtype]
    report = {}
    for name in names:
        g = out[name].detach().float().cpu().numpy().astype(np.float64)
        r = ref[name]
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads])
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite outputs (unwritten or overflow)"
        ma, rf = errors(g, r)
        report[name] = (ma, rf)
        if name in ("lse",):
            assert ma <= tol["lse"], f"{tag} {name}: max-abs {ma:.3e} > {tol['lse']}"
        elif name == "delta":
            # Delta is an intermediate: bounded by |dO| |O| accuracy, checked loosely
            assert ma <= 10 * tol["max_abs"], f"{tag} {name}: max-abs {ma:.3e}"
        else:
            lim = tol["max_abs"] if rel_to_max is None else rel_to_max * float(np.max(np.abs(r)))
            if bounds is not None and name in bounds:
                lim = bounds[name]
            if out16 is not None:  # error beyond the store's own rounding
                # the store rounds the kernel's value, which may sit in the binade above ref
                ma = float(np.max(np.abs(g - r) - half_ulp(np.maximum(np.abs(g), np.abs(r)), out16))) \
                    if g.size else 0.0
                report[name] = (ma, rf)
            assert ma <= lim, f"{tag} {name}: max-abs {ma:.3e} > {lim}"
            fro_lim = tol["rel_fro"]
            if bounds is not None and name + "_fro" in bounds:
                fro_lim = bounds[name + "_fro"]
            if fro_lim is not None:
                assert rf <= fro_lim, f"{tag} {name}: rel-Frobenius {rf:.3e} > {fro_lim}"
    log(f"{tag} " + " ".join(f"{n}:{m:.2e}/{f:.1e}" for n, (m, f) in report.items()))
    return report
