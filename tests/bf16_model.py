"""Rounding model of the 16-bit attention path (test infrastructure, fp64).

The oracle computes attention exactly (fp64).  With 16-bit inputs the kernels
cannot: they accumulate in fp32 but round two intermediates to the input
format before the products that consume them, and the backward takes Delta
from the O the forward stored.  This module computes attention with exactly
those rounding points and nothing else (everything between them in fp64), so
the difference between it and the oracle is the error the method's
arithmetic itself makes at that precision.  It sets the tolerances the GPU
tests use where the fixed bounds do not apply, and shows that the fixed
bounds hold with margin at the workloads.

Rounding points (per head; S the scaled, masked scores):
  forward   m = rowmax S ; E = exp(S - m) ; l = rowsum E ; Er = rnd(E)
            O = (Er V) / rowsum Er      stored as fp32 (or rnd16 with 16-bit outputs)
            LSE = m + ln l              fp32 (from the unrounded weights)
  backward  P = exp(S - LSE)            fp32 (from the stored LSE)
            dP = dO V^T ; Delta = rowsum(dO o O_stored)
            dV = rnd(P)^T dO ; dS = rnd(P o (dP - Delta))
            dQ = scale dS K ; dK = scale dS^T Q      stored as fp32 (or rnd16)

rnd is round-to-nearest-even to the input format (of the fp32 value, as the
kernels round their fp32 registers).  Not modelled: the order of the fp32
sums (a change at fp32's resolution, far below the 16-bit roundings) and the
forward's running maximum: the kernels shift the weights by the maximum of
the tiles seen so far rather than the row's, which changes which rounding
each weight gets but not its size, since O is divided by the sum of the very
weights it was built from (a one-key row gives that key's value exactly
either way).

The operations are those of the oracle's definition (oracle/attention.py):
no blocking, no reordering; only the rounding steps are added.
"""
from __future__ import annotations

import numpy as np

from oracle import allowed_mask
from workload import round_to


def _rnd(x, fmt):
    """fp64 -> fp32 -> fmt (round to nearest even) -> fp64; fmt None: no rounding."""
    if fmt is None:
        return np.asarray(x, dtype=np.float64)
    return round_to(np.asarray(x, dtype=np.float32), fmt).astype(np.float64)


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def attention_model(q, k, v, do, scale, mask_mode=0, cu_seqlens=None, heads=None, fmt="bf16", out16=False):
    """Forward and backward with the 16-bit path's rounding points.

    q, do: [B, H, S, D] and k, v: [B, H_kv, S, D] arrays holding input-format
    values (H_kv dividing H; query head h uses K/V head h // (H / H_kv), and
    dK, dV sum the group's query heads in fp64 before their one store).
    fmt: "bf16" or "f16" (the input format), or None for no rounding at all
    (then the result is the oracle's up to fp32 storage of the outputs).
    out16: O, dQ, dK, dV stored in fmt instead of fp32 (and Delta taken from
    that stored O).  heads: list of (b, h), default all (grouped heads need
    all).  Returns a dict like the oracle's: o, lse, dq, dk, dv, delta
    (float64 arrays; heads not computed are NaN).
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, S, D = q.shape
    H_kv = k.shape[1]
    if H % H_kv or v.shape[1] != H_kv or (heads is not None and H_kv != H):
        raise ValueError("H_kv must divide H; grouped heads are modelled for all heads at once")
    G = H // H_kv
    allowed = allowed_mask(S, mask_mode, cu_seqlens)
    store = (lambda x: _rnd(x, fmt)) if out16 and fmt is not None else _f32
    out = {n: np.full((B, H, S, D), np.nan) for n in ("o", "dq")}
    out.update({n: np.full((B, H_kv, S, D), np.nan if G == 1 else 0.0) for n in ("dk", "dv")})
    out["lse"] = np.full((B, H, S), np.nan)
    out["delta"] = np.full((B, H, S), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        qh, kh, vh, doh = q[b, h], k[b, h // G], v[b, h // G], do[b, h]
        s = np.where(allowed, scale * (qh @ kh.T), -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l_sum = e.sum(axis=1)
        er = _rnd(e, fmt)
        o = store((er @ vh) / er.sum(axis=1)[:, None])
        lse = _f32(m + np.log(l_sum))
        p = _f32(np.exp(s - lse[:, None]))
        dp = doh @ vh.T
        delta = _f32((doh * o).sum(axis=1))
        ds = _rnd(p * (dp - delta[:, None]), fmt)
        out["o"][b, h] = o
        out["lse"][b, h] = lse
        out["delta"][b, h] = delta
        out["dq"][b, h] = store(scale * (ds @ kh))
        if G == 1:
            out["dv"][b, h] = store(_rnd(p, fmt).T @ doh)
            out["dk"][b, h] = store(scale * (ds.T @ qh))
        else:
            out["dv"][b, h // G] += _rnd(p, fmt).T @ doh
            out["dk"][b, h // G] += scale * (ds.T @ qh)
    if G > 1:
        out["dv"] = store(out["dv"])
        out["dk"] = store(out["dk"])
    return out


def max_errors(got, ref, names=("o", "lse", "dq", "dk", "dv"), heads=None):
    """Max-abs and relative-Frobenius error of each output (over `heads`, or
    wherever ref is finite)."""
    res = {}
    for n in names:
        g, r = np.asarray(got[n], dtype=np.float64), np.asarray(ref[n], dtype=np.float64)
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads])
        d = g - r
        res[n] = (float(np.max(np.abs(d))), float(np.linalg.norm(d) / np.linalg.norm(r)))
    return res
