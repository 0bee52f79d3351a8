"""Rotary position embedding (RoPE) on queries and keys before attention, and
its gradient, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed.  ARK's model rotates queries and keys by their position,
from precomputed sine and cosine tables (ARK, "Inference architecture (EKO)"
in the pipeline list, and the "Positional encoding" row of the model table),
after Su et al. 2021, RoFormer (ARK, references); Forge's attention takes
RoPE behind the same interface as grouped-query attention (Forge,
"Architecture").  RoFormer's rotation splits the head dimension into D/2
interleaved pairs (x_2i, x_2i+1) and turns pair i at position p by the angle
p * theta_i, theta_i = base^(-2i/D):

    y_2i   = x_2i cos(p theta_i) - x_2i+1 sin(p theta_i)
    y_2i+1 = x_2i sin(p theta_i) + x_2i+1 cos(p theta_i)

Attention (``attention.py``) then runs on the rotated queries and keys; the
values are not rotated.  Each pair's rotation is orthogonal, so the gradient
with respect to an unrotated input is the gradient with respect to its
rotated form turned back by the opposite angle.

Readings where the pages are silent (each is listed in the design notes):
  * positions count from 0 at the start of the sequence; with packed
    documents each document is its own sequence and its positions restart
    at 0;
  * base 10000 unless given (RoFormer's value);
  * with 16-bit inputs the rotated queries and keys are held in the input
    dtype (nearest value, ties to even), as a model that runs in that dtype
    holds them, and attention runs on those values; the gradient passes the
    rounding unchanged (the derivative of a dtype cast is taken as 1).
"""
from __future__ import annotations

import numpy as np

from .attention import MASK_CAUSAL, MASK_DOC_CAUSAL, attention_bwd_ref

ROPE_BASE = 10000.0

# (significant bits including the leading one, smallest normal exponent,
# largest finite value) of the 16-bit formats
_FORMATS = {
    "bf16": (8, -126, float.fromhex("0x1.fep127")),
    "f16": (11, -14, 65504.0),
}


def round_to_dtype(x, dtype):
    """Round float64 values to the nearest value of ``dtype`` ("f32", "bf16"
    or "f16"), ties to even, returned as float64.  Out-of-range values go to
    +-inf; values below the smallest normal round on the subnormal grid.
    "f64" returns the values unchanged."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    bits, emin, fmax = _FORMATS[dtype]
    _, e = np.frexp(x)                         # x = m 2^e, 1/2 <= |m| < 1
    e = np.maximum(e - 1, emin)                # exponent of the leading bit (normal range floor)
    quantum = np.ldexp(1.0, e - (bits - 1))    # spacing of representable values there
    y = np.rint(x / quantum) * quantum         # rint: nearest, ties to even
    return np.where(np.abs(y) > fmax, np.copysign(np.inf, x), y)


def rope_angles(n_pos, D, base=ROPE_BASE):
    """Angle p * theta_i of pair i at position p: float64 [n_pos, D/2]."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / D)
    return np.arange(n_pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_positions(S, mask_mode=MASK_CAUSAL, cu_seqlens=None):
    """Position of each of the S rows: the row index, or with packed documents
    the offset from the start of the row's document."""
    s = np.arange(S)
    if mask_mode == MASK_CAUSAL:
        return s
    if mask_mode != MASK_DOC_CAUSAL:
        raise ValueError("unknown mask mode")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    doc = np.searchsorted(cu, s, side="right") - 1
    return s - cu[doc]


def rope_rotate(x, pos, base=ROPE_BASE, inverse=False):
    """Rotate x [..., S, D] row by row (row s at position pos[s]); ``inverse``
    turns by the opposite angles (the transpose of the rotation)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = rope_angles(int(np.max(pos)) + 1, D, base)[np.asarray(pos)]   # [S, D/2]
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def attention_rope_ref(q, k, v, do, scale, mask_mode=MASK_CAUSAL, cu_seqlens=None, base=ROPE_BASE,
                       dtype="f32"):
    """Rotate q and k, hold them in ``dtype``, run attention forward and
    backward on them, and turn dq and dk back to the unrotated inputs.

    Returns the dict of ``attention_bwd_ref`` (o, lse, dq, dk, dv, delta) with
    dq and dk taken with respect to the unrotated q and k, plus ``q_rot`` and
    ``k_rot`` (the rotated, dtype-held values attention ran on).
    """
    S = np.asarray(q).shape[2]
    pos = rope_positions(S, mask_mode, cu_seqlens)
    q_rot = round_to_dtype(rope_rotate(q, pos, base), dtype)
    k_rot = round_to_dtype(rope_rotate(k, pos, base), dtype)
    out = attention_bwd_ref(q_rot, k_rot, v, do, scale, mask_mode, cu_seqlens)
    out["dq"] = rope_rotate(out["dq"], pos, base, inverse=True)
    out["dk"] = rope_rotate(out["dk"], pos, base, inverse=True)
    out["q_rot"] = q_rot
    out["k_rot"] = k_rot
    return out
