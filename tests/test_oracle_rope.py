"""Pins for the RoPE part of the oracle (oracle/rope.py), independent of its
own formulas: hand-worked rotations, RoFormer's complex-number form, the
relative-position property, orthogonality, document-local positions by
decomposition, central finite differences through the rotation, PyTorch
autograd over a complex-multiply rotation, and the 16-bit rounding against
library casts and worked ties.  A sign slip in one component, half-split
instead of interleaved pairs, a wrong frequency exponent, a missing inverse in
the gradient, or positions that do not restart per document fails one."""
import math

import numpy as np
import pytest

from oracle import (
    MASK_CAUSAL,
    MASK_DOC_CAUSAL,
    allowed_mask,
    attention_bwd_ref,
    attention_rope_ref,
    rope_angles,
    rope_positions,
    rope_rotate,
    round_to_dtype,
)

CU = np.array([0, 5, 6, 13, 20], dtype=np.int32)  # documents of length 5, 1, 7, 7


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------- the rotation

def test_worked_rotations():
    """D = 2: the only pair turns by p radians.  D = 4, base 10000: pair 1 turns
    by p / 100.  Values written out by hand (cos 1, sin 1, cos 0.5, sin 0.5)."""
    c1, s1 = 0.5403023058681398, 0.8414709848078965
    y = rope_rotate(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([1, 1]))
    np.testing.assert_allclose(y, [[c1, s1], [-s1, c1]], rtol=0, atol=1e-15)
    # position 50: pair 0 by 50 rad, pair 1 by 0.5 rad
    c5, s5 = 0.8775825618903728, 0.479425538604203
    y = rope_rotate(np.array([[0.0, 0.0, 2.0, 0.0]]), np.array([50]))
    np.testing.assert_allclose(y, [[0.0, 0.0, 2 * c5, 2 * s5]], rtol=0, atol=1e-15)
    y = rope_rotate(np.array([[3.0, 0.0, 0.0, 0.0]]), np.array([50]))
    np.testing.assert_allclose(y, [[3 * math.cos(50.0), 3 * math.sin(50.0), 0.0, 0.0]], rtol=0, atol=1e-14)


def test_position_zero_is_identity():
    x = _rand((3, 7, 64), 1)
    y = rope_rotate(x, np.zeros(7, dtype=np.int64))
    assert np.array_equal(x, y)


@pytest.mark.parametrize("D,base", [(32, 10000.0), (64, 10000.0), (128, 500000.0)])
def test_complex_multiply_form(D, base):
    """RoFormer's complex form: pair i is the complex number x_2i + i x_2i+1,
    multiplied by exp(i p base^(-2i/D)); frequencies from numpy's power of the
    even indices, independently of the oracle."""
    S = 37
    x = _rand((2, S, D), D)
    pos = np.arange(S)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    freq = np.power(base, -np.arange(0, D, 2) / D)
    w = z * np.exp(1j * np.outer(pos, freq))
    y = rope_rotate(x, pos, base)
    np.testing.assert_allclose(y[..., 0::2], w.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], w.imag, rtol=0, atol=1e-13)


def test_angles_table():
    a = rope_angles(5, 8, 10000.0)
    assert a.shape == (5, 4)
    np.testing.assert_allclose(a[3], [3.0, 0.3, 0.03, 0.003], rtol=1e-15)


def test_relative_position_and_orthogonality():
    """<R(p+t) q, R(r+t) k> = <R(p) q, R(r) k>; pair norms are kept; the
    inverse undoes the rotation and is its transpose."""
    D = 64
    q, k = _rand((D,), 3), _rand((D,), 4)
    def rot(x, p, inverse=False):
        return rope_rotate(x[None, :], np.array([p]), inverse=inverse)[0]
    ref = rot(q, 7) @ rot(k, 3)
    for t in (1, 100, 4000):
        assert abs(rot(q, 7 + t) @ rot(k, 3 + t) - ref) < 1e-10
    y = rot(q, 123)
    np.testing.assert_allclose(np.hypot(y[0::2], y[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-14)
    np.testing.assert_allclose(rot(y, 123, inverse=True), q, atol=1e-14)
    assert abs(rot(q, 55) @ k - q @ rot(k, 55, inverse=True)) < 1e-12


def test_positions():
    np.testing.assert_array_equal(rope_positions(4), [0, 1, 2, 3])
    np.testing.assert_array_equal(rope_positions(5, MASK_DOC_CAUSAL, [0, 3, 5]), [0, 1, 2, 0, 1])
    np.testing.assert_array_equal(rope_positions(20, MASK_DOC_CAUSAL, CU),
                                  [0, 1, 2, 3, 4, 0, 0, 1, 2, 3, 4, 5, 6, 0, 1, 2, 3, 4, 5, 6])


# --------------------------------------------------------- 16-bit rounding

def test_bf16_rounding_matches_torch_cast():
    """On float32-exact values (including exact ties) rounding to bf16 equals
    PyTorch's float32 -> bfloat16 cast (nearest, ties to even)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    bits = x32.view(np.uint32)
    bits[:2000] = (bits[:2000] & 0xFFFF0000) | 0x8000  # exact halfway cases
    x32 = bits.view(np.float32)
    want = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to_dtype(x32.astype(np.float64), "bf16"), want)


def test_f16_rounding_matches_numpy_cast():
    """On float32-exact values rounding to fp16 equals numpy's float32 ->
    float16 cast, across normal, subnormal and overflowing magnitudes."""
    rng = np.random.default_rng(6)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-28, 18, 20000))).astype(np.float32)
    with np.errstate(over="ignore"):
        want = x32.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(round_to_dtype(x32.astype(np.float64), "f16"), want)


def test_rounding_worked_ties_and_limits():
    r = round_to_dtype
    assert r(1 + 2.0 ** -8, "bf16") == 1.0                      # tie, even neighbour below
    assert r(1 + 3 * 2.0 ** -8, "bf16") == 1 + 2.0 ** -6        # tie, even neighbour above
    assert r(2049.0, "f16") == 2048.0 and r(2051.0, "f16") == 2052.0
    assert r(65519.0, "f16") == 65504.0 and np.isinf(r(65520.0, "f16"))
    assert r(2.0 ** -25, "f16") == 0.0                          # half the smallest subnormal: tie to 0
    assert r(3 * 2.0 ** -25, "f16") == 2.0 ** -23
    assert r(-(1 + 2.0 ** -9), "bf16") == -1.0
    x = _rand(1000, 7)
    for dt in ("bf16", "f16", "f32"):
        y = r(x, dt)
        assert np.array_equal(r(y, dt), y)                      # idempotent
    assert np.array_equal(r(x, "f64"), x)


# --------------------------------------------------------- attention + RoPE

def _inputs(B, H, S, D, seed, H_kv=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, D))
    k = rng.standard_normal((B, H_kv or H, S, D))
    v = rng.standard_normal((B, H_kv or H, S, D))
    do = rng.standard_normal((B, H, S, D))
    return q, k, v, do


def _loss(q, k, v, do, scale, mode, cu, base):
    r = attention_rope_ref(q, k, v, do, scale, mode, cu, base, dtype="f64")
    return float(np.sum(r["o"] * do))


@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_rope_gradients_match_central_differences(mode):
    B, H, S, D = 1, 2, 20, 8
    q, k, v, do = _inputs(B, H, S, D, 11)
    scale, base = 1 / math.sqrt(D), 100.0
    cu = CU if mode == MASK_DOC_CAUSAL else None
    r = attention_rope_ref(q, k, v, do, scale, mode, cu, base, dtype="f64")
    h = 1e-6
    rng = np.random.default_rng(12)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(12):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"dq": (q, k, v), "dk": (q, k, v), "dv": (q, k, v)}[name]
            ip = [xp if a is x else a for a in args]
            im = [xm if a is x else a for a in args]
            fd = (_loss(*ip, do, scale, mode, cu, base) - _loss(*im, do, scale, mode, cu, base)) / (2 * h)
            assert abs(fd - r[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, r[name][idx])


def test_rope_matches_torch_complex_rotation_and_autograd():
    """PyTorch in float64: rotation by complex multiplication (view_as_complex,
    polar), SDPA with the causal flag, autograd for the gradients."""
    torch = pytest.importorskip("torch")
    B, H, H_kv, S, D = 2, 4, 2, 24, 16
    q, k, v, do = _inputs(B, H, S, D, 13, H_kv)
    scale = 1 / math.sqrt(D)
    r = attention_rope_ref(q, k, v, do, scale, base=10000.0, dtype="f64")

    freq = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(S, D // 2, dtype=torch.float64), torch.outer(torch.arange(S, dtype=torch.float64), freq))

    def rope(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(x.shape)

    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(rope(tq), rope(tk), tv, is_causal=True, scale=scale,
                                                          enable_gqa=True)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], to.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_rope_packed_equals_documents_run_alone():
    """Packed documents with RoPE = each document run alone as a causal
    sequence with RoPE: positions restart at every document."""
    q, k, v, do = _inputs(1, 2, 20, 16, 14)
    scale = 0.25
    r = attention_rope_ref(q, k, v, do, scale, MASK_DOC_CAUSAL, CU, dtype="f64")
    for a, b in zip(CU[:-1], CU[1:]):
        s = slice(int(a), int(b))
        d = attention_rope_ref(q[:, :, s], k[:, :, s], v[:, :, s], do[:, :, s], scale, dtype="f64")
        for name in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(r[name][:, :, s], d[name], rtol=1e-12, atol=1e-13)


def test_rope_rotated_inputs_are_held_in_dtype():
    q, k, v, do = _inputs(1, 2, 12, 32, 15)
    pos = np.arange(12)
    for dt in ("bf16", "f16", "f32"):
        r = attention_rope_ref(q, k, v, do, 0.2, dtype=dt)
        assert np.array_equal(r["q_rot"], round_to_dtype(rope_rotate(q, pos), dt))
        assert np.array_equal(r["k_rot"], round_to_dtype(rope_rotate(k, pos), dt))
        plain = attention_bwd_ref(r["q_rot"], r["k_rot"], v, do, 0.2)
        assert np.array_equal(r["o"], plain["o"])
        # the gradient passes the rounding: dq is plain dq turned back
        np.testing.assert_allclose(r["dq"], rope_rotate(plain["dq"], pos, inverse=True), rtol=0, atol=0)


def test_rope_mask_is_unchanged():
    """RoPE changes scores, never which keys a query may see: future keys stay
    invisible (bitwise) after rotation."""
    q, k, v, do = _inputs(1, 1, 10, 8, 16)
    r1 = attention_rope_ref(q, k, v, do, 0.3, dtype="f64")
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 6:] += 5.0
    v2[:, :, 6:] -= 3.0
    r2 = attention_rope_ref(q, k2, v2, do, 0.3, dtype="f64")
    assert np.array_equal(r1["o"][:, :, :6], r2["o"][:, :, :6])
    assert allowed_mask(10)[5, 6] == False  # noqa: E712
