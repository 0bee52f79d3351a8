"""Pins for the fp64 oracle, independent of the oracle's own formulas.

Each test fixes the oracle against something the mathematics or a separate
library settles: closed forms (Q = 0, row 0, V = 1, V = I), softmax
invariants, causality under perturbation, per-document decomposition,
central finite differences of L = sum(O * dO), the softmax shift invariance
of dK, and PyTorch's own CPU scaled-dot-product attention with autograd.
A plausible slip in the oracle (a dropped scale, an excluded diagonal, a
transposed operand, a log base, a sign in Delta) fails at least one.
"""
import math

import numpy as np
import pytest

from oracle import (
    MASK_CAUSAL,
    MASK_DOC_CAUSAL,
    allowed_mask,
    attention_bwd_ref,
    attention_dkdv_rows_ref,
    attention_dq_rows_ref,
    attention_fwd_ref,
    attention_fwd_rows_ref,
    delta_ref,
)

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


def _qkvdo(B, H, S, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, S, D)) for _ in range(4)]


CU_SMALL = np.array([0, 5, 6, 13, 20], dtype=np.int32)  # documents of length 5, 1, 7, 7


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_q_zero_gives_prefix_mean(mode):
    """Q = 0 makes every allowed score 0, so P is uniform over the allowed keys:
    O_i = mean of V over the allowed prefix, LSE_i = ln(number of allowed keys)."""
    B, H, S, D = 1, 2, 20, 8
    _, k, v, _ = _qkvdo(B, H, S, D, 1)
    q = np.zeros_like(k)
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    o, lse = attention_fwd_ref(q, k, v, 0.37, mode, cu)
    starts = np.zeros(S, dtype=int)
    if cu is not None:
        for a, e in zip(cu[:-1], cu[1:]):
            starts[a:e] = a
    for i in range(S):
        n = i - starts[i] + 1
        np.testing.assert_allclose(o[:, :, i], v[:, :, starts[i]:i + 1].mean(axis=2), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14)


def test_row_zero_attends_only_itself():
    """Query 0 sees key 0 alone: O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    B, H, S, D = 2, 3, 9, 16
    q, k, v, _ = _qkvdo(B, H, S, D, 2)
    scale = 0.25
    o, lse = attention_fwd_ref(q, k, v, scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    expect = scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], expect, rtol=1e-15, atol=1e-15)


def test_constant_v_gives_constant_o():
    B, H, S, D = 1, 2, 17, 8
    q, k, _, _ = _qkvdo(B, H, S, D, 3)
    v = np.ones((B, H, S, D))
    o, _ = attention_fwd_ref(q, k, v, 0.5)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_identity_v_exposes_probabilities(mode):
    """With D = S and V = I, O equals the probability matrix P itself:
    rows are >= 0, sum to 1 and are exactly 0 where the mask forbids."""
    S = 20
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, S, S)) * 2.0
    k = rng.standard_normal((1, 1, S, S)) * 2.0
    v = np.eye(S)[None, None]
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    p, _ = attention_fwd_ref(q, k, v, 0.3, mode, cu)
    p = p[0, 0]
    allowed = allowed_mask(S, mode, cu)
    assert np.all(p >= 0)
    assert np.all(p[~allowed] == 0.0)
    assert np.all(p[allowed] > 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_mask_shapes():
    m = allowed_mask(4)
    assert m.tolist() == [[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]]
    m = allowed_mask(5, MASK_DOC_CAUSAL, [0, 2, 5])
    assert m.astype(int).tolist() == [[1, 0, 0, 0, 0], [1, 1, 0, 0, 0],
                                      [0, 0, 1, 0, 0], [0, 0, 1, 1, 0], [0, 0, 1, 1, 1]]
    with pytest.raises(ValueError):
        allowed_mask(5, MASK_DOC_CAUSAL, [0, 4, 3, 5])  # a boundary that goes back
    with pytest.raises(ValueError):
        allowed_mask(5, MASK_DOC_CAUSAL, [0, 4])        # does not end at S
    # empty documents own no rows: the mask is that of the non-empty ones
    for cu in ([0, 3, 3, 5], [0, 0, 3, 5], [0, 3, 5, 5], [0, 0, 0, 3, 3, 5, 5]):
        assert (allowed_mask(5, MASK_DOC_CAUSAL, cu) == allowed_mask(5, MASK_DOC_CAUSAL, [0, 3, 5])).all()


# ---------------------------------------------------------------- causality

def test_future_keys_do_not_change_past_rows():
    """Perturbing K_j, V_j for j > i leaves O_i and LSE_i bitwise unchanged."""
    B, H, S, D = 1, 2, 24, 8
    q, k, v, _ = _qkvdo(B, H, S, D, 5)
    o, lse = attention_fwd_ref(q, k, v, 0.4)
    i = 10
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] += 3.0 * _rand(B, H, S - i - 1, D)
    v2[:, :, i + 1:] -= 5.0
    o2, lse2 = attention_fwd_ref(q, k2, v2, 0.4)
    assert np.array_equal(o[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(lse[:, :, :i + 1], lse2[:, :, :i + 1])
    assert not np.allclose(o[:, :, i + 1:], o2[:, :, i + 1:])


def test_backward_causality():
    """dQ_i depends on keys j <= i only; dK_j, dV_j on queries i >= j only."""
    B, H, S, D = 1, 1, 16, 8
    q, k, v, do = _qkvdo(B, H, S, D, 6)
    r = attention_bwd_ref(q, k, v, do, 0.3)
    c = 7
    # change the future keys: dQ of rows <= c unchanged
    k2, v2 = k.copy(), v.copy()
    k2[:, :, c + 1:] *= -2.0
    v2[:, :, c + 1:] += 1.0
    r2 = attention_bwd_ref(q, k2, v2, do, 0.3)
    np.testing.assert_allclose(r["dq"][:, :, :c + 1], r2["dq"][:, :, :c + 1], rtol=1e-13, atol=1e-14)
    # change the past queries and their upstream gradients: dK, dV of rows >= c+1 unchanged
    q3, do3 = q.copy(), do.copy()
    q3[:, :, :c + 1] += 1.5
    do3[:, :, :c + 1] *= 3.0
    r3 = attention_bwd_ref(q3, k, v, do3, 0.3)
    for name in ("dk", "dv"):
        np.testing.assert_allclose(r[name][:, :, c + 1:], r3[name][:, :, c + 1:], rtol=1e-13, atol=1e-14)
        assert not np.allclose(r[name][:, :, :c + 1], r3[name][:, :, :c + 1])


# ---------------------------------------------------------------- packed documents

def test_packed_equals_documents_run_alone():
    """Block-diagonal causal attention = each document through plain causal attention."""
    B, H, S, D = 1, 2, 20, 8
    q, k, v, do = _qkvdo(B, H, S, D, 7)
    scale = 0.35
    r = attention_bwd_ref(q, k, v, do, scale, MASK_DOC_CAUSAL, CU_SMALL)
    for a, e in zip(CU_SMALL[:-1], CU_SMALL[1:]):
        sl = slice(a, e)
        ri = attention_bwd_ref(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], scale)
        for name in ("o", "lse", "dq", "dk", "dv", "delta"):
            np.testing.assert_allclose(r[name][:, :, sl], ri[name], rtol=1e-13, atol=1e-14)


def test_empty_documents_change_nothing():
    """Empty documents (repeated boundaries, also first and last) leave every
    output, and the RoPE positions, as without them."""
    B, H, S, D = 1, 2, 20, 8
    q, k, v, do = _qkvdo(B, H, S, D, 9)
    ref = attention_bwd_ref(q, k, v, do, 0.35, MASK_DOC_CAUSAL, CU_SMALL)
    a, b = int(CU_SMALL[1]), int(CU_SMALL[2])
    cu_e = np.array([0, 0] + [int(x) for x in CU_SMALL[1:2]] * 3 + [int(x) for x in CU_SMALL[2:]] + [S],
                    dtype=np.int32)
    assert a < b and cu_e[0] == 0 and cu_e[-1] == S
    r = attention_bwd_ref(q, k, v, do, 0.35, MASK_DOC_CAUSAL, cu_e)
    for name in ("o", "lse", "dq", "dk", "dv", "delta"):
        np.testing.assert_array_equal(r[name], ref[name])
    from oracle import rope_positions
    assert (rope_positions(S, MASK_DOC_CAUSAL, cu_e) == rope_positions(S, MASK_DOC_CAUSAL, CU_SMALL)).all()


def test_single_document_equals_causal():
    B, H, S, D = 2, 2, 12, 8
    q, k, v, do = _qkvdo(B, H, S, D, 8)
    a = attention_bwd_ref(q, k, v, do, 0.3, MASK_CAUSAL)
    b = attention_bwd_ref(q, k, v, do, 0.3, MASK_DOC_CAUSAL, [0, S])
    for name in a:
        assert np.array_equal(a[name], b[name])


def test_other_document_perturbation_is_invisible():
    B, H, S, D = 1, 1, 20, 8
    q, k, v, do = _qkvdo(B, H, S, D, 9)
    r = attention_bwd_ref(q, k, v, do, 0.3, MASK_DOC_CAUSAL, CU_SMALL)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for x in (q2, k2, v2, do2):
        x[:, :, 6:13] += 2.0  # document 2 only
    r2 = attention_bwd_ref(q2, k2, v2, do2, 0.3, MASK_DOC_CAUSAL, CU_SMALL)
    for name in r:
        np.testing.assert_allclose(r[name][:, :, :6], r2[name][:, :, :6], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r[name][:, :, 13:], r2[name][:, :, 13:], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, scale, mode, cu):
    o, _ = attention_fwd_ref(q, k, v, scale, mode, cu)
    return float(np.sum(o * do))


@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_gradients_match_central_differences_everywhere(mode):
    """dQ, dK, dV against central differences of L = sum(O * dO), every element."""
    B, H, S, D = 1, 1, 20, 4
    q, k, v, do = _qkvdo(B, H, S, D, 10)
    scale = 0.6
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    r = attention_bwd_ref(q, k, v, do, scale, mode, cu)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, scale, mode, cu)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, scale, mode, cu)
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - r[name])) / np.max(np.abs(r[name]))
        assert err < 1e-7, (name, err)


def test_gradients_match_central_differences_tiny_config_sample():
    """Sampled central differences at the tiny fp32 workload's shape (B1 H2 S64 D32)."""
    B, H, S, D = 1, 2, 64, 32
    q, k, v, do = _qkvdo(B, H, S, D, 11)
    scale = 1 / math.sqrt(D)
    r = attention_bwd_ref(q, k, v, do, scale)
    rng = np.random.default_rng(12)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(25):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, scale, MASK_CAUSAL, None)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, scale, MASK_CAUSAL, None)
            x[idx] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - r[name][idx]) <= 1e-7 * max(1.0, np.max(np.abs(r[name]))), (name, idx)


@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_shift_invariance_and_delta_identity(mode):
    """Softmax is invariant to adding a constant per row, so sum_j dS_ij = 0, which
    makes sum_j dK_j = 0 per head (and per document).  Delta = rowsum(dO o O)."""
    B, H, S, D = 2, 2, 20, 8
    q, k, v, do = _qkvdo(B, H, S, D, 13)
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    r = attention_bwd_ref(q, k, v, do, 0.4, mode, cu)
    bounds = cu if cu is not None else [0, S]
    for a, e in zip(bounds[:-1], bounds[1:]):
        np.testing.assert_allclose(r["dk"][:, :, a:e].sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(r["delta"], delta_ref(do, r["o"]), rtol=1e-13, atol=1e-13)


def test_q_zero_backward_closed_form():
    """Q = 0: P_ij = 1/(i+1) for j <= i, so dV_j = sum_{i >= j} dO_i / (i + 1) and dK = 0."""
    B, H, S, D = 1, 2, 16, 4
    _, k, v, do = _qkvdo(B, H, S, D, 14)
    q = np.zeros_like(k)
    r = attention_bwd_ref(q, k, v, do, 0.5)
    w = 1.0 / (np.arange(S) + 1.0)
    expect = np.flip(np.cumsum(np.flip(do * w[None, None, :, None], axis=2), axis=2), axis=2)
    np.testing.assert_allclose(r["dv"], expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)


def test_gradients_linear_in_upstream():
    B, H, S, D = 1, 1, 12, 4
    q, k, v, do = _qkvdo(B, H, S, D, 15)
    do2 = _rand(B, H, S, D)
    r1 = attention_bwd_ref(q, k, v, do, 0.3)
    r2 = attention_bwd_ref(q, k, v, do2, 0.3)
    r12 = attention_bwd_ref(q, k, v, 2.0 * do - 0.5 * do2, 0.3)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r12[name], 2.0 * r1[name] - 0.5 * r2[name], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- library cross-check

@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_matches_torch_cpu_sdpa_and_autograd(mode):
    """PyTorch's CPU scaled_dot_product_attention in float64, differentiated by autograd,
    and scipy's logsumexp, agree with the oracle to rounding."""
    torch = pytest.importorskip("torch")
    from scipy.special import logsumexp

    B, H, S, D = 2, 3, 20, 16
    q, k, v, do = _qkvdo(B, H, S, D, 16)
    scale = 1 / math.sqrt(D)
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    r = attention_bwd_ref(q, k, v, do, scale, mode, cu)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    mask = torch.tensor(allowed_mask(S, mode, cu))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], to.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), rtol=1e-11, atol=1e-12)
    scores = scale * np.einsum("bhid,bhjd->bhij", q, k)
    scores = np.where(allowed_mask(S, mode, cu), scores, -np.inf)
    np.testing.assert_allclose(r["lse"], logsumexp(scores, axis=-1), rtol=1e-13, atol=1e-13)


def test_torch_causal_flag_agrees_with_mask_reading():
    """is_causal=True in PyTorch means keys j <= i, the reading the oracle takes."""
    torch = pytest.importorskip("torch")
    B, H, S, D = 1, 2, 16, 8
    q, k, v, _ = _qkvdo(B, H, S, D, 17)
    o, _ = attention_fwd_ref(q, k, v, 1 / math.sqrt(D))
    to = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(x) for x in (q, k, v)), is_causal=True)
    np.testing.assert_allclose(o, to.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- row-wise forms

@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
def test_rowwise_forms_agree_with_full(mode):
    """The per-row functions used for sampled checks at large sizes reproduce the
    full-matrix oracle, which the tests above pin."""
    B, H, S, D = 1, 2, 20, 8
    q, k, v, do = _qkvdo(B, H, S, D, 18)
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    r = attention_bwd_ref(q, k, v, do, 0.3, mode, cu)
    rows = [0, 4, 5, 6, 12, 19]
    o, lse = attention_fwd_rows_ref(q, k, v, 0.3, 0, 1, rows, mode, cu)
    np.testing.assert_allclose(o, r["o"][0, 1, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, r["lse"][0, 1, rows], rtol=1e-13, atol=1e-14)
    dq = attention_dq_rows_ref(q, k, v, do, 0.3, 0, 1, rows, mode, cu)
    np.testing.assert_allclose(dq, r["dq"][0, 1, rows], rtol=1e-12, atol=1e-13)
    dk, dv = attention_dkdv_rows_ref(q, k, v, do, 0.3, 0, 1, rows, mode, cu)
    np.testing.assert_allclose(dk, r["dk"][0, 1, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, r["dv"][0, 1, rows], rtol=1e-12, atol=1e-13)


def test_heads_selection_computes_only_those_heads():
    B, H, S, D = 2, 2, 8, 4
    q, k, v, do = _qkvdo(B, H, S, D, 19)
    full = attention_bwd_ref(q, k, v, do, 0.3)
    part = attention_bwd_ref(q, k, v, do, 0.3, heads=[(1, 0)])
    for name in full:
        assert np.array_equal(full[name][1, 0], part[name][1, 0])
        assert np.all(np.isnan(part[name][0, 0]))


# ---------------------------------------------------------------- grouped-query attention

def _gqa_inputs(B, H, H_kv, S, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, D))
    k = rng.standard_normal((B, H_kv, S, D))
    v = rng.standard_normal((B, H_kv, S, D))
    do = rng.standard_normal((B, H, S, D))
    return q, k, v, do


@pytest.mark.parametrize("mode", [MASK_CAUSAL, MASK_DOC_CAUSAL])
@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 2), (4, 1)])
def test_gqa_equals_mha_on_repeated_kv(mode, H, H_kv):
    """Grouped heads = plain attention with each K/V head repeated for its G query
    heads (consecutive heads share one K/V head); dK, dV = sums over the copies."""
    B, S, D = 2, 20, 8
    q, k, v, do = _gqa_inputs(B, H, H_kv, S, D, 20 + H + H_kv)
    G = H // H_kv
    cu = CU_SMALL if mode == MASK_DOC_CAUSAL else None
    r = attention_bwd_ref(q, k, v, do, 0.35, mode, cu)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    m = attention_bwd_ref(q, kr, vr, do, 0.35, mode, cu)
    for name in ("o", "lse", "dq", "delta"):
        np.testing.assert_allclose(r[name], m[name], rtol=1e-13, atol=1e-14)
    for name in ("dk", "dv"):
        summed = m[name].reshape(B, H_kv, G, S, D).sum(axis=2)
        np.testing.assert_allclose(r[name], summed, rtol=1e-12, atol=1e-13)
    o, lse = attention_fwd_ref(q, k, v, 0.35, mode, cu)
    np.testing.assert_allclose(o, m["o"], rtol=1e-13, atol=1e-14)


def test_gqa_matches_torch_enable_gqa_and_autograd():
    """PyTorch's CPU SDPA with enable_gqa=True in float64, differentiated by autograd."""
    torch = pytest.importorskip("torch")
    B, H, H_kv, S, D = 2, 6, 2, 18, 16
    q, k, v, do = _gqa_inputs(B, H, H_kv, S, D, 31)
    scale = 1 / math.sqrt(D)
    r = attention_bwd_ref(q, k, v, do, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale,
                                                          enable_gqa=True)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(r["o"], to.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_gqa_gradients_match_central_differences():
    """dK and dV of a shared K/V head against central differences of L = sum(O * dO)."""
    B, H, H_kv, S, D = 1, 4, 2, 10, 4
    q, k, v, do = _gqa_inputs(B, H, H_kv, S, D, 32)
    scale = 0.5

    def loss():
        o, _ = attention_fwd_ref(q, k, v, scale)
        return float(np.sum(o * do))

    r = attention_bwd_ref(q, k, v, do, scale)
    h = 1e-6
    for name, x in (("dk", k), ("dv", v), ("dq", q)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            orig = x[idx]
            x[idx] = orig + h
            lp = loss()
            x[idx] = orig - h
            lm = loss()
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - r[name])) / np.max(np.abs(r[name]))
        assert err < 1e-7, (name, err)


def test_gqa_rejects_heads_that_do_not_divide():
    q, k, v, do = _gqa_inputs(1, 4, 3, 8, 4, 33)
    with pytest.raises(ValueError):
        attention_fwd_ref(q, k, v, 0.5)
    q, k, v, do = _gqa_inputs(1, 4, 2, 8, 4, 33)
    with pytest.raises(ValueError):
        attention_bwd_ref(q, k, v, do, 0.5, heads=[(0, 1)])


# ---------------------------------------------------------------- decode with a K/V cache

def test_decode_equals_last_row_of_causal_attention():
    """The decode step for a query at position n-1 is row n-1 of causal attention over
    the first n tokens (per head, with grouped K/V heads repeated)."""
    from oracle import attention_decode_ref
    rng = np.random.default_rng(40)
    B, H, H_kv, S_max, D = 3, 4, 2, 24, 8
    G = H // H_kv
    k = rng.standard_normal((B, H_kv, S_max, D))
    v = rng.standard_normal((B, H_kv, S_max, D))
    q_seq = rng.standard_normal((B, H, S_max, D))
    lens = [24, 1, 13]
    q = np.stack([q_seq[b, :, lens[b] - 1] for b in range(B)])
    o, lse = attention_decode_ref(q, k, v, lens, 0.4)
    for b, n in enumerate(lens):
        kr = np.repeat(k[b:b + 1, :, :n], G, axis=1)
        vr = np.repeat(v[b:b + 1, :, :n], G, axis=1)
        fo, flse = attention_fwd_ref(q_seq[b:b + 1, :, :n], kr, vr, 0.4)
        np.testing.assert_allclose(o[b], fo[0, :, n - 1], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[b], flse[0, :, n - 1], rtol=1e-13, atol=1e-14)


def test_decode_matches_torch_sdpa():
    """One query attending every cached key: PyTorch's CPU SDPA (no mask) in float64."""
    torch = pytest.importorskip("torch")
    from oracle import attention_decode_ref
    rng = np.random.default_rng(41)
    B, H, H_kv, S_max, D = 2, 8, 2, 40, 16
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S_max, D))
    v = rng.standard_normal((B, H_kv, S_max, D))
    lens = [40, 17]
    o, _ = attention_decode_ref(q, k, v, lens, 0.25)
    for b, n in enumerate(lens):
        to = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b][None, :, None]), torch.tensor(k[b][None, :, :n]), torch.tensor(v[b][None, :, :n]),
            scale=0.25, enable_gqa=True)
        np.testing.assert_allclose(o[b], to.numpy()[0, :, 0], rtol=1e-12, atol=1e-13)


def test_decode_single_key_and_constant_values():
    from oracle import attention_decode_ref
    rng = np.random.default_rng(42)
    q = rng.standard_normal((1, 2, 8))
    k = rng.standard_normal((1, 2, 5, 8))
    v = rng.standard_normal((1, 2, 5, 8))
    o, lse = attention_decode_ref(q, k, v, [1], 0.5)       # one key: O = V_0, LSE = scale q.k_0
    np.testing.assert_allclose(o[0], v[0, :, 0], rtol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * np.einsum("hd,hd->h", q[0], k[0, :, 0]), rtol=1e-14)
    o, _ = attention_decode_ref(q, k, np.ones_like(v), [5], 0.5)  # V = 1 -> O = 1
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)
