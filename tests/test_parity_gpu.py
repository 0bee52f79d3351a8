"""GPU parity: the HIP kernels through the C ABI against the fp64 oracle.

Every workload (tiny fp32, 12M-class ctx 512, 237M-class ctx 1024, long context
8192, packed documents) on several seeds, plus edge shapes (ragged tails, one
row, one head, head dims 32/64/128, both input dtypes), packed-document edge
cases, large logits, NaN propagation and NaN-poisoned outputs.
Tolerances: fp32 inputs max-abs 1e-4; bf16 inputs max-abs 2e-2 and relative
Frobenius 1e-2 per output tensor, LSE 1e-3 (tests/gpu_util.py).
"""
import math

import numpy as np
import pytest

from oracle import (MASK_CAUSAL, MASK_DOC_CAUSAL, attention_dkdv_rows_ref, attention_dq_rows_ref,
                    attention_fwd_rows_ref)
from tests.gpu_util import check_delta, compare, log, oracle, run_hip, to_device
from workload import CONFIGS, AttnConfig, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


FULL_CASES = [("tiny_f32", s) for s in (1, 11, 12, 13)] + \
             [("lm12m_ctx512", s) for s in (2, 11, 12, 13)] + \
             [("lm237m_ctx1024", s) for s in (3, 11, 12, 13)]


@pytest.mark.parametrize("cfg,seed", FULL_CASES)
def test_parity_full_oracle(cfg, seed):
    """Every element of every output against the full fp64 oracle."""
    c = CONFIGS[cfg]
    log(f"[parity] {cfg} seed={seed} B{c.B} H{c.H} S{c.S} D{c.D} {c.dtype}")
    x = make_inputs(c, seed)
    out = run_hip(x)
    ref = oracle(x)
    compare(out, ref, c.dtype, tag=f"{cfg}/{seed}")
    check_delta(out, x)


SAMPLED_CASES = [("long_ctx8192", s) for s in (4, 11, 12)] + [("packed_docs8192", s) for s in (5, 11, 12)]


@pytest.mark.parametrize("cfg,seed", SAMPLED_CASES)
def test_parity_full_size_sampled_heads(cfg, seed):
    """Full-size workloads: two whole heads against the oracle, plus, in every
    head, sampled rows of O, LSE and dQ and sampled keys of dK and dV (each
    computed on its own by the row-wise oracle), and Delta against the GPU's
    own O everywhere."""
    c = CONFIGS[cfg]
    log(f"[parity] {cfg} seed={seed} B{c.B} H{c.H} S{c.S} D{c.D} {c.dtype} (sampled heads)")
    x = make_inputs(c, seed)
    out = run_hip(x)
    rng = np.random.default_rng(seed)
    heads = [(0, int(rng.integers(0, c.H))), (0, c.H - 1)]
    ref = oracle(x, heads=heads)
    compare(out, ref, c.dtype, heads=heads, tag=f"{cfg}/{seed}")
    o = out["o"].cpu().numpy()
    lse = out["lse"].cpu().numpy()
    dq = out["dq"].cpu().numpy()
    dk = out["dk"].cpu().numpy()
    dv = out["dv"].cpu().numpy()
    cu = x["cu_seqlens"]
    for h in range(c.H):
        rows = sorted(set([0, c.S - 1] + [int(r) for r in rng.integers(0, c.S, 4)]))
        ro, rl = attention_fwd_rows_ref(x["q"], x["k"], x["v"], x["scale"], 0, h, rows, c.mask_mode, cu)
        assert np.max(np.abs(o[0, h, rows] - ro)) <= 2e-2
        assert np.max(np.abs(lse[0, h, rows] - rl)) <= 1e-3
        rq = attention_dq_rows_ref(x["q"], x["k"], x["v"], x["do"], x["scale"], 0, h, rows[:3], c.mask_mode, cu)
        assert np.max(np.abs(dq[0, h, rows[:3]] - rq)) <= 2e-2
        # dK, dV of sampled keys: the row-wise oracle visits every query that
        # reaches them, so keys late in the sequence (causal) or in a short
        # document (packed) keep it to a few hundred rows per head
        cols = _sampled_keys(rng, c.S, cu)
        rk, rv = attention_dkdv_rows_ref(x["q"], x["k"], x["v"], x["do"], x["scale"], 0, h, cols, c.mask_mode, cu)
        assert np.max(np.abs(dk[0, h, cols] - rk)) <= 2e-2, (h, cols)
        assert np.max(np.abs(dv[0, h, cols] - rv)) <= 2e-2, (h, cols)
    check_delta(out, x)


def _sampled_keys(rng, S, cu):
    """Four keys whose gradients the row-wise oracle computes from a few hundred
    query rows: the last key, two in the final 320 positions, and (packed
    documents) one in a random document of at most 400 tokens."""
    keys = {S - 1, int(rng.integers(S - 320, S)), int(rng.integers(S - 320, S))}
    if cu is None:
        keys.add(int(rng.integers(S - 160, S)))
    else:
        lens = np.diff(cu)
        short = [d for d in range(len(lens)) if 0 < lens[d] <= 400] or [int(np.argmin(np.where(lens > 0, lens, S)))]
        d = short[int(rng.integers(0, len(short)))]
        keys.add(int(rng.integers(cu[d], cu[d + 1])))
    return sorted(keys)


def _shape_cfg(dtype, D, mask_mode=MASK_CAUSAL, qkv_scale=1.0):
    return AttnConfig("edge", B=1, H=1, S=1, D=D, dtype=dtype, qkv_scale=qkv_scale, mask_mode=mask_mode)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("S", [1, 17, 100, 1000])
def test_edge_sequence_lengths(dtype, D, S):
    """Ragged tails and tiny sequences with B*H = 1."""
    log(f"[edge] S={S} D={D} {dtype}")
    x = make_inputs(_shape_cfg(dtype, D), 100 + S + D, shape=(1, 1, S, D))
    compare(run_hip(x), oracle(x), dtype, tag=f"edge S{S} D{D} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,S,D", [(2, 3, 130, 64), (3, 2, 257, 32), (1, 2, 383, 128)])
def test_multi_head_ragged(dtype, B, H, S, D):
    log(f"[edge] B{B} H{H} S{S} D{D} {dtype}")
    x = make_inputs(_shape_cfg(dtype, D), 7 * S + D, shape=(B, H, S, D))
    compare(run_hip(x), oracle(x), dtype, tag=f"B{B}H{H}S{S}D{D} {dtype}")


def _doc_inputs(dtype, D, cu, H=2, seed=0):
    cu = np.asarray(cu, dtype=np.int32)
    S = int(cu[-1])
    x = make_inputs(_shape_cfg(dtype, D), seed, shape=(1, H, S, D))
    x["cu_seqlens"] = cu
    x["mask_mode"] = MASK_DOC_CAUSAL
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_documents_with_length_one_and_ragged(dtype, D):
    cu = [0, 1, 2, 50, 51, 180, 181, 300, 429, 430]
    log(f"[doc] cu={cu} D={D} {dtype}")
    x = _doc_inputs(dtype, D, cu, seed=D)
    compare(run_hip(x), oracle(x), dtype, tag=f"doc D{D} {dtype}")


@pytest.mark.parametrize("seed", [21, 22])
def test_packed_small_random_documents(seed):
    """Packed mode at a size the oracle checks fully: 1000 tokens, lengths in [1, 300]."""
    from workload import make_cu_seqlens
    cu = make_cu_seqlens(1000, 1, 300, seed)
    log(f"[doc] random cu ({len(cu) - 1} docs) seed={seed}")
    x = _doc_inputs("bf16", 64, cu, H=4, seed=seed)
    compare(run_hip(x), oracle(x), "bf16", tag=f"doc random {seed}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_document_equals_causal_bitwise(dtype):
    S = 300
    log(f"[doc] single document vs causal {dtype}")
    x = make_inputs(_shape_cfg(dtype, 64), 31, shape=(1, 3, S, 64))
    a = run_hip(x)
    y = dict(x)
    y["cu_seqlens"] = np.array([0, S], dtype=np.int32)
    y["mask_mode"] = MASK_DOC_CAUSAL
    b = run_hip(y)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((a[n] == b[n]).all()), n


EMPTY_DOC_CU = ([0, 1, 2, 50, 51, 180, 181, 300, 429, 430],
                [0, 0, 1, 2, 2, 2, 50, 51, 180, 181, 181, 300, 429, 430, 430, 430])


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 128)])
def test_empty_documents_change_nothing(dtype, D):
    """Empty documents (repeated boundaries: first, in between, several in a
    row, last) own no rows: outputs match the oracle and are bitwise those of
    the same call without them."""
    cu, cu_e = EMPTY_DOC_CU
    log(f"[doc] empty documents D={D} {dtype}")
    x = _doc_inputs(dtype, D, cu_e, seed=5 + D)
    assert len(cu_e) - 1 > 0 and int(np.min(np.diff(cu_e))) == 0
    got = run_hip(x)
    compare(got, oracle(x), dtype, tag=f"empty docs D{D} {dtype}")
    y = dict(x)
    y["cu_seqlens"] = np.asarray(cu, dtype=np.int32)
    ref = run_hip(y)
    for n in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert bool((got[n] == ref[n]).all()), n


@pytest.mark.parametrize("B", [47, 48])
def test_dq_tile_choice_boundary(B):
    """Causal 16-bit D = 64 dQ takes 64-key tiles when B * H * ceil(S / 128)
    is under 768 workgroups and 32-key tiles from 768 on: B = 47 and 48 at
    H = 2, S = 1024 give 752 and 768.  Sampled heads against the oracle."""
    H, S, D = 2, 1024, 64
    log(f"[edge] dQ tile choice B{B} H{H} S{S} D{D} ({B * H * S // 128} workgroups)")
    x = make_inputs(_shape_cfg("bf16", D), 60 + B, shape=(B, H, S, D))
    heads = [(0, 0), (B - 1, 1), (B // 2, 0)]
    compare(run_hip(x), oracle(x, heads=heads), "bf16", heads=heads, tag=f"dq tiles B{B}")


def test_large_logits():
    """Q and K scaled by 4 (scores with standard deviation about 16, far outside
    the workloads): stresses the running-maximum rescaling.  Bounds: twice the
    16-bit rounding model's own error on this input (tests/test_bf16_model.py:
    the gradients then grow with |Q| and |K|, and O, Delta and the gradients
    inherit the rounding of a row's few dominant weights)."""
    from tests.test_bf16_model import large_logit_bounds, large_logit_inputs
    x = large_logit_inputs()
    log("[stress] large logits")
    out = run_hip(x)
    ref = oracle(x)
    bounds, model = large_logit_bounds(x)
    got = {n: out[n].cpu().numpy().astype(np.float64) for n in ("o", "lse", "dq", "dk", "dv")}
    for n, lim in bounds.items():
        err = float(np.max(np.abs(got[n] - ref[n])))
        log(f"[stress] {n}: max-abs {err:.4f} (model {model[n][0]:.4f}, bound {lim:.4f})")
        assert np.all(np.isfinite(got[n])), n
        assert err <= max(lim, 1e-3 if n == "lse" else 0.0), n
        rf = float(np.linalg.norm(got[n] - ref[n]) / np.linalg.norm(ref[n]))
        assert rf <= 1e-2, (n, rf)
    check_delta(out, x)


def test_nan_row_reaches_only_its_outputs():
    import torch
    x = make_inputs(CONFIGS["lm12m_ctx512"], 51, shape=(1, 2, 256, 64))
    dev = to_device(x)
    i = 77
    dev["q"][0, 1, i, 5] = float("nan")
    log("[nan] NaN in one query row")
    out = run_hip(x, dev=dev)
    o = out["o"].cpu().numpy()
    lse = out["lse"].cpu().numpy()
    assert np.all(np.isnan(o[0, 1, i])) and np.isnan(lse[0, 1, i])
    mask = np.ones(256, bool)
    mask[i] = False
    assert np.all(np.isfinite(o[0, 1, mask])) and np.all(np.isfinite(o[0, 0]))
    ref = oracle(x)
    assert np.max(np.abs(o[0, 1, mask] - ref["o"][0, 1, mask])) <= 2e-2
    del torch


def test_lse_may_be_null():
    import torch
    import causal_attention_amd as ca
    x = make_inputs(CONFIGS["lm12m_ctx512"], 61, shape=(1, 2, 200, 64))
    dev = to_device(x)
    o1, lse = ca.forward(dev["q"], dev["k"], dev["v"], x["scale"])
    o2 = torch.full_like(o1, float("nan"))
    ca.attn_fwd(dev["q"], dev["k"], dev["v"], o2, None, x["scale"])
    torch.cuda.synchronize()
    assert bool((o1 == o2).all())


def test_scale_is_honoured():
    """A non-default temperature reaches the kernels (checked against the oracle)."""
    x = make_inputs(CONFIGS["lm12m_ctx512"], 71, shape=(1, 2, 160, 64))
    x["scale"] = 0.3
    compare(run_hip(x), oracle(x), "bf16", tag="scale 0.3")
    assert not math.isclose(x["scale"], 1 / 8)
