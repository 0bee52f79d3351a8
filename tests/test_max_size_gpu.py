"""GPU parity at the largest sizes the library accepts.

* Element count: B*H*S*D must stay below 2^31; 64 x 32 x 8191 x 128 is
  2^31 - 262144.  Panels of the last heads start past 4 GiB (bf16 inputs) and
  8 GiB (fp32 outputs), so the 64-bit panel offsets are exercised.  Three whole
  heads are checked against the oracle.
* Sequence length, causal: S = 2^20 - 1 rows in one head.  The oracle checks
  sampled rows of O, LSE and dQ (each row on its own), dK and dV of the last
  keys (only the last queries reach them), and two sums over the whole head
  that hold at any size.
* Sequence length, packed documents: S = 2^22 - 1, the longest sequence whose
  fp32 output panel (S * D * 4 bytes) stays below 2^31 bytes at D = 128.
  Whole documents at both ends and in between are checked against the oracle.

Every output starts as NaN and must be finite everywhere afterwards.
Tolerances as in the other parity tests: bf16 inputs, max-abs 2e-2 on O, dQ,
dK, dV and 1e-3 on LSE.
"""
import numpy as np
import pytest

from oracle import (MASK_CAUSAL, MASK_DOC_CAUSAL, attention_bwd_ref, attention_dkdv_rows_ref,
                    attention_dq_rows_ref, attention_fwd_rows_ref)
from tests.gpu_util import compare, log, run_hip, to_device
from workload import AttnConfig, make_cu_seqlens, make_inputs, make_inputs_device

pytestmark = pytest.mark.gpu

NAMES = ("o", "lse", "dq", "dk", "dv", "delta")


@pytest.fixture(autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()
    yield
    torch.cuda.empty_cache()  # these tests hold tens of GiB


def _cfg():
    return AttnConfig("max_size", B=1, H=1, S=1, D=128, dtype="bf16")


def _all_finite(out):
    import torch
    for n, t in out.items():
        assert bool(torch.isfinite(t).all()), f"{n}: non-finite element (unwritten or overflow)"


def _host(dev, b, h, rows=slice(None)):
    """Inputs of head (b, h), rows `rows`, as [1, 1, rows, D] float64 host arrays."""
    return {n: dev[n][b:b + 1, h:h + 1, rows].double().cpu().numpy() for n in ("q", "k", "v", "do")}


def test_max_element_count_whole_heads():
    B, H, S, D = 64, 32, 8191, 128
    assert B * H * S * D == 2 ** 31 - 262144
    log(f"[max] element count B{B} H{H} S{S} D{D} bf16")
    dev = make_inputs_device(_cfg(), 4101, (B, H, S, D))
    dev.update(cu=None, max_seqlen=None)
    x = dict(B=B, H=H, S=S, D=D, k=dev["k"], mask_mode=MASK_CAUSAL, scale=D ** -0.5)
    out = run_hip(x, dev)
    _all_finite(out)
    rng = np.random.default_rng(4102)
    for b, h in [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]:
        xs = _host(dev, b, h)
        ref = attention_bwd_ref(xs["q"], xs["k"], xs["v"], xs["do"], x["scale"], MASK_CAUSAL, None)
        got = {n: out[n][b:b + 1, h:h + 1] for n in NAMES}
        compare(got, ref, "bf16", tag=f"max elements head ({b},{h})")


def test_long_sequence_causal_sampled():
    """One head of 2^20 - 1 rows.

    Besides rows checked one by one, two sums over the whole head hold exactly
    for the true gradients: every row of P sums to one, so the dV rows add up
    to the dO rows, sum_j dV_j = sum_i dO_i; and every row of dS = P o (dP -
    Delta) sums to zero, so sum_j dK_j = scale * sum_i (sum_j dS_ij) Q_i = 0.
    The kernels round P and dS to bf16 (round-to-nearest-even) before the
    products, which leaves random error: a row's rounding errors add up to
    about 2^-8/sqrt(3) * |P_i| (|P_i| the Euclidean norm of the row), and with
    these inputs |P_i|^2 is about e/i, so the dV column sums scatter by at
    most about 0.0023 * sqrt(e * ln S) ~ 0.015.  The same rounding model
    (bf16 P in the forward's O and in dV, bf16 dS in dK) evaluated in fp64 at
    S = 4096 gives standard deviations of 0.007 for both sums, growing like
    sqrt(ln S).  The bounds, 0.3 and 0.5, are over twenty times that, while
    dropping one 128-row query tile moves the dV sums by about sqrt(128) ~ 11,
    and a Delta of zero moves the dK sums by several units.
    """
    S, D = 2 ** 20 - 1, 128
    log(f"[max] long causal S{S} D{D} bf16")
    cfg = AttnConfig("long_causal", B=1, H=1, S=S, D=D, dtype="bf16")
    x = make_inputs(cfg, 4201)
    dev = to_device(x)
    out = run_hip(x, dev)
    _all_finite(out)
    o, lse, dq = (out[n][0, 0].cpu().numpy() for n in ("o", "lse", "dq"))
    rng = np.random.default_rng(4202)
    rows = sorted(set([0, 1, 127, 128, 4095, S // 2, S - 129, S - 1] + [int(r) for r in rng.integers(0, S, 2)]))
    ro, rl = attention_fwd_rows_ref(x["q"], x["k"], x["v"], x["scale"], 0, 0, rows)
    err_o, err_l = float(np.max(np.abs(o[rows] - ro))), float(np.max(np.abs(lse[rows] - rl)))
    log(f"[max] long causal rows {rows}: O {err_o:.2e} LSE {err_l:.2e}")
    assert err_o <= 2e-2 and err_l <= 1e-3
    qrows = [1, S // 2 + 5, S - 1]
    rq = attention_dq_rows_ref(x["q"], x["k"], x["v"], x["do"], x["scale"], 0, 0, qrows)
    err_q = float(np.max(np.abs(dq[qrows] - rq)))
    cols = list(range(S - 24, S))
    rk, rv = attention_dkdv_rows_ref(x["q"], x["k"], x["v"], x["do"], x["scale"], 0, 0, cols)
    dk, dv = (out[n][0, 0].cpu().numpy().astype(np.float64) for n in ("dk", "dv"))
    err_k, err_v = float(np.max(np.abs(dk[cols] - rk))), float(np.max(np.abs(dv[cols] - rv)))
    sum_v = float(np.max(np.abs(dv.sum(axis=0) - x["do"][0, 0].astype(np.float64).sum(axis=0))))
    sum_k = float(np.max(np.abs(dk.sum(axis=0))))
    log(f"[max] long causal dQ {err_q:.2e} dK {err_k:.2e} dV {err_v:.2e} sum dV-dO {sum_v:.2e} sum dK {sum_k:.2e}")
    assert err_q <= 2e-2 and err_k <= 2e-2 and err_v <= 2e-2
    assert sum_v <= 0.3 and sum_k <= 0.5


def test_max_sequence_packed_documents():
    import torch
    H, S, D = 2, 2 ** 22 - 1, 128
    assert S * D * 4 == 2 ** 31 - 512
    cu = make_cu_seqlens(S, 1, 2048, 4301)
    lens = np.diff(cu)
    log(f"[max] packed documents S{S} H{H} D{D} bf16, {len(lens)} documents")
    dev = make_inputs_device(_cfg(), 4302, (1, H, S, D))
    dev.update(cu=torch.from_numpy(cu).to("cuda"), max_seqlen=int(lens.max()))
    x = dict(B=1, H=H, S=S, D=D, k=dev["k"], mask_mode=MASK_DOC_CAUSAL, scale=D ** -0.5)
    out = run_hip(x, dev)
    _all_finite(out)
    rng = np.random.default_rng(4303)
    docs = sorted(set([0, len(lens) - 1, int(np.argmax(lens))] + [int(d) for d in rng.integers(0, len(lens), 3)]))
    for d in docs:
        ds, de = int(cu[d]), int(cu[d + 1])
        for h in range(H):
            xs = _host(dev, 0, h, slice(ds, de))
            ref = attention_bwd_ref(xs["q"], xs["k"], xs["v"], xs["do"], x["scale"], MASK_DOC_CAUSAL,
                                    np.array([0, de - ds], dtype=np.int32))
            got = {n: out[n][0:1, h:h + 1, ds:de] for n in NAMES}
            compare(got, ref, "bf16", tag=f"max packed doc {d} rows [{ds},{de}) head {h}")
