"""GPU parity for fp16 inputs (ATTN_DTYPE_F16: the fp16 matrix cores with fp32
accumulation, P and dS rounded to fp16) against the fp64 oracle, forward and
backward, causal and packed documents, grouped K/V heads.  Same bounds as bf16
inputs (tests/gpu_util.py)."""
import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL
from tests.gpu_util import compare, log, oracle, run_hip
from workload import CONFIGS, AttnConfig, make_cu_seqlens, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def f16_inputs(B, H, S, D, seed, H_kv=None):
    x = make_inputs(AttnConfig("f16", B=B, H=H, S=S, D=D, dtype="f16"), seed, shape=(B, H, S, D))
    if H_kv is not None:
        x["k"] = np.ascontiguousarray(x["k"][:, :H_kv])
        x["v"] = np.ascontiguousarray(x["v"][:, :H_kv])
    return x


@pytest.mark.parametrize("B,H,S,D", [(2, 4, 700, 64), (1, 2, 1000, 128), (3, 2, 257, 32), (1, 1, 1, 64),
                                     (2, 3, 130, 128)])
def test_fp16_parity(B, H, S, D):
    log(f"[f16] B{B} H{H} S{S} D{D}")
    x = f16_inputs(B, H, S, D, 300 + S + D)
    compare(run_hip(x), oracle(x), "f16", tag=f"f16 B{B} H{H} S{S} D{D}")


def test_fp16_full_ctx1024_shape():
    """The 237M-class layer shape (B8 H16 S1024 D64) in fp16, every output element."""
    c = CONFIGS["lm237m_ctx1024"]
    log("[f16] B8 H16 S1024 D64")
    x = f16_inputs(c.B, c.H, c.S, c.D, 3)
    compare(run_hip(x), oracle(x), "f16", tag="f16 ctx1024")


@pytest.mark.parametrize("D", [64, 128])
def test_fp16_packed_documents(D):
    cu = make_cu_seqlens(900, 1, 300, 61 + D)
    log(f"[f16] packed ({len(cu) - 1} docs) D{D}")
    x = f16_inputs(1, 4, int(cu[-1]), D, 62 + D)
    x["cu_seqlens"] = cu
    x["mask_mode"] = MASK_DOC_CAUSAL
    compare(run_hip(x), oracle(x), "f16", tag=f"f16 packed D{D}")


def test_fp16_grouped_heads():
    log("[f16] B2 H8 H_kv2 S400 D64")
    x = f16_inputs(2, 8, 400, 64, 63, H_kv=2)
    compare(run_hip(x), oracle(x), "f16", tag="f16 gqa")


def test_fp16_bitwise_reproducible():
    x = f16_inputs(1, 4, 513, 64, 64)
    log("[f16] reproducibility")
    a = run_hip(x)
    b = run_hip(x)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert bool((a[n] == b[n]).all()), n
