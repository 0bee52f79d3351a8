"""GPU: the work-ranked packed-document schedule.

Packed documents are scheduled one of two ways (attn_device.h, doc_tile): with
at most 256 documents and 256 tiles of the longest document, a head's tiles
are ranked by work across all documents and dealt heaviest first; otherwise
one block per (tile of the longest document, document, head), empty tiles
exiting at once.  The schedule only decides which workgroup computes which
tile, not how a tile is computed, so both must give bitwise the same
outputs.  The tests switch schedules without changing the attention: empty
documents appended after the last token (they own no rows) push the document
count past 256, and a max_seqlen above the longest document (the contract
only bounds it below) pushes the tile count past 256.  The ranked outputs are
also checked against the fp64 oracle.
"""
import numpy as np
import pytest

from tests.gpu_util import compare, log, oracle, run_hip, to_device
from workload import AttnConfig, make_cu_seqlens, make_inputs
from workload.synth import MASK_DOC_CAUSAL

pytestmark = pytest.mark.gpu

NAMES = ("o", "lse", "dq", "dk", "dv", "delta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_attention_amd as ca
    ca.load_library()


def _inputs(dtype, D, cu, H, seed):
    cfg = AttnConfig("doc_schedule", B=1, H=H, S=int(cu[-1]), D=D, dtype=dtype)
    x = make_inputs(cfg, seed)
    x["cu_seqlens"] = np.asarray(cu, dtype=np.int32)
    x["mask_mode"] = MASK_DOC_CAUSAL
    return x


def _same(a, b, tag):
    for n in NAMES:
        assert bool((a[n] == b[n]).all()), f"{tag}: {n} differs between the two schedules"


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("f32", 32)])
def test_more_than_256_documents_bitwise(dtype, D):
    """The same packing with about 30 documents (ranked) and with empty ones
    appended up to 260 documents (per-document grid)."""
    cu = make_cu_seqlens(2000, 1, 120, 40 + D)
    n_docs = len(cu) - 1
    log(f"[schedule] {n_docs} documents vs 260, {dtype} D={D}")
    x = _inputs(dtype, D, cu, H=3, seed=D)
    ranked = run_hip(x)
    compare(ranked, oracle(x), dtype, tag=f"ranked {dtype} D{D}")
    y = dict(x)
    y["cu_seqlens"] = np.concatenate([np.asarray(cu, dtype=np.int32), np.full(260 - n_docs, cu[-1], dtype=np.int32)])
    assert len(y["cu_seqlens"]) - 1 > 256
    _same(ranked, run_hip(y), f"{dtype} D{D}")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64)])
def test_256_documents_bitwise(dtype, D):
    """Exactly 256 documents (the ranked limit: every lane of the rank scan
    holds four documents, so documents 64-255 exercise its later chunks),
    some of them empty and a few of several tiles, against the same rows with
    one more empty document (257: per-document grid)."""
    lens = np.random.default_rng(256).integers(0, 24, 256)
    lens[[3, 64, 130, 200, 255]] = 0
    lens[[70, 150, 190, 250]] = [300, 140, 260, 129]  # several tiles, in the later chunks
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    log(f"[schedule] 256 documents ({int(cu[-1])} tokens) vs 257, {dtype} D={D}")
    x = _inputs(dtype, D, cu, H=2, seed=9)
    ranked = run_hip(x)
    compare(ranked, oracle(x), dtype, tag=f"256 docs {dtype} D{D}")
    y = dict(x)
    y["cu_seqlens"] = np.concatenate([cu, [cu[-1]]]).astype(np.int32)
    _same(ranked, run_hip(y), f"256 docs {dtype} D{D}")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128)])
def test_max_seqlen_past_rank_limit_bitwise(dtype, D):
    """33,000 tokens in documents of at most 1,500: max_seqlen = the longest
    document (ranked) against max_seqlen = S (258 tiles of 128 rows: the
    per-document grid in every kernel)."""
    cu = make_cu_seqlens(33000, 200, 1500, 77)
    log(f"[schedule] max_seqlen past the rank limit: {len(cu) - 1} documents, {dtype} D={D}")
    x = _inputs(dtype, D, cu, H=1, seed=5)
    dev = to_device(x)
    ranked = run_hip(x, dev=dev)
    dev["max_seqlen"] = int(cu[-1])
    assert (dev["max_seqlen"] + 127) // 128 > 256
    _same(ranked, run_hip(x, dev=dev), f"{dtype} D{D} max_seqlen=S")
