"""The seeded generator: determinism, bf16 rounding, document boundaries, pair counts."""
import numpy as np
import pytest

from oracle import MASK_DOC_CAUSAL, allowed_mask
from workload import CONFIGS, allowed_pair_count, make_cu_seqlens, make_inputs, round_to_bf16


def test_same_seed_same_tensors():
    cfg = CONFIGS["lm12m_ctx512"]
    a = make_inputs(cfg, 3, shape=(2, 2, 64, 64))
    b = make_inputs(cfg, 3, shape=(2, 2, 64, 64))
    c = make_inputs(cfg, 4, shape=(2, 2, 64, 64))
    for name in ("q", "k", "v", "do"):
        assert np.array_equal(a[name], b[name])
        assert not np.array_equal(a[name], c[name])


def test_qkv_scale_applies_to_qkv_only():
    cfg = CONFIGS["lm12m_ctx512"]
    x = make_inputs(cfg, 5, shape=(1, 4, 256, 64))
    assert 0.6 < np.std(x["q"]) < 0.8
    assert 0.9 < np.std(x["do"]) < 1.1


def test_bf16_rounding_matches_torch_cast():
    """Round-to-nearest-even to bf16, checked against PyTorch's float32 -> bfloat16 cast."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact ties: the 17th bit set, lower bits clear, both parities
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2.0 ** -130], np.float32)])
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_inputs_are_representable():
    torch = pytest.importorskip("torch")
    x = make_inputs(CONFIGS["lm237m_ctx1024"], 1, shape=(1, 2, 64, 64))
    for name in ("q", "k", "v", "do"):
        t = torch.from_numpy(x[name])
        assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t)


@pytest.mark.parametrize("seed", [0, 1, 500, 12345])
def test_cu_seqlens_invariants(seed):
    cu = make_cu_seqlens(8192, 32, 1024, seed)
    lens = np.diff(cu)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == 8192
    assert np.all(lens >= 1) and np.all(lens <= 1024)
    assert np.all(lens[:-1] >= 32)


def test_cu_seqlens_known_draw():
    """The first draw from default_rng(0) in [32, 1024] is 876, ... (16 documents, last 431)."""
    cu = make_cu_seqlens(8192, 32, 1024, 0)
    lens = np.diff(cu)
    assert len(lens) == 16 and lens[0] == 876 and lens[1] == 664 and lens[-1] == 431
    assert allowed_pair_count(8192, 1, 1, cu) == 2836311


@pytest.mark.parametrize("S,cu", [(1, None), (7, None), (64, None), (20, [0, 5, 6, 13, 20]), (9, [0, 9])])
def test_pair_count_brute_force(S, cu):
    mode = MASK_DOC_CAUSAL if cu is not None else 0
    assert allowed_pair_count(S, 2, 3, cu) == 6 * int(allowed_mask(S, mode, cu).sum())


def test_packed_config_draw():
    x = make_inputs(CONFIGS["packed_docs8192"], 5)
    cu = x["cu_seqlens"]
    assert x["q"].shape == (1, 16, 8192, 64)
    assert cu[-1] == 8192 and len(cu) >= 9


def test_grouped_query_config_draws_fewer_kv_heads():
    cfg = CONFIGS["lm237m_ctx1024_gqa4"]
    small = make_inputs(cfg, 6, shape=(1, 4, 8, 64))  # an explicit shape keeps K/V at H heads
    assert small["k"].shape == (1, 4, 8, 64)
    from dataclasses import replace
    tiny = replace(cfg, B=1, S=8)
    x = make_inputs(tiny, 6)
    assert x["q"].shape == (1, 16, 8, 64) and x["do"].shape == (1, 16, 8, 64)
    assert x["k"].shape == (1, 4, 8, 64) and x["v"].shape == (1, 4, 8, 64)


def test_fp16_rounding_is_nearest_even():
    """Round-to-nearest-even to IEEE half: every result is representable, lies within
    half a unit in the last place of the input, and equals PyTorch's float32 -> float16
    cast on inputs that are exact in float32 (PyTorch's float64 -> float16 cast rounds
    twice, through float32, so it is not the reference for float64 inputs)."""
    torch = pytest.importorskip("torch")
    from workload import round_to_f16
    x = np.random.default_rng(3).standard_normal(10000) * np.logspace(-4, 4, 10000)
    r = round_to_f16(x).astype(np.float64)
    assert np.array_equal(r, r.astype(np.float16).astype(np.float64))
    ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(x - r) <= ulp / 2)
    x32 = x.astype(np.float32)
    ref = torch.tensor(x32).to(torch.float16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_f16(x32), ref)
