"""Seeded synthetic attention workloads.

The pages train small transformers on text corpora that are not available here
(TinyStories, Spanish Wikipedia, WikiText-103, FineWeb-Edu).  What reaches the
attention kernel is four activation tensors Q, K, V and dO of shape
[B, H, S, D]; these are stood in for by i.i.d. standard-normal draws at the
shapes of the five workloads below.  Packed short documents (Cort33x,
"Preserving context in the data") are described by cumulative sequence
boundaries ``cu_seqlens``.

Recipe (stated once so that every consumer draws the same numbers):

* generator ``numpy.random.default_rng(seed)`` (PCG64);
* draw ``standard_normal`` float64 arrays in the order Q, K, V, dO, each a full
  C-order [B, H, S, D] array (K and V [B, H_kv, S, D] for grouped-query
  workloads);
* multiply Q, K, V (not dO) by ``qkv_scale``;
* round to the input dtype (bf16: round-to-nearest-even from float32; fp16:
  round-to-nearest-even from float64; fp32:
  round-to-nearest from float64);
* document lengths for the packed workload come from a separate generator
  ``default_rng(doc_seed)``: integers uniform in [lo, hi] (both inclusive) are
  drawn until their sum reaches the total; the last length is cut so the sum
  is exactly the total.

Inputs of billions of elements (the largest shapes the kernels accept) are too
big to draw on the host; ``make_inputs_device`` draws them on the GPU instead:
a ``torch.Generator`` on that device seeded with ``seed``, float32
``torch.randn`` tensors in the order Q, K, V, dO, Q/K/V multiplied by
``qkv_scale``, then converted (round-to-nearest-even) to the input dtype.  The
oracle is given slices of those tensors copied to the host, which are exactly
the values the kernels read.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK_CAUSAL = 0
MASK_DOC_CAUSAL = 1


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str  # "f32", "bf16" or "f16": the dtype of Q, K, V and dO
    qkv_scale: float = 1.0
    mask_mode: int = MASK_CAUSAL
    doc_len_range: tuple | None = None  # (lo, hi) inclusive, packed mode only
    doc_seed: int = 500
    H_kv: int | None = None  # key/value heads (grouped-query attention); None = H
    rope: bool = False       # rotary position embedding of q and k before attention
    out16: bool = False      # O, dQ, dK, dV stored in the (16-bit) input dtype instead of fp32
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """Softmax temperature 1/sqrt(D) (Vaswani et al.; the tiny fp32 case states it)."""
        return 1.0 / math.sqrt(self.D)


# The five workloads.  Shapes follow the models on the pages: the 12M-class
# model at context 512 (Forge, benchmarks), the 237M 30-layer model with head
# dim 64 at context 1024 (ARK, model table), a long-context window of 8192
# tokens (Cort33x, 2K-8K sequence lengths) and packed short documents
# (Cort33x, "Preserving context in the data").
CONFIGS = {
    "tiny_f32": AttnConfig("tiny_f32", B=1, H=2, S=64, D=32, dtype="f32",
                           note="tiny fp32 causal case, parity only"),
    "lm12m_ctx512": AttnConfig("lm12m_ctx512", B=16, H=6, S=512, D=64, dtype="bf16",
                               qkv_scale=1.0 / math.sqrt(2.0),
                               note="12M-class LM attention layer"),
    "lm237m_ctx1024": AttnConfig("lm237m_ctx1024", B=8, H=16, S=1024, D=64, dtype="bf16",
                                 note="237M-class 30-layer LM, one attention layer"),
    "long_ctx8192": AttnConfig("long_ctx8192", B=1, H=16, S=8192, D=128, dtype="bf16",
                               note="long-context training window"),
    "packed_docs8192": AttnConfig("packed_docs8192", B=1, H=16, S=8192, D=64, dtype="bf16",
                                  mask_mode=MASK_DOC_CAUSAL, doc_len_range=(32, 1024),
                                  note="packed short documents, block-diagonal causal"),
    # Grouped-query attention (Forge, "Architecture": attention with GQA): the
    # context-1024 shape with 4 key/value heads for the 16 query heads.
    "lm237m_ctx1024_gqa4": AttnConfig("lm237m_ctx1024_gqa4", B=8, H=16, S=1024, D=64, dtype="bf16", H_kv=4,
                                      note="237M-class layer with grouped-query attention"),
    # ... and the long-context window with 4 key/value heads for its 16 query heads.
    "long_ctx8192_gqa4": AttnConfig("long_ctx8192_gqa4", B=1, H=16, S=8192, D=128, dtype="bf16", H_kv=4,
                                    note="long-context window with grouped-query attention"),
    # The same layer with rotary position embedding of q and k (ARK, model
    # table: RoPE; Forge, "Architecture": attention with RoPE), base 10000.
    "lm237m_ctx1024_rope": AttnConfig("lm237m_ctx1024_rope", B=8, H=16, S=1024, D=64, dtype="bf16", rope=True,
                                      note="237M-class layer with RoPE on q and k"),
    # The same layer with O, dQ, dK, dV stored in bf16 (what a bf16 model
    # consumes next) instead of fp32.
    "lm237m_ctx1024_out16": AttnConfig("lm237m_ctx1024_out16", B=8, H=16, S=1024, D=64, dtype="bf16", out16=True,
                                       note="237M-class layer with bf16 outputs"),
}


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) via float32; returns float32.

    The float64 draw is first rounded to float32, then the low 16 bits of the
    float32 pattern are rounded away with ties-to-even.  Inputs are finite.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def round_to_f16(x) -> np.ndarray:
    """Round to the nearest IEEE half (ties to even); returns float32 holding it."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    """Round to input dtype `dtype` ("bf16", "f16" or "f32"); returns float32."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f16":
        return round_to_f16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def make_cu_seqlens(total: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Cumulative document boundaries [0, L0, L0+L1, ..., total] as int32."""
    if total < 1 or lo < 1 or hi < lo:
        raise ValueError("need total >= 1 and 1 <= lo <= hi")
    rng = np.random.default_rng(seed)
    lengths = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lengths.append(n)
        acc += n
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return cu


def allowed_pair_count(S: int, B: int = 1, H: int = 1, cu_seqlens=None) -> int:
    """Number of (query, key) pairs the mask lets through, per the counting convention
    used for throughput: S(S+1)/2 per causal head, or the sum over documents."""
    if cu_seqlens is None:
        per_head = S * (S + 1) // 2
    else:
        lens = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
        per_head = int(np.sum(lens * (lens + 1) // 2))
    return B * H * per_head


def make_inputs(cfg: AttnConfig, seed: int, shape=None):
    """Draw Q, K, V, dO for ``cfg`` (optionally overriding (B, H, S, D) with ``shape``).

    Returns a dict with
      ``q, k, v, do``: float32 arrays holding exactly the input-dtype values,
      ``cu_seqlens``: int32 boundaries (packed mode) or None,
      ``B, H, S, D, scale, mask_mode, dtype``.
    The fp64 oracle takes ``x.astype(np.float64)``; the GPU takes the same
    values in the input dtype.
    """
    B, H, S, D = shape if shape is not None else (cfg.B, cfg.H, cfg.S, cfg.D)
    H_kv = cfg.H_kv if (cfg.H_kv is not None and shape is None) else H
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        x = rng.standard_normal((B, H_kv if name in ("k", "v") else H, S, D))
        if name != "do":
            x = x * cfg.qkv_scale
        out[name] = round_to(x, cfg.dtype)
    cu = None
    if cfg.mask_mode == MASK_DOC_CAUSAL:
        if B != 1:
            raise ValueError("packed documents use B = 1")
        lo, hi = cfg.doc_len_range
        cu = make_cu_seqlens(S, lo, hi, cfg.doc_seed)
    out.update(cu_seqlens=cu, B=B, H=H, S=S, D=D, scale=1.0 / math.sqrt(D),
               mask_mode=cfg.mask_mode, dtype=cfg.dtype)
    return out


def make_inputs_device(cfg: AttnConfig, seed: int, shape, device="cuda", H_kv=None):
    """Q, K, V, dO of ``shape`` = (B, H, S, D) drawn on ``device`` (torch tensors
    in the input dtype, K and V with ``H_kv`` heads if given), by the device
    recipe in the module docstring."""
    import torch
    B, H, S, D = shape
    H_kv = H if H_kv is None else H_kv
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cfg.dtype]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        x = torch.randn((B, H_kv if name in ("k", "v") else H, S, D), generator=g, device=device,
                        dtype=torch.float32)
        if name != "do":
            x.mul_(cfg.qkv_scale)
        out[name] = x.to(dt)
        del x
    return out


@dataclass(frozen=True)
class DecodeConfig:
    """One decode step against a key/value cache: q [B, H, D], caches [B, H_kv, S_max, D],
    every batch entry's cache filled to `length` (<= S_max)."""
    name: str
    B: int
    H: int
    H_kv: int
    S_max: int
    D: int
    dtype: str
    length: int


# Generation with the long-context model shape (16 heads of 128) over a full
# 8192-token cache (Forge, "Roadmap": generation with a key/value cache; Cort33x: 2K-8K
# training contexts), eight sequences at once.
DECODE_CONFIGS = {
    "decode_ctx8192": DecodeConfig("decode_ctx8192", B=8, H=16, H_kv=16, S_max=8192, D=128, dtype="bf16",
                                   length=8192),
}


def make_decode_inputs(cfg: DecodeConfig, seed: int, lens=None):
    """Seeded decode inputs: ``standard_normal`` draws in the order q, k_cache,
    v_cache from ``default_rng(seed)``, rounded like make_inputs; ``lens`` (int32
    [B]) defaults to ``cfg.length`` for every entry."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape in (("q", (cfg.B, cfg.H, cfg.D)), ("k", (cfg.B, cfg.H_kv, cfg.S_max, cfg.D)),
                        ("v", (cfg.B, cfg.H_kv, cfg.S_max, cfg.D))):
        x = rng.standard_normal(shape)
        out[name] = round_to(x, cfg.dtype)
    lens = np.full(cfg.B, cfg.length, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    out.update(lens=lens, scale=1.0 / math.sqrt(cfg.D), dtype=cfg.dtype)
    return out
