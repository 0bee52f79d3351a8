"""The C-ABI library without a GPU: it loads, exports what the header declares, and
rejects invalid arguments before making any HIP call."""
import ctypes
import re

import pytest

import causal_attention_amd as ca
from causal_attention_amd import _binding

FAKE = 0x10000  # never dereferenced: every call below fails validation first, or is made without a GPU


def _has_gpu():
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="module")
def lib():
    return ca.load_library()


def test_exports_every_header_function(lib):
    names = ca.header_functions()
    assert set(names) == set(_binding.SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name


def test_header_status_codes_match_binding():
    with open(_binding.HEADER_PATH) as f:
        text = f.read()
    codes = dict((name, int(val)) for name, val in re.findall(r"(ATTN_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text))
    assert {v: k for k, v in codes.items()} == _binding.STATUS_NAMES


def test_abi_version(lib):
    assert lib.attn_abi_version() == 192


def test_build_id_is_the_source_digest(lib):
    """The library carries the digest of the sources it was built from, and it
    is the digest of the tree it sits in (load_library refuses it otherwise)."""
    from causal_attention_amd.build import source_digest
    built = lib.attn_build_id().decode()
    assert re.fullmatch(r"[0-9a-f]{16}", built)
    assert built == source_digest() == ca.build_id()


def test_clock_probe_rejects_invalid_arguments(lib):
    assert lib.attn_clock_probe(None, 100, None) == -1
    assert lib.attn_clock_probe(FAKE, 0, None) == -2


def test_stale_library_is_refused(lib, monkeypatch):
    """A library whose build id differs from the tree's sources does not load."""
    from causal_attention_amd import build as _build
    monkeypatch.setattr(_build, "source_digest", lambda: "0123456789abcdef")
    saved = _binding._lib
    _binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="built from other sources"):
            _binding.load_library()
    finally:
        _binding._lib = saved


def test_status_strings(lib):
    for code in list(_binding.STATUS_NAMES) + [-100, 7]:
        s = lib.attn_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.attn_status_string(-3) == b"head dimension D must be 32, 64 or 128"


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=2, S=64, D=64, scale=0.125, mask=0,
             cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"], a["scale"],
                        a["mask"], a["cu"], a["n"], a["mx"], a["dtype"], a["stream"])


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE,
             B=1, H=2, S=64, D=64, scale=0.125, mask=0, cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                        a["delta"], a["B"], a["H"], a["S"], a["D"], a["scale"], a["mask"], a["cu"], a["n"],
                        a["mx"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(D=48), -3), (dict(D=256), -3), (dict(D=0), -3),
    (dict(dtype=3), -4), (dict(dtype=-1), -4),
    (dict(mask=2), -5), (dict(mask=-1), -5),
    (dict(mask=1, cu=None, n=1, mx=64), -1),
    (dict(mask=1, cu=FAKE, n=1, mx=64, B=2), -6),
    (dict(mask=1, cu=FAKE, n=0, mx=64), -6),
    (dict(mask=1, cu=FAKE, n=-1, mx=64), -6),
    (dict(mask=1, cu=FAKE, n=2, mx=0), -6),
    (dict(mask=1, cu=FAKE, n=2, mx=65), -6),
    (dict(S=0), -2), (dict(S=-5), -2), (dict(B=0), -2), (dict(H=0), -2),
    (dict(B=1024, H=1024, S=2048), -2),
    (dict(scale=float("nan")), -9), (dict(scale=float("inf")), -9), (dict(scale=0.0), -9),
    (dict(scale=-0.1), -9),
])
def test_fwd_rejects_invalid_arguments(lib, kw, code):
    assert _fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), -1), (dict(lse=None), -1), (dict(delta=None), -1), (dict(dq=None), -1),
    (dict(dk=None), -1), (dict(dv=None), -1), (dict(o=None), -1),
    (dict(D=16), -3), (dict(dtype=5), -4), (dict(mask=3), -5),
    (dict(mask=1, cu=FAKE, n=1, mx=64, B=3), -6), (dict(S=0), -2), (dict(scale=float("nan")), -9),
])
def test_bwd_rejects_invalid_arguments(lib, kw, code):
    assert _bwd(lib, **kw) == code


def test_stage_entry_points_reject_invalid_arguments(lib):
    assert lib.attn_bwd_preprocess(FAKE, FAKE, None, 1, 1, 64, 64, 1, None) == -1
    assert lib.attn_bwd_preprocess(FAKE, FAKE, FAKE, 1, 1, 64, 40, 1, None) == -3
    assert lib.attn_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 64, 0.1, 0,
                             None, 0, 0, 1, None) == -1
    assert lib.attn_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 1,
                             None, 0, 0, 1, None) == -1
    assert lib.attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0,
                           None, 0, 0, 7, None) == -4
    assert lib.attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, -1.0, 0,
                           None, 0, 0, 1, None) == -9
    dqd = lib.attn_bwd_dq_delta
    assert dqd(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0, None, 0, 0, 1, None) == -1
    assert dqd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 64, 0.1, 0, None, 0, 0, 1, None) == -1
    assert dqd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 48, 0.1, 0, None, 0, 0, 1, None) == -3
    assert dqd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 4, None, 0, 0, 1, None) == -5
    assert dqd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 64, 64, 0.1, 1, FAKE, 1, 64, 1, None) == -6
    assert dqd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.0, 0, None, 0, 0, 1, None) == -9


def _fwd_gqa(lib, H_kv, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=4, S=64, D=64, scale=0.125, mask=0,
             cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], H_kv, a["S"], a["D"],
                            a["scale"], a["mask"], a["cu"], a["n"], a["mx"], a["dtype"], a["stream"])


def _bwd_gqa(lib, H_kv, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE,
             B=1, H=4, S=64, D=64, scale=0.125, mask=0, cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_bwd_gqa(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                            a["delta"], a["B"], a["H"], H_kv, a["S"], a["D"], a["scale"], a["mask"], a["cu"],
                            a["n"], a["mx"], a["dtype"], a["stream"])


@pytest.mark.parametrize("H,H_kv", [(4, 0), (4, 3), (4, 5), (4, -1), (6, 4)])
def test_gqa_rejects_head_counts_that_do_not_divide(lib, H, H_kv):
    assert _fwd_gqa(lib, H_kv, H=H) == -10
    assert _bwd_gqa(lib, H_kv, H=H) == -10


def test_gqa_checks_the_rest_as_the_plain_calls(lib):
    assert _fwd_gqa(lib, 2, q=None) == -1
    assert _fwd_gqa(lib, 2, D=40) == -3
    assert _bwd_gqa(lib, 2, dk=None) == -1
    assert _bwd_gqa(lib, 1, mask=1, cu=FAKE, n=1, mx=64, B=2) == -6
    assert _bwd_gqa(lib, 2, scale=0.0) == -9


def _bwd_gqa_ws(lib, H_kv, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE,
             B=1, H=16, S=8192, D=128, scale=0.125, mask=0, cu=None, n=0, mx=0, dtype=1, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(kw)
    return lib.attn_bwd_gqa_ws(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                               a["delta"], a["B"], a["H"], H_kv, a["S"], a["D"], a["scale"], a["mask"], a["cu"],
                               a["n"], a["mx"], a["dtype"], a["ws"], a["wsb"], a["stream"])


def test_gqa_workspace_size(lib):
    """Parts P: the smallest divisor of the group size G that brings the 64-key
    units (B * H_kv * ceil(S / 64)) to 1024, else G; 2 * P * B * H_kv * S * D * 4
    bytes.  16-bit inputs, D = 128, even groups under 1024 units only."""
    f = lib.attn_bwd_gqa_workspace_bytes
    # B1 H16/4 S8192: 512 units, P = 2
    assert f(1, 16, 4, 8192, 128, 0, 0, 0, 1) == 2 * 2 * 1 * 4 * 8192 * 128 * 4
    # B1 H16/1 S8192: 128 units, P = 8 (2 and 4 fall short)
    assert f(1, 16, 1, 8192, 128, 0, 0, 0, 2) == 8 * 2 * 1 * 1 * 8192 * 128 * 4
    # B1 H8/2 S2048: 64 units, no divisor reaches 1024: P = G = 4
    assert f(1, 8, 2, 2048, 128, 0, 0, 0, 1) == 4 * 2 * 1 * 2 * 2048 * 128 * 4
    # packed documents: 4 documents, longest 1000 -> 4 * 4 * 16 = 256 units, P = 4
    assert f(1, 16, 4, 3000, 128, 1, 4, 1000, 1) == 4 * 2 * 1 * 4 * 3000 * 128 * 4
    # D <= 64: groups of 8 and more, 128-key units: B8 H16/1 S1024 -> 64 units, P = 16
    assert f(8, 16, 1, 1024, 64, 0, 0, 0, 1) == 16 * 2 * 8 * 1 * 1024 * 64 * 4
    # B1 H16/2 S8192 D32: 128 units, P = 8
    assert f(1, 16, 2, 8192, 32, 0, 0, 0, 2) == 8 * 2 * 1 * 2 * 8192 * 32 * 4
    # no split: fp32 inputs, D = 64 with a group under 8, odd group at D = 128, plain heads,
    # 1024 units and more
    assert f(1, 16, 4, 8192, 128, 0, 0, 0, 0) == 0
    assert f(1, 16, 4, 8192, 64, 0, 0, 0, 1) == 0
    assert f(16, 16, 1, 8192, 64, 0, 0, 0, 1) == 0
    assert f(1, 12, 4, 8192, 128, 0, 0, 0, 1) == 0
    assert f(1, 16, 16, 8192, 128, 0, 0, 0, 1) == 0
    assert f(1, 16, 8, 8192, 128, 0, 0, 0, 1) == 0
    # invalid arguments: 0 (the call reports them)
    assert f(1, 16, 3, 8192, 128, 0, 0, 0, 1) == 0
    assert f(0, 16, 4, 8192, 128, 0, 0, 0, 1) == 0
    assert f(1, 16, 4, 8192, 128, 1, 0, 1000, 1) == 0


def test_gqa_workspace_is_checked(lib):
    need = lib.attn_bwd_gqa_workspace_bytes(1, 16, 4, 8192, 128, 0, 0, 0, 1)
    assert _bwd_gqa_ws(lib, 4, ws=None) == -11
    assert _bwd_gqa_ws(lib, 4, wsb=need - 1) == -11
    assert _bwd_gqa_ws(lib, 4, ws=FAKE + 8) == -11  # not 16-byte aligned
    # the other checks come first, as in attn_bwd_gqa
    assert _bwd_gqa_ws(lib, 3, ws=None) == -10
    assert _bwd_gqa_ws(lib, 4, dk=None) == -1
    assert _bwd_gqa_ws(lib, 4, scale=0.0) == -9
    # where no split applies the workspace may be NULL (the call fails later only for lack of a GPU;
    # with one it would launch on the fake pointers, so it is made only where there is none)
    if not _has_gpu():
        assert _bwd_gqa_ws(lib, 4, D=64, ws=None, wsb=0, S=64) == -7


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, o=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40, B=2, H=8, H_kv=2,
             S_max=4096, D=64, scale=0.125, max_len=4096, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"], a["H"],
                           a["H_kv"], a["S_max"], a["D"], a["scale"], a["max_len"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(lens=None), -1), (dict(o=None), -1),
    (dict(D=48), -3), (dict(dtype=3), -4), (dict(H_kv=3), -10), (dict(H_kv=0), -10),
    (dict(H=64, H_kv=1), -8),                       # a group wider than one wave's 32 columns
    (dict(max_len=0), -2), (dict(max_len=4097), -2), (dict(S_max=0), -2), (dict(B=0), -2),
    (dict(scale=float("inf")), -9), (dict(ws=None), -11), (dict(wsb=16), -11),
])
def test_decode_rejects_invalid_arguments(lib, kw, code):
    assert _decode(lib, **kw) == code


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, o=FAKE, lse=FAKE, B=2, H=8, H_kv=2, S_max=4096, D=64, scale=0.125,
             max_len=4096, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_decode_noalloc(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                                   a["S_max"], a["D"], a["scale"], a["max_len"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(lens=None), -1), (dict(o=None), -1), (dict(D=48), -3), (dict(dtype=3), -4),
    (dict(H_kv=3), -10), (dict(H=64, H_kv=1), -8), (dict(max_len=0), -2), (dict(max_len=4097), -2),
    (dict(scale=float("nan")), -9),
    # 1024 chunks x 32 query heads x 129 floats: more than the 16 MiB scratch
    (dict(B=1, H=32, H_kv=1, S_max=65536, max_len=65536, D=128), -14),
])
def test_decode_noalloc_rejects_invalid_arguments(lib, kw, code):
    assert _decode_noalloc(lib, **kw) == code


def test_decode_noalloc_scratch_limit(lib):
    """The refusal follows the workspace attn_decode would need: the largest
    split that fits passes validation (and fails later only for lack of a GPU)."""
    assert lib.attn_decode_workspace_bytes(1, 32, 1, 128, 65536) > ca.ATTN_DECODE_SCRATCH_BYTES
    assert lib.attn_decode_workspace_bytes(1, 16, 1, 128, 65536) <= ca.ATTN_DECODE_SCRATCH_BYTES
    if not _has_gpu():
        assert _decode_noalloc(lib, B=1, H=16, H_kv=1, S_max=65536, max_len=65536, D=128) == -7
    with open(_binding.HEADER_PATH) as f:
        assert "#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)" in f.read()
    assert ca.ATTN_DECODE_SCRATCH_BYTES == 16 << 20


def test_decode_workspace_size(lib):
    # many (batch, K/V head) pairs and a short cache: one chunk each, no workspace
    assert lib.attn_decode_workspace_bytes(64, 64, 64, 64, 32) == 0
    # long cache: split into chunks, partial O (D floats) and LSE per chunk and query head
    n = lib.attn_decode_workspace_bytes(2, 8, 2, 64, 4096)
    assert n > 0 and n % (2 * 8 * 65 * 4) == 0
    assert lib.attn_decode_workspace_bytes(0, 8, 2, 64, 4096) == 0
    # a valid call without workspace is accepted when none is needed (fails later only for lack of a
    # GPU; with one it would launch on the fake pointers, so it is made only where there is none)
    if not _has_gpu():
        assert _decode(lib, B=64, H=64, H_kv=64, S_max=32, max_len=32, ws=None, wsb=0) == -7


def _rope(lib, **kw):
    a = dict(q=FAKE, k=FAKE, qr=FAKE, kr=FAKE, tab=FAKE, npos=64, B=1, H=4, H_kv=2, S=64, D=64, mask=0, cu=None,
             n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_rope(a["q"], a["k"], a["qr"], a["kr"], a["tab"], a["npos"], a["B"], a["H"], a["H_kv"], a["S"],
                         a["D"], a["mask"], a["cu"], a["n"], a["mx"], a["dtype"], a["stream"])


def _fwd_rope(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qr=FAKE, kr=FAKE, o=FAKE, lse=FAKE, tab=FAKE, npos=64, B=1, H=4, H_kv=2, S=64,
             D=64, scale=0.125, mask=0, cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_fwd_rope(a["q"], a["k"], a["v"], a["qr"], a["kr"], a["o"], a["lse"], a["tab"], a["npos"], a["B"],
                             a["H"], a["H_kv"], a["S"], a["D"], a["scale"], a["mask"], a["cu"], a["n"], a["mx"],
                             a["dtype"], a["stream"])


def _bwd_rope(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE, tab=FAKE,
             npos=64, B=1, H=4, H_kv=2, S=64, D=64, scale=0.125, mask=0, cu=None, n=0, mx=0, dtype=1, stream=None)
    a.update(kw)
    return lib.attn_bwd_rope(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                             a["delta"], a["tab"], a["npos"], a["B"], a["H"], a["H_kv"], a["S"], a["D"], a["scale"],
                             a["mask"], a["cu"], a["n"], a["mx"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(tab=None), -12), (dict(npos=63), -12), (dict(npos=0), -12),
    (dict(mask=1, cu=FAKE, n=2, mx=40, npos=39), -12),
    (dict(q=None), -1), (dict(D=48), -3), (dict(dtype=3), -4), (dict(H_kv=3), -10),
    (dict(mask=2), -5), (dict(mask=1, cu=FAKE, n=2, mx=40, B=2), -6), (dict(S=0), -2),
])
def test_rope_entry_points_reject_invalid_arguments(lib, kw, code):
    assert _rope(lib, **kw) == code
    assert _fwd_rope(lib, **kw) == code
    assert _bwd_rope(lib, **kw) == code


def test_rope_entry_points_check_their_own_pointers(lib):
    assert _rope(lib, qr=None) == -1 and _rope(lib, kr=None) == -1
    assert _fwd_rope(lib, kr=None) == -1 and _fwd_rope(lib, o=None) == -1 and _fwd_rope(lib, v=None) == -1
    assert _bwd_rope(lib, dk=None) == -1 and _bwd_rope(lib, delta=None) == -1
    assert _fwd_rope(lib, scale=float("nan")) == -9 and _bwd_rope(lib, scale=-1.0) == -9
    # packed documents need positions up to the longest document only
    if not _has_gpu():
        assert _rope(lib, mask=1, cu=FAKE, n=2, mx=40, npos=40) == -7


@pytest.mark.parametrize("args,code", [
    ((None, 64, 64, 10000.0), -1), ((FAKE, 0, 64, 10000.0), -2), ((FAKE, 64, 48, 10000.0), -3),
    ((FAKE, 64, 64, 0.0), -12), ((FAKE, 64, 64, -2.0), -12), ((FAKE, 64, 64, float("inf")), -12),
    ((FAKE, 64, 64, float("nan")), -12), ((FAKE, 1 << 25, 128, 10000.0), -2),
])
def test_rope_table_rejects_invalid_arguments(lib, args, code):
    assert lib.attn_rope_table(*args, None) == code


def _params(**kw):
    p = _binding.AttnParams()
    base = dict(q=FAKE, k=FAKE, v=FAKE, dO=FAKE, o=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, delta=FAKE, B=1, H=4,
                H_kv=0, S=64, D=64, scale=0.125, mask_mode=0, cu_seqlens=None, n_seqs=0, max_seqlen=0, dtype=1,
                out_dtype=0, rope_table=None, rope_npos=0, q_rot=None, k_rot=None)
    base.update(kw)
    for name, val in base.items():
        setattr(p, name, val)
    return ctypes.byref(p)


@pytest.mark.parametrize("kw,code", [
    (dict(out_dtype=2), -4), (dict(out_dtype=7), -4), (dict(dtype=0, out_dtype=1), -4),
    (dict(dtype=2, out_dtype=1), -4), (dict(q=None), -1), (dict(H_kv=3), -10), (dict(D=40), -3),
    (dict(mask_mode=1, cu_seqlens=FAKE, n_seqs=2, max_seqlen=40, B=2), -6), (dict(scale=0.0), -9),
    # 2^18 tiles of 64 rows x 2^13 documents x 1 head = 2^31 workgroups
    (dict(mask_mode=1, cu_seqlens=FAKE, n_seqs=1 << 13, max_seqlen=(1 << 24) - 1, S=(1 << 24) - 1, D=32, H=1), -6),
    (dict(rope_table=FAKE, rope_npos=64, q_rot=None, k_rot=FAKE), -1),
    (dict(rope_table=FAKE, rope_npos=63, q_rot=FAKE, k_rot=FAKE), -12),
])
def test_ex_entry_points_reject_invalid_arguments(lib, kw, code):
    assert lib.attn_fwd_ex(_params(**kw), None) == code
    assert lib.attn_bwd_ex(_params(**kw), None) == code


def _strided(slot, triple, **kw):
    ref = _params(**kw)
    ref._obj.strides[slot][:] = list(triple)
    return ref


@pytest.mark.parametrize("slot,triple", [
    (0, (0, 0, 63)), (1, (-1, 64, 64)), (2, (4096, -64, 64)), (3, (0, 0, 32)), (7, (1, 1, 1)),
    (0, (0, 0, 1 << 31)), (4, (0, 0, 1 << 26)),   # a panel past 2^31 bytes (S = 64 rows)
])
def test_ex_rejects_invalid_strides(lib, slot, triple):
    # both calls check every row (one attn_params serves the pair)
    assert lib.attn_fwd_ex(_strided(slot, triple), None) == -13
    assert lib.attn_bwd_ex(_strided(slot, triple), None) == -13


def test_ex_accepts_strided_layouts(lib):
    """[B, S, H, D] views ({S*H*D, D, H*D}), head broadcast (head stride 0) and
    padded rows pass validation (and fail later only for lack of a GPU; with one
    they would launch on the fake pointers, so the test needs a host without)."""
    if _has_gpu():
        pytest.skip("the calls would launch kernels on fake pointers")
    for slot in range(8):
        assert lib.attn_bwd_ex(_strided(slot, (64 * 4 * 64, 64, 4 * 64)), None) == -7
    assert lib.attn_fwd_ex(_strided(1, (64 * 64, 0, 64)), None) == -7
    assert lib.attn_fwd_ex(_strided(0, (4 * 64 * 128, 64 * 128, 128)), None) == -7


def test_ex_entry_points_check_their_own_fields(lib):
    assert lib.attn_fwd_ex(None, None) == -1 and lib.attn_bwd_ex(None, None) == -1
    assert lib.attn_bwd_ex(_params(dO=None), None) == -1 and lib.attn_bwd_ex(_params(delta=None), None) == -1
    if not _has_gpu():
        assert lib.attn_fwd_ex(_params(dO=None, dq=None), None) == -7  # the forward reads neither


def test_params_struct_layout_matches_the_header(tmp_path):
    """Field offsets and size of attn_params as a C compiler lays them out
    (gcc on the header) equal the ctypes mirror's."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in _binding.AttnParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"attn_api.h\"\nint main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(attn_params, {f}));\n' for f in fields)
                   + '  printf("%zu\\n", sizeof(attn_params));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    inc = str(__import__("pathlib").Path(_binding.HEADER_PATH).parent)
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(_binding.AttnParams, f).offset for f in fields] + [ctypes.sizeof(_binding.AttnParams)]
    assert got == want


def test_no_device_reports_hip_error(lib):
    """A valid call with no GPU present fails with ATTN_ERR_HIP instead of aborting."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _fwd(lib) == -7
    assert lib.attn_bwd_dq_delta(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 0.1, 0, None, 0, 0,
                                 1, None) == -7
    assert _decode(lib) == -7
    assert _decode_noalloc(lib) == -7
    assert _fwd_gqa(lib, 2) == -7
    assert _bwd_gqa(lib, 1) == -7
    assert _rope(lib) == -7 and _fwd_rope(lib) == -7 and _bwd_rope(lib) == -7
    assert lib.attn_rope_table(FAKE, 64, 64, 10000.0, None) == -7
    assert lib.attn_fwd_ex(_params(out_dtype=1), None) == -7 and lib.attn_bwd_ex(_params(H_kv=2), None) == -7


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ca.attn_fwd(q, q, q, torch.zeros(1, 1, 16, 32), torch.zeros(1, 1, 16), 0.1)


def test_binding_rejects_unsupported_dtype():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 16, 32, dtype=torch.float64)
    with pytest.raises(TypeError):
        ca.attn_fwd(q, q, q, None, None, 0.1)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="build the HIP library"):
        _binding._lib, saved = None, _binding._lib
        try:
            _binding.load_library(str(tmp_path / "nope.so"))
        finally:
            _binding._lib = saved


def test_signatures_cover_argument_counts():
    """argtypes lengths equal the parameter counts in the header."""
    with open(_binding.HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    for name, args in _binding.SIGNATURES.items():
        m = re.search(name + r"\s*\(([^)]*)\)", text)
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), name
    assert ctypes.sizeof(ctypes.c_int) == 4
