"""ctypes binding of libcausal_attn.so (include/attn_api.h).

Argument marshalling only: every function here checks that the torch tensors
it is given match the C ABI's layout contract, passes their device pointers
and the current HIP stream to the library, and raises on a non-zero status.
All arithmetic runs in the library's HIP kernels; if the library is missing
this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcausal_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "attn_api.h")

ATTN_OK = 0
ATTN_MASK_CAUSAL = 0
ATTN_MASK_DOC_CAUSAL = 1
ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
ATTN_DTYPE_F16 = 2
ATTN_DECODE_SCRATCH_BYTES = 16 << 20  # include/attn_api.h: the static scratch of attn_decode_noalloc

STATUS_NAMES = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_HEAD_DIM",
    -4: "ATTN_ERR_DTYPE", -5: "ATTN_ERR_MASK", -6: "ATTN_ERR_SEQLENS", -7: "ATTN_ERR_HIP",
    -8: "ATTN_ERR_UNIMPLEMENTED", -9: "ATTN_ERR_SCALE", -10: "ATTN_ERR_HEADS", -11: "ATTN_ERR_WORKSPACE",
    -12: "ATTN_ERR_ROPE", -13: "ATTN_ERR_STRIDE", -14: "ATTN_ERR_SCRATCH",
}


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


class AttnParams(ctypes.Structure):
    """attn_params of include/attn_api.h, field for field."""
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("dO", _P), ("o", _P), ("lse", _P), ("dq", _P), ("dk", _P),
                ("dv", _P), ("delta", _P), ("B", _I), ("H", _I), ("H_kv", _I), ("S", _I), ("D", _I),
                ("scale", _F), ("mask_mode", _I), ("cu_seqlens", _P), ("n_seqs", _I), ("max_seqlen", _I),
                ("dtype", _I), ("out_dtype", _I), ("rope_table", _P), ("rope_npos", _I), ("q_rot", _P),
                ("k_rot", _P), ("strides", (ctypes.c_int64 * 3) * 8), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t)]


STRIDE_SLOT = {"q": 0, "k": 1, "v": 2, "o": 3, "dO": 4, "dq": 5, "dk": 6, "dv": 7}

# argtypes of every exported function, in the header's order
SIGNATURES = {
    "attn_fwd": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_preprocess": [_P, _P, _P, _I, _I, _I, _I, _I, _P],
    "attn_bwd_dkdv": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_dq": [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_dq_delta": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_fwd_gqa": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_gqa": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_gqa_workspace_bytes": [_I, _I, _I, _I, _I, _I, _I, _I, _I],
    "attn_bwd_gqa_ws": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P,
                        ctypes.c_size_t, _P],
    "attn_decode_workspace_bytes": [_I, _I, _I, _I, _I],
    "attn_decode": [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _I, _F, _I, _I, _P],
    "attn_decode_noalloc": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P],
    "attn_rope_table": [_P, _I, _I, _F, _P],
    "attn_rope": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I, _I, _P],
    "attn_fwd_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _I, _I, _I, _P],
    "attn_bwd_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _I, _I,
                      _I, _P],
    "attn_fwd_ex": [ctypes.POINTER(AttnParams), _P],
    "attn_bwd_ex": [ctypes.POINTER(AttnParams), _P],
    "attn_status_string": [_I],
    "attn_abi_version": [],
    "attn_build_id": [],
    "attn_clock_probe": [_P, ctypes.c_ulonglong, _P],
}

_lib = None


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/attn_api.h."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|char|void|size_t)\s*\*?\s*(attn_\w+)\s*\(", text, flags=re.M)


def _init_device_runtime():
    """Bring up the HIP runtime and torch's device context before the library's
    code objects register with it: kernels of a library loaded into a process
    whose runtime was not yet initialised failed to launch (ATTN_ERR_HIP, then
    hipErrorOutOfMemory).  Without a GPU this does nothing (the library still
    loads, e.g. to check its exports and argument validation)."""
    try:
        import torch
    except ImportError:
        return
    if torch.cuda.is_available():
        torch.cuda.init()


def load_library(path: str = LIB_PATH, check_build: bool = True) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built, or if it
    was built from other sources than the tree it sits in (its attn_build_id
    differs from the digest of csrc/, the header and the build flags): a stale
    library is never run in place of the current kernels."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} not found: build the HIP library first "
            "(python -m causal_attention_amd.build or __graft_entry__.build())")
    _init_device_runtime()
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = {"attn_status_string": ctypes.c_char_p, "attn_build_id": ctypes.c_char_p,
                      "attn_decode_workspace_bytes": ctypes.c_size_t,
                      "attn_bwd_gqa_workspace_bytes": ctypes.c_size_t}.get(name, ctypes.c_int)
    if check_build:
        from .build import source_digest
        built, want = lib.attn_build_id().decode(), source_digest()
        if built != want:
            raise RuntimeError(
                f"{path} was built from other sources (build id {built}, sources {want}): "
                "rebuild it (python -m causal_attention_amd.build or __graft_entry__.build())")
    _lib = lib
    return lib


def clock_probe(out, ticks, stream=None):
    """Enqueue the clock probe: out (device uint64/int64 tensor of 2) receives
    shader-clock cycles and 100 MHz ticks over about `ticks` ticks."""
    _check(load_library().attn_clock_probe(_ptr(out, "out"), int(ticks), _stream(stream)))


def build_id() -> str:
    """The source digest the loaded library was built from."""
    return load_library().attn_build_id().decode()


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, status_string(status))


# ---------------------------------------------------------------------------
# torch-facing wrappers

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float16:
        return ATTN_DTYPE_F16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (bfloat16, float16 or float32)")


def _ptr(t, name, shape=None, dtype=None, device=None):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    del torch
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, device):
    torch = _torch()
    if mask_mode == ATTN_MASK_DOC_CAUSAL:
        if cu_seqlens is None:
            raise ValueError("packed-document mode needs cu_seqlens")
        cu_ptr = _ptr(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=device)
        if n_seqs is None:
            n_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("packed-document mode needs max_seqlen (host integer)")
        return cu_ptr, int(n_seqs), int(max_seqlen)
    return None, 0, 0


def _qkv_info(q, k, v, grouped=True):
    """(B, H, H_kv, S, D, dtype code) of q [B,H,S,D] and k, v [B,H_kv,S,D]."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, D]")
    B, H, S, D = q.shape
    if k.dim() != 4:
        raise ValueError("k must be [B, H_kv, S, D]")
    H_kv = k.shape[1] if grouped else H
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, H_kv, S, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, {H_kv}, S, D] with q's dtype"
                             + ("" if grouped else " (this entry point has no grouped heads)"))
    return B, H, H_kv, S, D, _dtype_code(q)


def attn_fwd(q, k, v, o, lse, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None, n_seqs=None,
             max_seqlen=None, stream=None):
    """Enqueue the forward: o [B,H,S,D] fp32 and lse [B,H,S] fp32 (or None).
    k and v may have fewer heads than q (grouped-query attention: attn_fwd_gqa)."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, S, D, dt = _qkv_info(q, k, v)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    ptrs = (_ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
            _ptr(o, "o", (B, H, S, D), torch.float32, dev), _ptr(lse, "lse", (B, H, S), torch.float32, dev))
    tail = (S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream))
    if H_kv == H:
        _check(lib.attn_fwd(*ptrs, B, H, *tail))
    else:
        _check(lib.attn_fwd_gqa(*ptrs, B, H, H_kv, *tail))


def bwd_workspace_bytes(B, H, H_kv, S, D, dtype, mask_mode=ATTN_MASK_CAUSAL, n_seqs=0, max_seqlen=0):
    """Bytes of workspace with which attn_bwd (attn_bwd_gqa_ws) splits grouped
    heads' dK/dV step (0: the split does not apply).  dtype: a torch dtype."""
    torch = _torch()
    code = {torch.float32: ATTN_DTYPE_F32, torch.bfloat16: ATTN_DTYPE_BF16, torch.float16: ATTN_DTYPE_F16}[dtype]
    return int(load_library().attn_bwd_gqa_workspace_bytes(int(B), int(H), int(H_kv), int(S), int(D),
                                                           int(mask_mode), int(n_seqs), int(max_seqlen), code))


def attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
             n_seqs=None, max_seqlen=None, stream=None, workspace=None):
    """Enqueue the backward: dq [B,H,S,D], dk, dv [B,H_kv,S,D] fp32; delta [B,H,S] fp32
    workspace.  k and v may have fewer heads than q (attn_bwd_gqa).  workspace:
    a device tensor of at least bwd_workspace_bytes(...) bytes, or None; when
    given, the call is attn_bwd_gqa_ws (grouped heads' dK/dV split into parts
    where that applies)."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, S, D, dt = _qkv_info(q, k, v)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    f32 = torch.float32
    ptrs = (_ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
            _ptr(o, "o", (B, H, S, D), f32, dev), _ptr(dO, "dO", (B, H, S, D), q.dtype, dev),
            _ptr(lse, "lse", (B, H, S), f32, dev), _ptr(dq, "dq", (B, H, S, D), f32, dev),
            _ptr(dk, "dk", (B, H_kv, S, D), f32, dev), _ptr(dv, "dv", (B, H_kv, S, D), f32, dev),
            _ptr(delta, "delta", (B, H, S), f32, dev))
    tail = (S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream))
    if workspace is not None:
        ws = _ptr(workspace, "workspace", device=dev)
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib.attn_bwd_gqa_ws(*ptrs, B, H, H_kv, *tail[:-1], ws, nbytes, tail[-1]))
    elif H_kv == H:
        _check(lib.attn_bwd(*ptrs, B, H, *tail))
    else:
        _check(lib.attn_bwd_gqa(*ptrs, B, H, H_kv, *tail))


def attn_bwd_preprocess(o, dO, delta, stream=None):
    torch = _torch()
    lib = load_library()
    B, H, S, D = dO.shape
    dev = dO.device
    _check(lib.attn_bwd_preprocess(
        _ptr(o, "o", (B, H, S, D), torch.float32, dev), _ptr(dO, "dO", device=dev),
        _ptr(delta, "delta", (B, H, S), torch.float32, dev), B, H, S, D, _dtype_code(dO), _stream(stream)))


def attn_bwd_dkdv(q, k, v, dO, lse, delta, dk, dv, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
                  n_seqs=None, max_seqlen=None, stream=None):
    torch = _torch()
    lib = load_library()
    B, H, _, S, D, dt = _qkv_info(q, k, v, grouped=False)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    f32 = torch.float32
    _check(lib.attn_bwd_dkdv(
        _ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
        _ptr(dO, "dO", (B, H, S, D), q.dtype, dev), _ptr(lse, "lse", (B, H, S), f32, dev),
        _ptr(delta, "delta", (B, H, S), f32, dev), _ptr(dk, "dk", (B, H, S, D), f32, dev),
        _ptr(dv, "dv", (B, H, S, D), f32, dev),
        B, H, S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream)))


def attn_bwd_dq(q, k, v, dO, lse, delta, dq, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
                n_seqs=None, max_seqlen=None, stream=None):
    torch = _torch()
    lib = load_library()
    B, H, _, S, D, dt = _qkv_info(q, k, v, grouped=False)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    f32 = torch.float32
    _check(lib.attn_bwd_dq(
        _ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
        _ptr(dO, "dO", (B, H, S, D), q.dtype, dev), _ptr(lse, "lse", (B, H, S), f32, dev),
        _ptr(delta, "delta", (B, H, S), f32, dev), _ptr(dq, "dq", (B, H, S, D), f32, dev),
        B, H, S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream)))


def attn_bwd_dq_delta(q, k, v, o, dO, lse, dq, delta, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
                      n_seqs=None, max_seqlen=None, stream=None):
    """Enqueue the backward's first stage: delta [B,H,S] and dq [B,H,S,D] fp32 from o
    (attn_bwd runs this, then attn_bwd_dkdv)."""
    torch = _torch()
    lib = load_library()
    B, H, _, S, D, dt = _qkv_info(q, k, v, grouped=False)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    f32 = torch.float32
    _check(lib.attn_bwd_dq_delta(
        _ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
        _ptr(o, "o", (B, H, S, D), f32, dev), _ptr(dO, "dO", (B, H, S, D), q.dtype, dev),
        _ptr(lse, "lse", (B, H, S), f32, dev), _ptr(dq, "dq", (B, H, S, D), f32, dev),
        _ptr(delta, "delta", (B, H, S), f32, dev),
        B, H, S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream)))


def _rope_table_ptr(tab, D, dev):
    torch = _torch()
    if tab is None or tab.dim() != 3 or tuple(tab.shape[1:]) != (D // 2, 2):
        raise ValueError(f"the RoPE table must be [n_pos, {D // 2}, 2] float32")
    return _ptr(tab, "rope table", dtype=torch.float32, device=dev), int(tab.shape[0])


def attn_rope_table(tab, base=10000.0, stream=None):
    """Fill tab [n_pos, D/2, 2] fp32 with (cos, sin) of p * base^(-2i/D)."""
    lib = load_library()
    if tab.dim() != 3 or tab.shape[2] != 2:
        raise ValueError("the RoPE table must be [n_pos, D/2, 2] float32")
    n_pos, half = int(tab.shape[0]), int(tab.shape[1])
    _check(lib.attn_rope_table(_ptr(tab, "tab", dtype=_torch().float32), n_pos, 2 * half, float(base),
                               _stream(stream)))


def attn_rope(q, k, q_rot, k_rot, tab, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None, n_seqs=None,
              max_seqlen=None, stream=None):
    """Enqueue the rotation: q_rot, k_rot (q's and k's shapes and dtype; may be q, k)."""
    lib = load_library()
    B, H, H_kv, S, D, dt = _qkv_info(q, k, k)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    tp, n_pos = _rope_table_ptr(tab, D, dev)
    _check(lib.attn_rope(
        _ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(q_rot, "q_rot", tuple(q.shape), q.dtype, dev),
        _ptr(k_rot, "k_rot", tuple(k.shape), k.dtype, dev), tp, n_pos, B, H, H_kv, S, D, int(mask_mode), cu, ns, ms,
        dt, _stream(stream)))


def attn_fwd_rope(q, k, v, q_rot, k_rot, o, lse, tab, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
                  n_seqs=None, max_seqlen=None, stream=None):
    """Enqueue RoPE on q, k (into q_rot, k_rot, kept for the backward), then the forward."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, S, D, dt = _qkv_info(q, k, v)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    tp, n_pos = _rope_table_ptr(tab, D, dev)
    _check(lib.attn_fwd_rope(
        _ptr(q, "q", device=dev), _ptr(k, "k", device=dev), _ptr(v, "v", device=dev),
        _ptr(q_rot, "q_rot", tuple(q.shape), q.dtype, dev), _ptr(k_rot, "k_rot", tuple(k.shape), k.dtype, dev),
        _ptr(o, "o", (B, H, S, D), torch.float32, dev), _ptr(lse, "lse", (B, H, S), torch.float32, dev),
        tp, n_pos, B, H, H_kv, S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream)))


def attn_bwd_rope(q_rot, k_rot, v, o, dO, lse, dq, dk, dv, delta, tab, scale, mask_mode=ATTN_MASK_CAUSAL,
                  cu_seqlens=None, n_seqs=None, max_seqlen=None, stream=None):
    """Enqueue the backward on the rotated q_rot, k_rot; dq and dk come out with
    respect to the unrotated q and k."""
    torch = _torch()
    lib = load_library()
    B, H, H_kv, S, D, dt = _qkv_info(q_rot, k_rot, v)
    dev = q_rot.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    tp, n_pos = _rope_table_ptr(tab, D, dev)
    f32 = torch.float32
    _check(lib.attn_bwd_rope(
        _ptr(q_rot, "q_rot", device=dev), _ptr(k_rot, "k_rot", device=dev), _ptr(v, "v", device=dev),
        _ptr(o, "o", (B, H, S, D), f32, dev), _ptr(dO, "dO", (B, H, S, D), q_rot.dtype, dev),
        _ptr(lse, "lse", (B, H, S), f32, dev), _ptr(dq, "dq", (B, H, S, D), f32, dev),
        _ptr(dk, "dk", (B, H_kv, S, D), f32, dev), _ptr(dv, "dv", (B, H_kv, S, D), f32, dev),
        _ptr(delta, "delta", (B, H, S), f32, dev), tp, n_pos,
        B, H, H_kv, S, D, float(scale), int(mask_mode), cu, ns, ms, dt, _stream(stream)))


def _out_code(o, q):
    """Output dtype code from the output tensor: fp32, or q's 16-bit dtype."""
    torch = _torch()
    if o.dtype == torch.float32:
        return ATTN_DTYPE_F32
    if o.dtype == q.dtype and q.dtype in (torch.bfloat16, torch.float16):
        return _dtype_code(q)
    raise TypeError(f"outputs must be float32 or the inputs' 16-bit dtype, not {o.dtype}")


def _view(p, t, name, shape, dtype, device):
    """Pointer of a [B, H, S, D] view whose last dimension is contiguous, its
    (batch, head, sequence) element strides recorded in p.strides."""
    if t is None:
        return None
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}, not {tuple(t.shape)} {t.dtype}")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    p.strides[STRIDE_SLOT[name]][:] = [t.stride(0), t.stride(1), t.stride(2)]
    return t.data_ptr()


def _params(q, k, v, o, lse, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, rope_table, q_rot, k_rot):
    B, H, H_kv, S, D, dt = _qkv_info(q, k, v)
    dev = q.device
    cu, ns, ms = _mask_args(mask_mode, cu_seqlens, n_seqs, max_seqlen, dev)
    p = AttnParams()
    p.q = _view(p, q, "q", (B, H, S, D), q.dtype, dev)
    p.k = _view(p, k, "k", (B, H_kv, S, D), q.dtype, dev)
    p.v = _view(p, v, "v", (B, H_kv, S, D), q.dtype, dev)
    out = _out_code(o, q)
    p.o = _view(p, o, "o", (B, H, S, D), o.dtype, dev)
    p.lse = _ptr(lse, "lse", (B, H, S), _torch().float32, dev)
    p.B, p.H, p.H_kv, p.S, p.D = B, H, H_kv, S, D
    p.scale, p.mask_mode, p.cu_seqlens, p.n_seqs, p.max_seqlen = float(scale), int(mask_mode), cu, ns, ms
    p.dtype, p.out_dtype = dt, out
    if rope_table is not None:
        p.rope_table, p.rope_npos = _rope_table_ptr(rope_table, D, dev)
        p.q_rot = _ptr(q_rot, "q_rot", tuple(q.shape), q.dtype, dev)
        p.k_rot = _ptr(k_rot, "k_rot", tuple(k.shape), k.dtype, dev)
    return p, (B, H, H_kv, S, D, dev)


def attn_fwd_ex(q, k, v, o, lse, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None, n_seqs=None, max_seqlen=None,
                rope_table=None, q_rot=None, k_rot=None, stream=None):
    """Forward with every option: grouped K/V heads (k, v with fewer heads),
    RoPE (rope_table given: q, k rotated into contiguous q_rot, k_rot), 16-bit
    outputs (o in the inputs' bf16/fp16 dtype instead of float32), and any
    [B, H, S, D] views with a contiguous last dimension (e.g. x.transpose(1, 2)
    of a [B, S, H, D] tensor), passed by their strides without copies."""
    p, _ = _params(q, k, v, o, lse, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, rope_table, q_rot, k_rot)
    _check(load_library().attn_fwd_ex(ctypes.byref(p), _stream(stream)))


def attn_bwd_ex(q, k, v, o, dO, lse, dq, dk, dv, delta, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None,
                n_seqs=None, max_seqlen=None, rope_table=None, q_rot=None, k_rot=None, stream=None, workspace=None):
    """Backward with every option (see attn_fwd_ex).  With RoPE the kernels read
    q_rot, k_rot (q, k only give shapes); dq, dk, dv in o's dtype.  workspace:
    None, or a device tensor of at least bwd_workspace_bytes(...) bytes with
    which grouped heads split their dK/dV step."""
    p, (B, H, H_kv, S, D, dev) = _params(q, k, v, o, lse, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen,
                                         rope_table, q_rot, k_rot)
    p.dO = _view(p, dO, "dO", (B, H, S, D), q.dtype, dev)
    p.dq = _view(p, dq, "dq", (B, H, S, D), o.dtype, dev)
    p.dk = _view(p, dk, "dk", (B, H_kv, S, D), o.dtype, dev)
    p.dv = _view(p, dv, "dv", (B, H_kv, S, D), o.dtype, dev)
    p.delta = _ptr(delta, "delta", (B, H, S), _torch().float32, dev)
    if workspace is not None:
        p.workspace = _ptr(workspace, "workspace", device=dev)
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().attn_bwd_ex(ctypes.byref(p), _stream(stream)))


def decode_workspace_bytes(B, H, H_kv, D, max_len):
    return int(load_library().attn_decode_workspace_bytes(int(B), int(H), int(H_kv), int(D), int(max_len)))


def attn_decode(q, k_cache, v_cache, cache_lens, o, lse, workspace, scale, max_len, stream=None):
    """Enqueue one decode step: q [B,H,D] against the first cache_lens[b] rows of
    k_cache, v_cache [B,H_kv,S_max,D]; o [B,H,D] and lse [B,H] (or None) fp32;
    workspace: a device tensor of at least decode_workspace_bytes(...) bytes (or
    None when that is 0)."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, D] and the caches [B, H_kv, S_max, D]")
    B, H, D = q.shape
    _, H_kv, S_max, _ = k_cache.shape
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if tuple(t.shape) != (B, H_kv, S_max, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H_kv, S_max, D] with q's dtype")
    dev = q.device
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace", device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.attn_decode(
        _ptr(q, "q", device=dev), _ptr(k_cache, "k_cache", device=dev), _ptr(v_cache, "v_cache", device=dev),
        _ptr(cache_lens, "cache_lens", (B,), torch.int32, dev), _ptr(o, "o", (B, H, D), torch.float32, dev),
        _ptr(lse, "lse", (B, H), torch.float32, dev), ws_ptr, ws_bytes,
        B, H, H_kv, S_max, D, float(scale), int(max_len), _dtype_code(q), _stream(stream)))


def attn_decode_noalloc(q, k_cache, v_cache, cache_lens, o, lse, scale, max_len, stream=None):
    """attn_decode without a workspace: the chunk partials go to the library's
    static per-GPU scratch (ATTN_DECODE_SCRATCH_BYTES); calls that overlap on
    one GPU race.  Raises AttnError (ATTN_ERR_SCRATCH) when the split needs more."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, H, D] and the caches [B, H_kv, S_max, D]")
    B, H, D = q.shape
    _, H_kv, S_max, _ = k_cache.shape
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if tuple(t.shape) != (B, H_kv, S_max, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [B, H_kv, S_max, D] with q's dtype")
    dev = q.device
    _check(lib.attn_decode_noalloc(
        _ptr(q, "q", device=dev), _ptr(k_cache, "k_cache", device=dev), _ptr(v_cache, "v_cache", device=dev),
        _ptr(cache_lens, "cache_lens", (B,), torch.int32, dev), _ptr(o, "o", (B, H, D), torch.float32, dev),
        _ptr(lse, "lse", (B, H), torch.float32, dev),
        B, H, H_kv, S_max, D, float(scale), int(max_len), _dtype_code(q), _stream(stream)))


# ---------------------------------------------------------------------------
# Allocating conveniences (torch supplies the device memory).

def decode(q, k_cache, v_cache, cache_lens, scale, max_len, stream=None):
    """Returns (o, lse) of one decode step as new fp32 device tensors."""
    torch = _torch()
    B, H, D = q.shape
    H_kv = k_cache.shape[1]
    o = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    n = decode_workspace_bytes(B, H, H_kv, D, max_len)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    attn_decode(q, k_cache, v_cache, cache_lens, o, lse, ws, scale, max_len, stream)
    return o, lse

def forward(q, k, v, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None, max_seqlen=None, stream=None,
            out_dtype=None):
    """Returns (o, lse) as new device tensors: o in ``out_dtype`` (float32 by
    default, or q's bf16/fp16 dtype), lse float32."""
    torch = _torch()
    B, H, S, D = q.shape
    o = torch.empty((B, H, S, D), dtype=out_dtype or torch.float32, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if o.dtype == torch.float32:
        attn_fwd(q, k, v, o, lse, scale, mask_mode, cu_seqlens, None, max_seqlen, stream)
    else:
        attn_fwd_ex(q, k, v, o, lse, scale, mask_mode, cu_seqlens, None, max_seqlen, stream=stream)
    return o, lse


def backward(q, k, v, o, dO, lse, scale, mask_mode=ATTN_MASK_CAUSAL, cu_seqlens=None, max_seqlen=None,
             stream=None):
    """Returns (dq, dk, dv, delta) as new device tensors: gradients in o's dtype
    (float32, or q's bf16/fp16 dtype), delta float32."""
    torch = _torch()
    B, H, S, D = q.shape
    dq = torch.empty((B, H, S, D), dtype=o.dtype, device=q.device)
    dk = torch.empty(tuple(k.shape), dtype=o.dtype, device=q.device)
    dv = torch.empty_like(dk)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    ws = None
    if k.shape[1] != H:  # grouped heads: the workspace with which their dK/dV step may split
        doc = mask_mode == ATTN_MASK_DOC_CAUSAL and cu_seqlens is not None and max_seqlen is not None
        n_seqs = cu_seqlens.numel() - 1 if doc else 0
        ms = int(max_seqlen) if doc else 0
        nbytes = bwd_workspace_bytes(B, H, k.shape[1], S, D, q.dtype, mask_mode, n_seqs, ms)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if o.dtype == torch.float32 and q.is_contiguous() and k.is_contiguous() and v.is_contiguous():
        attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta, scale, mask_mode, cu_seqlens, None, max_seqlen, stream,
                 workspace=ws)
    else:
        attn_bwd_ex(q, k, v, o, dO, lse, dq, dk, dv, delta, scale, mask_mode, cu_seqlens, None, max_seqlen,
                    stream=stream, workspace=ws)
    return dq, dk, dv, delta


def rope_table(n_pos, D, base=10000.0, device="cuda", stream=None):
    """Returns a new [n_pos, D/2, 2] fp32 device table of (cos, sin) for RoPE."""
    torch = _torch()
    tab = torch.empty((n_pos, D // 2, 2), dtype=torch.float32, device=device)
    attn_rope_table(tab, base, stream)
    return tab
