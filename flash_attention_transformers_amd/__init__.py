"""libmattn: fused scaled-dot-product attention for MI355X (gfx950).

Thin ctypes binding over the C ABI declared in include/mattn.h.  Every step
of the computation runs in the HIP kernels of libmattn.so; this module only
marshals arguments.  PyTorch supplies device memory and the current stream.

    o, lse = fwd(q, k, v, causal=False, scale=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=False, scale=None)
    o, lse = fwd_kvcache(q, k_cache, v_cache, block_table, seqlens_k, causal=True)

The ``mattn_*`` functions mirror the C entry points one to one and take
pre-allocated tensors.  There is no fallback: if libmattn.so is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmattn.so")

MATTN_OK, MATTN_ERR_INVALID_ARG, MATTN_ERR_UNSUPPORTED, MATTN_ERR_LAUNCH = 0, 1, 2, 3
MATTN_ERR_SCRATCH = 4
MATTN_SCRATCH_BYTES = 128 << 20  # static backward scratch of mattn_bwd_noalloc
MATTN_BF16, MATTN_F32 = 0, 1
MATTN_BWD_PREPROCESS, MATTN_BWD_DKDV, MATTN_BWD_DQ = 1, 2, 4
MATTN_BWD_ALL = MATTN_BWD_PREPROCESS | MATTN_BWD_DKDV | MATTN_BWD_DQ

_lib = None


class MattnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmattn: {msg} (status {status})")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libmattn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mattn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.mattn_fwd.restype = i
    lib.mattn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i,
                              vp, sz, vp]
    lib.mattn_bwd.restype = i
    lib.mattn_bwd_stages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                     i, vp, sz, ctypes.c_uint, vp]
    lib.mattn_bwd_stages.restype = i
    lib.mattn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                      i, vp]
    lib.mattn_bwd_noalloc.restype = i
    lib.mattn_bwd_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.mattn_bwd_workspace_size.restype = sz
    lib.mattn_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i,
                                      vp, sz, vp]
    lib.mattn_fwd_kvcache.restype = i
    lib.mattn_fwd_kvcache_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.mattn_fwd_kvcache_workspace_size.restype = sz
    lib.mattn_strerror.argtypes = [i]
    lib.mattn_strerror.restype = ctypes.c_char_p
    lib.mattn_version.argtypes = []
    lib.mattn_version.restype = i
    _lib = lib
    return lib


def mattn_strerror(status: int) -> str:
    return load_library().mattn_strerror(status).decode()


def mattn_version() -> int:
    return load_library().mattn_version()


def mattn_bwd_workspace_size(B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int) -> int:
    return load_library().mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D)


def _check(status: int):
    if status != MATTN_OK:
        raise MattnError(status, mattn_strerror(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return MATTN_BF16
    if t.dtype == torch.float32:
        return MATTN_F32
    raise TypeError(f"libmattn supports bfloat16 and float32, got {t.dtype}")


def _stream_handle(t, stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _shapes(q, k, v=None):
    """Problem sizes from q [B,Hq,Sq,D] and k [B,Hkv,Skv,D]; v, when given,
    must match k exactly."""
    for n, t in (("q", q), ("k", k)) + ((("v", v),) if v is not None else ()):
        if t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D [B, H, S, D] tensor, got shape {tuple(t.shape)}")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dim")
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    return B, Hq, Hkv, Sq, Skv, D


def _expect(name, t, shape, dtype):
    """`t` must have exactly `shape` and `dtype`."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _require(*ts):
    """Every tensor on one GPU and contiguous (BHSD row-major)."""
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libmattn tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("libmattn tensors must be contiguous (BHSD row-major)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"libmattn tensors must share one device: {t.device} and {dev}")


def _check_dense(q, k, v, o=None, lse=None, do=None, dq=None, dk=None, dv=None):
    """Shapes and dtypes of a dense call, checked before any device check or
    launch: the C side cannot see buffer extents, so a tensor smaller than
    the sizes imply would be read or written out of bounds."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    for n, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{n} must have q's dtype {q.dtype}, got {t.dtype}")
    for n, t in (("o", o), ("do", do), ("dq", dq)):
        if t is not None:
            _expect(n, t, q.shape, q.dtype)
    for n, t in (("dk", dk), ("dv", dv)):
        if t is not None:
            _expect(n, t, k.shape, q.dtype)
    if lse is not None:
        _expect("lse", lse, (B, Hq, Sq), torch.float32)
    return B, Hq, Hkv, Sq, Skv, D


def _workspace_bytes(workspace, need: int) -> int:
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return nbytes


def mattn_fwd(q, k, v, o, lse, causal: bool = False, scale: Optional[float] = None,
              stream=None) -> None:
    """Forward into pre-allocated o [B,Hq,Sq,D] and lse [B,Hq,Sq] (float32)."""
    B, Hq, Hkv, Sq, Skv, D = _check_dense(q, k, v, o=o, lse=lse)
    _require(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().mattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, int(causal),
                                  float(scale), _dtype_code(q), _stream_handle(q, stream))
    _check(st)


def mattn_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, causal: bool = False,
              scale: Optional[float] = None, stream=None) -> None:
    """Backward into pre-allocated dq, dk, dv; `workspace` is a uint8 device
    tensor of at least mattn_bwd_workspace_size() bytes."""
    B, Hq, Hkv, Sq, Skv, D = _check_dense(q, k, v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    nbytes = _workspace_bytes(workspace, mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D))
    _require(q, k, v, o, lse, do, dq, dk, dv, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().mattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, Hq, Hkv, Sq, Skv, D, int(causal),
                                  float(scale), _dtype_code(q), workspace.data_ptr(), nbytes,
                                  _stream_handle(q, stream))
    _check(st)


def mattn_bwd_stages(q, k, v, o, lse, do, dq, dk, dv, workspace, stages: int,
                     causal: bool = False, scale: Optional[float] = None, stream=None) -> None:
    """Enqueue only the selected backward stages (MATTN_BWD_* flags), in the
    order preprocess, dQ, dK/dV (separate calls follow the same order).  The
    bf16 dQ stage also forms the per-row D itself, so mattn_bwd enqueues dQ
    and dK/dV for bf16 and all three for fp32; the results are the same bits."""
    B, Hq, Hkv, Sq, Skv, D = _check_dense(q, k, v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv)
    nbytes = _workspace_bytes(workspace, mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D))
    _require(q, k, v, o, lse, do, dq, dk, dv, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = load_library().mattn_bwd_stages(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                         dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                                         int(causal), float(scale), _dtype_code(q),
                                         workspace.data_ptr(), nbytes, int(stages),
                                         _stream_handle(q, stream))
    _check(st)


def mattn_fwd_kvcache_workspace_size(B: int, Hq: int, Hkv: int, Sq: int, D: int, page_size: int,
                                     pages_per_seq: int) -> int:
    return load_library().mattn_fwd_kvcache_workspace_size(B, Hq, Hkv, Sq, D, page_size,
                                                           pages_per_seq)


def mattn_fwd_kvcache(q, k_cache, v_cache, block_table, seqlens_k, o, lse, workspace,
                      causal: bool = False, scale: Optional[float] = None, stream=None) -> None:
    """Forward over a paged KV cache into pre-allocated o and lse.

    q [B,Hq,Sq,D] bf16; k_cache/v_cache [num_pages,Hkv,page_size,D] bf16;
    block_table [B,pages_per_seq] int32; seqlens_k [B] int32; workspace a
    uint8 device tensor of at least mattn_fwd_kvcache_workspace_size() bytes
    (or None when that is 0)."""
    import torch

    for n, t in (("q", q), ("k_cache", k_cache)):
        if t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D tensor, got shape {tuple(t.shape)}")
    B, Hq, Sq, D = q.shape
    num_pages, Hkv, page_size, Dc = k_cache.shape
    if Dc != D:
        raise ValueError(f"k_cache head dim {Dc} does not match q's {D}")
    _expect("v_cache", v_cache, k_cache.shape, q.dtype)
    _expect("k_cache", k_cache, k_cache.shape, q.dtype)
    _expect("o", o, q.shape, q.dtype)
    _expect("lse", lse, (B, Hq, Sq), torch.float32)
    if block_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise TypeError("block_table and seqlens_k must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, pages_per_seq], got {tuple(block_table.shape)}")
    if seqlens_k.dim() != 1 or seqlens_k.shape[0] != B:
        raise ValueError(f"seqlens_k must hold B={B} values, got shape {tuple(seqlens_k.shape)}")
    pages_per_seq = block_table.shape[1]
    need = mattn_fwd_kvcache_workspace_size(B, Hq, Hkv, Sq, D, page_size, pages_per_seq)
    if workspace is not None:
        _workspace_bytes(workspace, need)
    elif need > 0:
        raise ValueError(f"this call needs a workspace of {need} bytes")
    _require(q, k_cache, v_cache, block_table, seqlens_k, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _require(q, workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load_library().mattn_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                          block_table.data_ptr(), seqlens_k.data_ptr(),
                                          o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Sq, D,
                                          num_pages, page_size, pages_per_seq, int(causal),
                                          float(scale), _dtype_code(q), ws_ptr, ws_bytes,
                                          _stream_handle(q, stream))
    _check(st)


def fwd_kvcache(q, k_cache, v_cache, block_table, seqlens_k, causal: bool = False,
                scale: Optional[float] = None, stream=None):
    """Allocate and return (o, lse) of attention over a paged KV cache."""
    import torch

    B, Hq, Sq, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    n = mattn_fwd_kvcache_workspace_size(B, Hq, k_cache.shape[1], Sq, D, k_cache.shape[2],
                                         block_table.shape[1])
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    mattn_fwd_kvcache(q, k_cache, v_cache, block_table, seqlens_k, o, lse, ws, causal, scale,
                      stream)
    return o, lse


def fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, stream=None):
    """Allocate and return (o, lse)."""
    import torch

    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    mattn_fwd(q, k, v, o, lse, causal, scale, stream)
    return o, lse


def bwd_workspace(q, k):
    import torch

    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k)
    n = mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: Optional[float] = None,
        workspace=None, stream=None) -> Tuple[object, object, object]:
    """Allocate and return (dq, dk, dv)."""
    import torch

    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None:
        workspace = bwd_workspace(q, k)
    mattn_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, causal, scale, stream)
    return dq, dk, dv
