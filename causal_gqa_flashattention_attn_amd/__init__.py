"""Python binding of ``libne_attn.so``: causal grouped-query FlashAttention for MI355X (gfx950).

The functions named like the C entry points (``ne_attn_fwd``, ``ne_attn_bwd``,
``ne_attn_fwd_ex``, ``ne_attn_bwd_ex``, ``ne_attn_bwd_dq_ex``, ``ne_attn_bwd_dkdv_ex``,
``ne_attn_bwd_fused``, ``ne_attn_bwd_noalloc``, ``ne_attn_decode``, ``ne_attn_prefill``,
``ne_attn_workspace_bytes``, ``ne_attn_decode_workspace_bytes``, ``ne_attn_bwd_workspace_bytes``,
``ne_attn_strerror``) only
marshal arguments: they read sizes from tensor shapes, pass ``data_ptr()`` and the current
HIP stream, and raise ``NeAttnError`` on a non-zero status.  All arithmetic happens in the HIP
kernels.  PyTorch provides device memory and streams.

``forward``, ``backward``, ``backward_fused``, ``decode``, ``prefill``, ``block_forward`` and
``block_backward`` are conveniences that allocate the outputs and the workspace with torch and
call the entry points.  They allocate on the stream the kernels run on (``stream``, else the
current stream), so torch's caching allocator never hands a workspace that is dropped on return
to other work while the kernels may still use it; the outputs belong to that stream too.

Tensor layout: q, o, dO, dq: [B, Hq, T, D]; k, v, dk, dv: [B, Hkv, T, D]; lse: [B, Hq, T]
float32; all contiguous on one GPU; float32, or bfloat16 through the ``_ex`` entry points.
Decode: q, o: [B, Hq, D]; k_cache, v_cache: [B, Hkv, Tc, D]; lse: [B, Hq]; lens: int32 [B].
Prefill: q, o: [B, Hq, Tq, D]; k_cache, v_cache: [B, Hkv, Tk, D]; lse: [B, Hq, Tq].
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "NeAttnError", "library_path", "load", "lib",
    "ne_attn_fwd", "ne_attn_bwd", "ne_attn_fwd_ex", "ne_attn_bwd_ex",
    "ne_attn_bwd_dq_ex", "ne_attn_bwd_dkdv_ex", "ne_attn_bwd_fused", "ne_attn_bwd_noalloc",
    "ne_attn_decode",
    "ne_attn_prefill", "ne_attn_workspace_bytes", "ne_attn_decode_workspace_bytes",
    "ne_attn_bwd_workspace_bytes", "ne_attn_strerror", "forward", "backward", "backward_fused",
    "decode", "prefill", "workspace", "ne_attn_block_fwd", "ne_attn_block_bwd",
    "ne_attn_block_workspace_bytes", "block_forward", "block_backward",
    "NE_OK", "NE_ERR_NULL", "NE_ERR_SHAPE", "NE_ERR_UNSUPPORTED", "NE_ERR_ALIGN", "NE_ERR_HIP",
    "NE_ERR_SCRATCH", "NE_F32", "NE_BF16", "EXPORTED_SYMBOLS",
]

(NE_OK, NE_ERR_NULL, NE_ERR_SHAPE, NE_ERR_UNSUPPORTED, NE_ERR_ALIGN, NE_ERR_HIP,
 NE_ERR_SCRATCH) = range(7)
NE_F32, NE_BF16 = 0, 1

EXPORTED_SYMBOLS = ("ne_attn_fwd", "ne_attn_bwd", "ne_attn_fwd_ex", "ne_attn_bwd_ex",
                    "ne_attn_bwd_dq_ex", "ne_attn_bwd_dkdv_ex", "ne_attn_bwd_fused",
                    "ne_attn_bwd_noalloc",
                    "ne_attn_decode", "ne_attn_prefill", "ne_attn_workspace_bytes", "ne_attn_decode_workspace_bytes",
                    "ne_attn_bwd_workspace_bytes", "ne_attn_strerror", "ne_attn_block_fwd",
                    "ne_attn_block_bwd", "ne_attn_block_workspace_bytes")

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None


class NeAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {ne_attn_strerror(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libne_attn.so")


def load():
    """Loads the built library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m causal_gqa_flashattention_attn_amd._build`")
    # torch ships its own HIP runtime with the same soname (libamdhip64.so.7).  Loading torch
    # first makes the library bind to that runtime; loading the library first would bring in a
    # second HIP runtime, whose launches cannot use torch's memory and streams.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.ne_attn_fwd.argtypes = [vp] * 5 + [i] * 6 + [vp]
    L.ne_attn_bwd.argtypes = [vp] * 10 + [i] * 6 + [vp]
    L.ne_attn_fwd_ex.argtypes = [vp] * 6 + [i] * 7 + [f, vp]
    L.ne_attn_bwd_ex.argtypes = [vp] * 10 + [i] * 7 + [f, vp]
    L.ne_attn_bwd_dq_ex.argtypes = [vp] * 8 + [i] * 7 + [f, vp]
    L.ne_attn_bwd_dkdv_ex.argtypes = [vp] * 8 + [i] * 7 + [f, vp]
    L.ne_attn_bwd_fused.argtypes = [vp] * 10 + [i] * 7 + [f, vp]
    L.ne_attn_bwd_noalloc.argtypes = [vp] * 9 + [i] * 7 + [f, vp]
    for name in ("ne_attn_fwd", "ne_attn_bwd", "ne_attn_fwd_ex", "ne_attn_bwd_ex",
                 "ne_attn_bwd_dq_ex", "ne_attn_bwd_dkdv_ex", "ne_attn_bwd_fused",
                 "ne_attn_bwd_noalloc"):
        getattr(L, name).restype = i
    L.ne_attn_workspace_bytes.argtypes = [i] * 6 + [f]
    L.ne_attn_workspace_bytes.restype = ctypes.c_size_t
    L.ne_attn_decode.argtypes = [vp] * 7 + [i] * 6 + [vp]
    L.ne_attn_prefill.argtypes = [vp] * 5 + [i] * 7 + [vp]
    L.ne_attn_decode_workspace_bytes.argtypes = [i] * 6
    L.ne_attn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.ne_attn_bwd_workspace_bytes.argtypes = [i, i, i]
    L.ne_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.ne_attn_block_workspace_bytes.argtypes = [i] * 5 + [f]
    L.ne_attn_block_workspace_bytes.restype = ctypes.c_size_t
    L.ne_attn_block_fwd.argtypes = [vp] * 6 + [i] * 5 + [f, f, vp]
    L.ne_attn_block_fwd.restype = i
    L.ne_attn_block_bwd.argtypes = [vp] * 10 + [i] * 5 + [f, f, vp]
    L.ne_attn_block_bwd.restype = i
    L.ne_attn_strerror.argtypes = [i]
    L.ne_attn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def lib():
    return load()


def ne_attn_strerror(status: int) -> str:
    return load().ne_attn_strerror(int(status)).decode()


def ne_attn_bwd_workspace_bytes(B: int, Hq: int, T: int) -> int:
    return int(load().ne_attn_bwd_workspace_bytes(int(B), int(Hq), int(T)))


def ne_attn_workspace_bytes(B: int, Hq: int, Hkv: int, T: int, D: int, dtype: int,
                            rope_base: float = 0.0) -> int:
    return int(load().ne_attn_workspace_bytes(int(B), int(Hq), int(Hkv), int(T), int(D),
                                              int(dtype), float(rope_base)))


def ne_attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Tc: int, D: int, dtype: int) -> int:
    return int(load().ne_attn_decode_workspace_bytes(int(B), int(Hq), int(Hkv), int(Tc), int(D),
                                                     int(dtype)))


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return NE_F32
    if t.dtype == torch.bfloat16:
        return NE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    B, Hq, T, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or tuple(k.shape[2:]) != (T, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    return B, Hq, k.shape[1], T, D


def _check_tensors(ts, dev):
    for name, t in ts.items():
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} must be on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream(stream, dev):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream, dev):
    """Context in which the conveniences allocate: `stream` made current (a torch stream, or a
    raw HIP stream handle wrapped as an external stream), or nothing when stream is None."""
    torch = _torch()
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=dev)
    return torch.cuda.stream(stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _raise(rc, where):
    if rc != NE_OK:
        raise NeAttnError(rc, where)


def _ws_check(ws, need, dev, name="workspace"):
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"{name} must hold at least {need} bytes")
    _check_tensors({name: ws}, dev)


def ne_attn_fwd_ex(q, k, v, o, lse, workspace=None, causal: bool = True, rope_base: float = 0.0,
                   stream=None):
    """workspace: a device tensor of at least ne_attn_workspace_bytes(...) bytes; may be None
    without RoPE."""
    torch = _torch()
    B, Hq, Hkv, T, D = _dims(q, k, v)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("o", o)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have dtype {q.dtype}")
    if o.shape != q.shape or tuple(lse.shape) != (B, Hq, T) or lse.dtype != torch.float32:
        raise ValueError("o must match q; lse must be float32 [B, Hq, T]")
    _check_tensors(dict(q=q, k=k, v=v, o=o, lse=lse), q.device)
    if workspace is not None:
        _ws_check(workspace, ne_attn_workspace_bytes(B, Hq, Hkv, T, D, dt, rope_base), q.device)
    elif rope_base > 0:
        raise ValueError("the forward with RoPE needs a workspace")
    ws = _p(workspace) if workspace is not None else None
    with torch.cuda.device(q.device):
        rc = load().ne_attn_fwd_ex(_p(q), _p(k), _p(v), _p(o), _p(lse), ws, B, Hq, Hkv, T, D,
                                   int(bool(causal)), dt, float(rope_base),
                                   _stream(stream, q.device))
    _raise(rc, "ne_attn_fwd_ex")


def ne_attn_fwd(q, k, v, o, lse, causal: bool = True, stream=None):
    torch = _torch()
    B, Hq, Hkv, T, D = _dims(q, k, v)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if o.shape != q.shape or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("o must match q; lse must be [B, Hq, T]")
    _check_tensors(dict(q=q, k=k, v=v, o=o, lse=lse), q.device)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, T, D,
                                int(bool(causal)), _stream(stream, q.device))
    _raise(rc, "ne_attn_fwd")


def _bwd_checks(q, k, v, o, lse, dO, dq, dk, dv, ws, rope_base=None, need_ws=True):
    """rope_base None: ws is the float32 delta workspace of ne_attn_bwd; otherwise the
    workspace of the _ex entry points for that RoPE setting.  need_ws False: no workspace."""
    torch = _torch()
    B, Hq, Hkv, T, D = _dims(q, k, v)
    for name, t in (("k", k), ("v", v), ("o", o), ("dO", dO), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have dtype {q.dtype}")
    if o.shape != q.shape or dO.shape != q.shape or dq.shape != q.shape:
        raise ValueError("o, dO, dq must match q")
    if dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("dk, dv must match k")
    if tuple(lse.shape) != (B, Hq, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, T]")
    ts = dict(q=q, k=k, v=v, o=o, lse=lse, dO=dO, dq=dq, dk=dk, dv=dv)
    if not need_ws:
        pass
    elif rope_base is None:
        if ws.dtype != torch.float32 or ws.numel() * 4 < ne_attn_bwd_workspace_bytes(B, Hq, T):
            raise ValueError("delta_ws must be float32 with at least B*Hq*T elements")
        ts["ws"] = ws
    else:
        _ws_check(ws, ne_attn_workspace_bytes(B, Hq, Hkv, T, D, _dtype_code(q), rope_base),
                  q.device)
        ts["ws"] = ws
    _check_tensors(ts, q.device)
    return B, Hq, Hkv, T, D


def ne_attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, workspace, causal: bool = True,
                   rope_base: float = 0.0, stream=None):
    torch = _torch()
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, o, lse, dO, dq, dk, dv, workspace, rope_base)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd_ex(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq), _p(dk),
                                   _p(dv), _p(workspace), B, Hq, Hkv, T, D, int(bool(causal)),
                                   _dtype_code(q), float(rope_base), _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd_ex")


def ne_attn_bwd_fused(q, k, v, o, lse, dO, dq, dk, dv, workspace, causal: bool = True,
                      rope_base: float = 0.0, stream=None):
    torch = _torch()
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, o, lse, dO, dq, dk, dv, workspace, rope_base)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd_fused(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                      _p(dk), _p(dv), _p(workspace), B, Hq, Hkv, T, D,
                                      int(bool(causal)), _dtype_code(q), float(rope_base),
                                      _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd_fused")


def ne_attn_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, causal: bool = True,
                        rope_base: float = 0.0, stream=None):
    """ne_attn_bwd_ex with the library's static scratch instead of a workspace: allocates
    nothing; calls that overlap on one GPU must be ordered by the caller."""
    torch = _torch()
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, o, lse, dO, dq, dk, dv, None, rope_base,
                                   need_ws=False)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd_noalloc(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                        _p(dk), _p(dv), B, Hq, Hkv, T, D, int(bool(causal)),
                                        _dtype_code(q), float(rope_base),
                                        _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd_noalloc")


def ne_attn_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, causal: bool = True, stream=None):
    torch = _torch()
    if q.dtype != torch.float32:
        raise TypeError("ne_attn_bwd takes float32 tensors")
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, o, lse, dO, dq, dk, dv, delta_ws)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq), _p(dk),
                                _p(dv), _p(delta_ws), B, Hq, Hkv, T, D, int(bool(causal)),
                                _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd")


def ne_attn_bwd_dq_ex(q, k, v, o, lse, dO, dq, workspace, causal: bool = True,
                      rope_base: float = 0.0, stream=None):
    """First backward pass: writes dq and fills the workspace."""
    torch = _torch()
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, o, lse, dO, dq, k, v, workspace, rope_base)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd_dq_ex(_p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                      _p(workspace), B, Hq, Hkv, T, D, int(bool(causal)),
                                      _dtype_code(q), float(rope_base), _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd_dq_ex")


def ne_attn_bwd_dkdv_ex(q, k, v, lse, dO, workspace, dk, dv, causal: bool = True,
                        rope_base: float = 0.0, stream=None):
    """Second backward pass: reads the workspace filled by the dq pass, writes dk and dv."""
    torch = _torch()
    B, Hq, Hkv, T, D = _bwd_checks(q, k, v, dO, lse, dO, dO, dk, dv, workspace, rope_base)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_bwd_dkdv_ex(_p(q), _p(k), _p(v), _p(lse), _p(dO), _p(workspace),
                                        _p(dk), _p(dv), B, Hq, Hkv, T, D, int(bool(causal)),
                                        _dtype_code(q), float(rope_base),
                                        _stream(stream, q.device))
    _raise(rc, "ne_attn_bwd_dkdv_ex")


def ne_attn_decode(q, k_cache, v_cache, lens, o, lse, workspace, stream=None):
    """One decode step: q [B, Hq, D] against the cache [B, Hkv, Tc, D], keys 0 .. lens[b]-1
    (lens: int32 [B] on the device)."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, D]; k_cache, v_cache [B, Hkv, Tc, D]")
    B, Hq, D = q.shape
    _, Hkv, Tc, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k_cache{tuple(k_cache.shape)}")
    dt = _dtype_code(q)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("o", o)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have dtype {q.dtype}")
    if o.shape != q.shape or tuple(lse.shape) != (B, Hq) or lse.dtype != torch.float32:
        raise ValueError("o must match q; lse must be float32 [B, Hq]")
    if tuple(lens.shape) != (B,) or lens.dtype != torch.int32:
        raise ValueError("lens must be int32 [B]")
    _check_tensors(dict(q=q, k_cache=k_cache, v_cache=v_cache, lens=lens, o=o, lse=lse),
                   q.device)
    _ws_check(workspace, ne_attn_decode_workspace_bytes(B, Hq, Hkv, Tc, D, dt), q.device)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_decode(_p(q), _p(k_cache), _p(v_cache), _p(lens), _p(o), _p(lse),
                                   _p(workspace), B, Hq, Hkv, Tc, D, dt,
                                   _stream(stream, q.device))
    _raise(rc, "ne_attn_decode")


def ne_attn_prefill(q, k_cache, v_cache, o, lse, stream=None):
    """A chunk of Tq queries at positions Tk-Tq .. Tk-1 against the cache [B, Hkv, Tk, D]."""
    torch = _torch()
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, Tq, D]; k_cache, v_cache [B, Hkv, Tk, D]")
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k_cache{tuple(k_cache.shape)}")
    dt = _dtype_code(q)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("o", o)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have dtype {q.dtype}")
    if o.shape != q.shape or tuple(lse.shape) != (B, Hq, Tq) or lse.dtype != torch.float32:
        raise ValueError("o must match q; lse must be float32 [B, Hq, Tq]")
    _check_tensors(dict(q=q, k_cache=k_cache, v_cache=v_cache, o=o, lse=lse), q.device)
    with torch.cuda.device(q.device):
        rc = load().ne_attn_prefill(_p(q), _p(k_cache), _p(v_cache), _p(o), _p(lse), B, Hq, Hkv,
                                    Tq, Tk, D, dt, _stream(stream, q.device))
    _raise(rc, "ne_attn_prefill")


# ----------------------------------------------------------------------------- conveniences

def workspace(q, k, rope_base: float = 0.0):
    """Allocates a workspace for the _ex entry points on the tensors' device."""
    torch = _torch()
    B, Hq, T, D = q.shape
    n = ne_attn_workspace_bytes(B, Hq, k.shape[1], T, D, _dtype_code(q), rope_base)
    if n == 0:
        raise ValueError("invalid shape for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def forward(q, k, v, causal: bool = True, rope_base: float = 0.0, stream=None):
    """Allocates o, lse (and with RoPE the workspace) and runs the forward pass; returns
    (o, lse)."""
    torch = _torch()
    with _alloc_on(stream, q.device):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        ws = workspace(q, k, rope_base) if rope_base > 0 else None
        ne_attn_fwd_ex(q, k, v, o, lse, ws, causal=causal, rope_base=rope_base, stream=stream)
    return o, lse


def backward(q, k, v, o, lse, dO, causal: bool = True, rope_base: float = 0.0, stream=None):
    """Allocates dq, dk, dv and the workspace and runs the backward pass."""
    torch = _torch()
    with _alloc_on(stream, q.device):
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        ne_attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, workspace(q, k, rope_base),
                       causal=causal, rope_base=rope_base, stream=stream)
    return dq, dk, dv


def backward_fused(q, k, v, o, lse, dO, causal: bool = True, rope_base: float = 0.0,
                   stream=None):
    """Single-pass backward (float32); dq is not bitwise reproducible."""
    torch = _torch()
    with _alloc_on(stream, q.device):
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        ne_attn_bwd_fused(q, k, v, o, lse, dO, dq, dk, dv, workspace(q, k, rope_base),
                          causal=causal, rope_base=rope_base, stream=stream)
    return dq, dk, dv


def decode(q, k_cache, v_cache, lens, stream=None):
    """Allocates o, lse and the workspace and runs one decode step; returns (o, lse)."""
    torch = _torch()
    B, Hq, D = q.shape
    n = ne_attn_decode_workspace_bytes(B, Hq, k_cache.shape[1], k_cache.shape[2], D,
                                       _dtype_code(q))
    if n == 0:
        raise ValueError("invalid shape for a decode workspace")
    with _alloc_on(stream, q.device):
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
        ne_attn_decode(q, k_cache, v_cache, lens, o, lse, ws, stream=stream)
    return o, lse


def prefill(q, k_cache, v_cache, stream=None):
    """Allocates o, lse and runs a prefill chunk; returns (o, lse)."""
    torch = _torch()
    with _alloc_on(stream, q.device):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        ne_attn_prefill(q, k_cache, v_cache, o, lse, stream=stream)
    return o, lse


# ----------------------------------------------------------------------- attention sub-block

def ne_attn_block_workspace_bytes(B: int, T: int, Hq: int, Hkv: int, D: int,
                                  rope_base: float = 0.0) -> int:
    return int(load().ne_attn_block_workspace_bytes(int(B), int(T), int(Hq), int(Hkv), int(D),
                                                    float(rope_base)))


def _block_check(x, gamma, w_qkv, w_o, Hq, Hkv, D):
    torch = _torch()
    B, T, C = x.shape
    if C != Hq * D or tuple(gamma.shape) != (C,) or tuple(w_qkv.shape) != (C, (Hq + 2 * Hkv) * D) \
            or tuple(w_o.shape) != (Hq * D, C):
        raise ValueError("sub-block shapes: x [B,T,Hq*D], gamma [C], w_qkv [C,(Hq+2Hkv)D], "
                         "w_o [Hq*D,C]")
    for name, t in (("x", x), ("gamma", gamma), ("w_qkv", w_qkv), ("w_o", w_o)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    return B, T


def _like_check(**pairs):
    """Each (tensor, model) pair: the tensor must be float32 with the model's shape."""
    torch = _torch()
    for name, (t, m) in pairs.items():
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(m.shape):
            raise ValueError(f"{name} must be float32 of shape {tuple(m.shape)}")


def ne_attn_block_fwd(x, gamma, w_qkv, w_o, y, workspace, Hq, Hkv, D, eps=1e-5, rope_base=0.0,
                      stream=None):
    torch = _torch()
    B, T = _block_check(x, gamma, w_qkv, w_o, Hq, Hkv, D)
    _like_check(y=(y, x))
    _ws_check(workspace, ne_attn_block_workspace_bytes(B, T, Hq, Hkv, D, rope_base), x.device)
    _check_tensors(dict(x=x, gamma=gamma, w_qkv=w_qkv, w_o=w_o, y=y), x.device)
    with torch.cuda.device(x.device):
        rc = load().ne_attn_block_fwd(_p(x), _p(gamma), _p(w_qkv), _p(w_o), _p(y), _p(workspace),
                                      B, T, Hq, Hkv, D, float(eps), float(rope_base),
                                      _stream(stream, x.device))
    _raise(rc, "ne_attn_block_fwd")


def ne_attn_block_bwd(x, gamma, w_qkv, w_o, dy, dx, dgamma, dw_qkv, dw_o, workspace, Hq, Hkv, D,
                      eps=1e-5, rope_base=0.0, stream=None):
    torch = _torch()
    B, T = _block_check(x, gamma, w_qkv, w_o, Hq, Hkv, D)
    _like_check(dy=(dy, x), dx=(dx, x), dgamma=(dgamma, gamma), dw_qkv=(dw_qkv, w_qkv),
                dw_o=(dw_o, w_o))
    _ws_check(workspace, ne_attn_block_workspace_bytes(B, T, Hq, Hkv, D, rope_base), x.device)
    _check_tensors(dict(x=x, gamma=gamma, w_qkv=w_qkv, w_o=w_o, dy=dy, dx=dx, dgamma=dgamma,
                        dw_qkv=dw_qkv, dw_o=dw_o), x.device)
    with torch.cuda.device(x.device):
        rc = load().ne_attn_block_bwd(_p(x), _p(gamma), _p(w_qkv), _p(w_o), _p(dy), _p(dx),
                                      _p(dgamma), _p(dw_qkv), _p(dw_o), _p(workspace), B, T, Hq,
                                      Hkv, D, float(eps), float(rope_base),
                                      _stream(stream, x.device))
    _raise(rc, "ne_attn_block_bwd")


def block_forward(x, gamma, w_qkv, w_o, Hq, Hkv, D, eps=1e-5, rope_base=0.0, stream=None):
    """Allocates y and the sub-block workspace and runs the forward; returns (y, workspace)."""
    torch = _torch()
    B, T = _block_check(x, gamma, w_qkv, w_o, Hq, Hkv, D)
    n = ne_attn_block_workspace_bytes(B, T, Hq, Hkv, D, rope_base)
    if n == 0:
        raise ValueError("invalid shape for a sub-block workspace")
    with _alloc_on(stream, x.device):
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        y = torch.empty_like(x)
        ne_attn_block_fwd(x, gamma, w_qkv, w_o, y, ws, Hq, Hkv, D, eps, rope_base, stream)
    return y, ws


def block_backward(x, gamma, w_qkv, w_o, dy, workspace, Hq, Hkv, D, eps=1e-5, rope_base=0.0,
                   stream=None):
    """Runs the sub-block backward after block_forward; returns (dx, dgamma, dw_qkv, dw_o)."""
    torch = _torch()
    with _alloc_on(stream, x.device):
        dx, dgamma = torch.empty_like(x), torch.empty_like(gamma)
        dw_qkv, dw_o = torch.empty_like(w_qkv), torch.empty_like(w_o)
        ne_attn_block_bwd(x, gamma, w_qkv, w_o, dy, dx, dgamma, dw_qkv, dw_o, workspace, Hq, Hkv,
                          D, eps, rope_base, stream)
    return dx, dgamma, dw_qkv, dw_o
