"""MI355X (gfx950) FlashAttention-2 forward (and backward): Python binding of libfa_fwd.so.

Argument marshalling only: every step of the forward pass runs in the HIP
library; PyTorch supplies device memory and the stream.  There is no fallback:
if the library is not built, or the device is not a gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

from .buildlib import LIB, build  # noqa: F401

__all__ = ["fa_fwd", "fa_fwd_ptr", "fa_fwd_cfg", "fa_fwd_ex", "fa_fwd_ex_ptr", "fa_fwd_splitkv",
           "splitkv_workspace_bytes", "splitkv_default_splits", "FwdDesc", "FaError", "strerror",
           "version", "default_cfg", "launch_cfg", "variants", "load_library", "EXPORTED_SYMBOLS", "fa_bwd", "fa_bwd_ptr",
           "bwd_workspace_bytes", "fa_bwd_ex", "fa_bwd_ex_ptr", "BwdDesc", "attention", "fa_fwd_splitkv_noalloc",
           "SPLITKV_NOALLOC_MAX_BYTES"]

EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_cfg", "fa_fwd_ex", "fa_fwd_ex_cfg", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
                    "fa_splitkv_workspace_bytes", "fa_splitkv_default_splits", "fa_default_cfg", "fa_launch_cfg", "fa_num_variants",
                    "fa_variant", "fa_variant_dtype", "fa_strerror", "fa_version", "fa_bwd", "fa_bwd_ex",
                    "fa_bwd_workspace_bytes")

STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM", 4: "FA_ERR_SCALE",
          5: "FA_ERR_ARG", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ALIAS", 8: "FA_ERR_NO_DEVICE",
          9: "FA_ERR_LAUNCH", 10: "FA_ERR_INTERNAL", 11: "FA_ERR_STRIDE", 12: "FA_ERR_WORKSPACE",
          13: "FA_ERR_SCRATCH"}


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


class TileCfg(ctypes.Structure):
    """fa_tile_cfg: (qb, waves, bk) or, for the key-split tile, (qb, waves, bk, ksplit)."""
    _fields_ = [("qb", ctypes.c_int), ("waves", ctypes.c_int), ("bk", ctypes.c_int), ("ksplit", ctypes.c_int)]

    def as_tuple(self):
        t = (self.qb, self.waves, self.bk)
        return t + (self.ksplit,) if self.ksplit > 1 else t


_LL3 = ctypes.c_longlong * 3
_LL2 = ctypes.c_longlong * 2


class FwdDesc(ctypes.Structure):
    """Mirror of ``fa_fwd_desc`` (include/fa_fwd.h): general lengths and strides."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("Nq", ctypes.c_int), ("Nk", ctypes.c_int),
                ("d", ctypes.c_int),
                ("q_stride", _LL3), ("k_stride", _LL3), ("v_stride", _LL3), ("o_stride", _LL3),
                ("lse_stride", _LL2),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("stream", ctypes.c_void_p),
                ("dtype", ctypes.c_int)]


class BwdDesc(ctypes.Structure):
    """Mirror of ``fa_bwd_desc`` (include/fa_bwd.h): strided, bf16 or fp16 backward."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dout", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("d", ctypes.c_int),
                ("q_stride", _LL3), ("k_stride", _LL3), ("v_stride", _LL3), ("o_stride", _LL3),
                ("do_stride", _LL3), ("dq_stride", _LL3), ("dk_stride", _LL3), ("dv_stride", _LL3),
                ("lse_stride", _LL2),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_longlong),
                ("stream", ctypes.c_void_p), ("Nk", ctypes.c_int)]


DTYPE_BF16, DTYPE_F16, DTYPE_F32 = 0, 1, 2
_DTYPE_NAMES = {"bf16": DTYPE_BF16, "f16": DTYPE_F16, "f32": DTYPE_F32}


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def load_library():
    """Load libfa_fwd.so from the package directory (raises if it is not built).

    torch (when installed) is imported first: its wheel ships its own HIP
    runtime, which this library must share.  Loaded before torch, the library
    would pull in the system runtime under another file name, torch would then
    load its own, and with two HIP runtimes in one process the one this library
    uses reports no device.
    """
    global _lib
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                raise FaError(10, "libfa_fwd.so is not built; run flashattention_forward_fa2_amd.build()")
            lib = ctypes.CDLL(LIB)
            fwd_args = [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P]
            lib.fa_fwd.argtypes = fwd_args
            lib.fa_fwd.restype = _I
            lib.fa_fwd_cfg.argtypes = fwd_args + [ctypes.POINTER(TileCfg)]
            lib.fa_fwd_cfg.restype = _I
            lib.fa_fwd_ex.argtypes = [ctypes.POINTER(FwdDesc)]
            lib.fa_fwd_ex.restype = _I
            lib.fa_fwd_ex_cfg.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(TileCfg)]
            lib.fa_fwd_ex_cfg.restype = _I
            lib.fa_fwd_splitkv.argtypes = [ctypes.POINTER(FwdDesc), _I, _P, ctypes.c_longlong]
            lib.fa_fwd_splitkv.restype = _I
            lib.fa_fwd_splitkv_noalloc.argtypes = [ctypes.POINTER(FwdDesc), _I]
            lib.fa_fwd_splitkv_noalloc.restype = _I
            lib.fa_splitkv_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
            lib.fa_splitkv_workspace_bytes.restype = ctypes.c_longlong
            lib.fa_splitkv_default_splits.argtypes = [_I, _I, _I, _I, _I, _I]
            lib.fa_splitkv_default_splits.restype = _I
            lib.fa_default_cfg.argtypes = [_I, _I, _I, ctypes.POINTER(TileCfg)]
            lib.fa_default_cfg.restype = _I
            lib.fa_launch_cfg.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(TileCfg)]
            lib.fa_launch_cfg.restype = _I
            lib.fa_num_variants.argtypes = []
            lib.fa_num_variants.restype = _I
            lib.fa_variant.argtypes = [_I, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(TileCfg)]
            lib.fa_variant.restype = _I
            lib.fa_variant_dtype.argtypes = [_I]
            lib.fa_variant_dtype.restype = _I
            lib.fa_strerror.argtypes = [_I]
            lib.fa_strerror.restype = ctypes.c_char_p
            lib.fa_version.argtypes = []
            lib.fa_version.restype = _I
            lib.fa_bwd_workspace_bytes.argtypes = [_I, _I, _I, _I]
            lib.fa_bwd_workspace_bytes.restype = ctypes.c_longlong
            lib.fa_bwd.argtypes = [_P] * 9 + [_I, _I, _I, _I, ctypes.c_float, _I, _P, ctypes.c_longlong, _P]
            lib.fa_bwd.restype = _I
            lib.fa_bwd_ex.argtypes = [ctypes.POINTER(BwdDesc)]
            lib.fa_bwd_ex.restype = _I
            _lib = lib
    return _lib


def strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def version() -> int:
    return int(load_library().fa_version())


def _check(status: int):
    if status != 0:
        raise FaError(status, strerror(status))


def default_cfg(N: int, d: int, causal: bool):
    c = TileCfg()
    _check(load_library().fa_default_cfg(int(N), int(d), int(bool(causal)), ctypes.byref(c)))
    return c.as_tuple()


def launch_cfg(B: int, H: int, Nq: int, d: int, causal: bool, dtype: str = "bf16"):
    """The tile fa_fwd / fa_fwd_ex launch for these sizes on the current device: ``(qb, waves, bk)``, or
    ``(qb, waves, bk, ksplit)`` for the key-split tile."""
    c = TileCfg()
    _check(load_library().fa_launch_cfg(int(B), int(H), int(Nq), int(d), int(bool(causal)), _DTYPE_NAMES[dtype],
                                        ctypes.byref(c)))
    return c.as_tuple()


def variants(dtype: str = "bf16"):
    """Compiled variants of one element type ("bf16", "f16" or "f32") as
    (d, causal, cfg) tuples, cfg as ``TileCfg.as_tuple`` gives it."""
    lib = load_library()
    want = _DTYPE_NAMES[dtype]
    out = []
    for i in range(lib.fa_num_variants()):
        d, c, cfg = _I(), _I(), TileCfg()
        _check(lib.fa_variant(i, ctypes.byref(d), ctypes.byref(c), ctypes.byref(cfg)))
        if lib.fa_variant_dtype(i) == want:
            out.append((d.value, c.value, cfg.as_tuple()))
    return out


def fa_fwd_ptr(q: int, k: int, v: int, out: int, lse: int, B: int, H: int, N: int, d: int,
               scale: float, causal: bool, stream: int = 0, cfg=None) -> int:
    """Raw-pointer call; returns the library's status code (does not raise)."""
    lib = load_library()
    args = (_P(q), _P(k), _P(v), _P(out), _P(lse), int(B), int(H), int(N), int(d),
            ctypes.c_float(scale), int(causal), _P(stream))
    if cfg is None:
        return int(lib.fa_fwd(*args))
    c = TileCfg(*cfg)
    return int(lib.fa_fwd_cfg(*args, ctypes.byref(c)))


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def fa_fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
           stream=None, cfg=None):
    """Attention forward on torch bf16 tensors [B, H, N, d] (contiguous, one device).

    Returns ``(out, lse)``: ``out`` bf16 [B, H, N, d], ``lse`` fp32 [B, H, N].
    ``scale`` defaults to the fp32 value of 1/sqrt(d).  Enqueued on ``stream``
    (default: the current stream); no synchronisation.
    """
    import torch
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous bfloat16 device tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, N]")
    st = fa_fwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    B, H, N, d, scale, causal, _stream_handle(stream, q.device), cfg)
    _check(st)
    return out, lse


def fa_fwd_cfg(q, k, v, cfg, scale: float | None = None, causal: bool = False, out=None, lse=None,
               stream=None):
    """``fa_fwd`` with an explicit ``(qb, waves, bk)`` tile configuration."""
    return fa_fwd(q, k, v, scale=scale, causal=causal, out=out, lse=lse, stream=stream, cfg=tuple(cfg))


def fa_fwd_ex_ptr(desc: FwdDesc, cfg=None) -> int:
    """Raw descriptor call; returns the library's status code (does not raise)."""
    lib = load_library()
    if cfg is None:
        return int(lib.fa_fwd_ex(ctypes.byref(desc)))
    c = TileCfg(*cfg)
    return int(lib.fa_fwd_ex_cfg(ctypes.byref(desc), ctypes.byref(c)))


def _make_desc(q, k, v, scale, causal, out, lse, stream):
    """Check torch views and fill an ``FwdDesc``; returns ``(desc, out, lse)``."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Nq, d], k and v one [B, H, Nk, d] shape")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("q, k, v must agree on B, H and d")
    Nk = k.shape[2]
    et = q.dtype
    if et not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError("q, k, v must be bfloat16, float16 or float32")
    for t in (q, k, v):
        if t.dtype != et or not t.is_cuda or t.stride(3) != 1:
            raise ValueError("q, k, v must be device views of one dtype with a contiguous last dimension")
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=et, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != (B, H, Nq, d) or out.dtype != et or out.stride(3) != 1:
        raise ValueError("out must be a [B, H, Nq, d] view of q's dtype with a contiguous last dimension")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or lse.stride(2) != 1:
        raise ValueError("lse must be an fp32 [B, H, Nq] view with unit row stride")
    desc = FwdDesc()
    desc.q, desc.k, desc.v, desc.out, desc.lse = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                   lse.data_ptr())
    desc.B, desc.H, desc.Nq, desc.Nk, desc.d = B, H, Nq, Nk, d
    desc.q_stride = _LL3(*q.stride()[:3])
    desc.k_stride = _LL3(*k.stride()[:3])
    desc.v_stride = _LL3(*v.stride()[:3])
    desc.o_stride = _LL3(*out.stride()[:3])
    desc.lse_stride = _LL2(*lse.stride()[:2])
    desc.scale = float(scale)
    desc.causal = int(bool(causal))
    desc.stream = _stream_handle(stream, q.device)
    desc.dtype = {torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}.get(et, DTYPE_BF16)
    return desc, out, lse


def fa_fwd_ex(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
              stream=None, cfg=None):
    """Attention forward on strided torch bf16, fp16 or fp32 views, N_q queries over N_k keys.

    ``q`` is [B, H, Nq, d] and ``k``, ``v`` are [B, H, Nk, d], each with any
    strides whose last one is 1 (a [B, N, H, d] tensor is passed as
    ``t.transpose(1, 2)``).  Causal masking is top-left: key j is visible to
    query i iff j <= i.  ``out`` (default: a new contiguous tensor) is a
    [B, H, Nq, d] view of q's dtype, ``lse`` a [B, H, Nq] fp32 view with unit
    row stride.  d is 32, 64, 128 or 256 (fp32: 64 or 128).
    Returns ``(out, lse)``; enqueued on ``stream`` (default: the current stream).
    """
    desc, out, lse = _make_desc(q, k, v, scale, causal, out, lse, stream)
    _check(fa_fwd_ex_ptr(desc, None if cfg is None else tuple(cfg)))
    return out, lse


def splitkv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0) -> int:
    n = int(load_library().fa_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits))
    if n < 0:
        _check(-n)
    return n


def splitkv_default_splits(B: int, H: int, Nq: int, Nk: int, d: int, causal: bool = False) -> int:
    n = int(load_library().fa_splitkv_default_splits(B, H, Nq, Nk, d, int(bool(causal))))
    if n < 0:
        _check(-n)
    return n


def fa_fwd_splitkv(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
                   stream=None, num_splits: int = 0, workspace=None):
    """``fa_fwd_ex`` computed over key splits and merged (Flash-Decoding).

    ``workspace``: a device tensor of at least ``splitkv_workspace_bytes(...)``
    bytes (default: allocated here through torch).  Returns ``(out, lse)``.
    """
    import torch
    desc, out, lse = _make_desc(q, k, v, scale, causal, out, lse, stream)
    need = splitkv_workspace_bytes(desc.B, desc.H, desc.Nq, desc.Nk, desc.d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(int(load_library().fa_fwd_splitkv(ctypes.byref(desc), int(num_splits), _P(workspace.data_ptr()),
                                             ctypes.c_longlong(nbytes))))
    return out, lse


# Bytes of the library's static split-key scratch (FA_SPLITKV_NOALLOC_MAX_BYTES).
SPLITKV_NOALLOC_MAX_BYTES = 32 << 20


def fa_fwd_splitkv_noalloc(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
                           stream=None, num_splits: int = 0):
    """``fa_fwd_splitkv`` with its partial results in the library's static
    per-GPU scratch instead of a workspace (nothing is allocated for them).
    Returns ``(out, lse)``; raises FA_ERR_SCRATCH when they would not fit."""
    desc, out, lse = _make_desc(q, k, v, scale, causal, out, lse, stream)
    _check(int(load_library().fa_fwd_splitkv_noalloc(ctypes.byref(desc), int(num_splits))))
    return out, lse


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    n = int(load_library().fa_bwd_workspace_bytes(B, H, N, d))
    if n < 0:
        _check(-n)
    return n


def fa_bwd_ptr(q: int, k: int, v: int, out: int, lse: int, dout: int, dq: int, dk: int, dv: int, B: int, H: int,
               N: int, d: int, scale: float, causal: bool, workspace: int, workspace_bytes: int,
               stream: int = 0) -> int:
    """Raw-pointer call of ``fa_bwd``; returns the library's status code (does not raise)."""
    lib = load_library()
    return int(lib.fa_bwd(_P(q), _P(k), _P(v), _P(out), _P(lse), _P(dout), _P(dq), _P(dk), _P(dv), int(B), int(H),
                          int(N), int(d), ctypes.c_float(scale), int(causal), _P(workspace),
                          ctypes.c_longlong(workspace_bytes), _P(stream)))


def fa_bwd(q, k, v, out, lse, dout, scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None,
           workspace=None, stream=None):
    """Attention backward on torch tensors: q, k, v, out, dout bf16 [B, H, N, d]
    and lse fp32 [B, H, N] (the forward's outputs for the same scale and mask),
    all contiguous on one device.  Returns ``(dq, dk, dv)``, bf16 [B, H, N, d].
    ``workspace``: a device tensor of at least ``bwd_workspace_bytes(...)`` bytes
    (default: allocated here through torch).  Enqueued on ``stream``; no
    synchronisation.
    """
    import torch
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout must share one [B, H, N, d] shape")
    for t in (q, k, v, out, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v, out, dout must be contiguous bfloat16 device tensors")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, N]")
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_like(q)
        if g.shape != q.shape or g.dtype != torch.bfloat16 or not g.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous bf16 tensors shaped like q")
        grads.append(g)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    st = fa_bwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                    grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), B, H, N, d, scale, causal,
                    workspace.data_ptr(), nbytes, _stream_handle(stream, q.device))
    _check(st)
    return tuple(grads)


def fa_bwd_ex_ptr(desc: BwdDesc) -> int:
    """Raw descriptor call of ``fa_bwd_ex``; returns the status code (does not raise)."""
    return int(load_library().fa_bwd_ex(ctypes.byref(desc)))


def fa_bwd_ex(q, k, v, out, lse, dout, scale: float | None = None, causal: bool = False, dq=None, dk=None,
              dv=None, workspace=None, stream=None):
    """Attention backward on strided bf16 or fp16 views, Nq queries over Nk keys.

    ``q, out, dout`` are [B, H, Nq, d] and ``k, v`` [B, H, Nk, d] views of one
    dtype with a contiguous last dimension (a [B, N, H, d] tensor is passed as
    ``t.transpose(1, 2)``), ``lse`` a [B, H, Nq] fp32 view with unit row stride:
    ``fa_fwd_ex``'s outputs for the same scale and (top-left) mask.  ``dq``
    (default: new) is shaped like q, ``dk, dv`` like k.  Returns
    ``(dq, dk, dv)``; enqueued on ``stream``, no synchronisation.
    """
    import torch
    if q.dim() != 4 or any(t.dim() != 4 or t.shape != q.shape for t in (out, dout)):
        raise ValueError("q, out, dout must share one [B, H, Nq, d] shape")
    if k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[1] != q.shape[1] \
            or k.shape[3] != q.shape[3]:
        raise ValueError("k, v must share one [B, H, Nk, d] shape agreeing with q on B, H, d")
    et = q.dtype
    if et not in (torch.bfloat16, torch.float16):
        raise ValueError("the backward takes bfloat16 or float16 tensors")
    for t in (q, k, v, out, dout):
        if t.dtype != et or not t.is_cuda or t.stride(3) != 1:
            raise ValueError("q, k, v, out, dout must be device views of one dtype with a contiguous last dimension")
    B, H, N, d = q.shape
    Nk = k.shape[2]
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.stride(2) != 1:
        raise ValueError("lse must be an fp32 [B, H, Nq] view with unit row stride")
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    grads = []
    for g, shape in ((dq, (B, H, N, d)), (dk, (B, H, Nk, d)), (dv, (B, H, Nk, d))):
        if g is None:
            g = torch.empty(shape, dtype=et, device=q.device)
        if tuple(g.shape) != shape or g.dtype != et or g.stride(3) != 1:
            raise ValueError("dq must be shaped like q and dk, dv like k, in q's dtype with a contiguous last dimension")
        grads.append(g)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    desc = BwdDesc()
    desc.q, desc.k, desc.v, desc.out, desc.lse, desc.dout = (t.data_ptr() for t in (q, k, v, out, lse, dout))
    desc.dq, desc.dk, desc.dv = (g.data_ptr() for g in grads)
    desc.B, desc.H, desc.N, desc.d, desc.Nk = B, H, N, d, Nk
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out), ("do_stride", dout),
                    ("dq_stride", grads[0]), ("dk_stride", grads[1]), ("dv_stride", grads[2])):
        setattr(desc, name, _LL3(*t.stride()[:3]))
    desc.lse_stride = _LL2(*lse.stride()[:2])
    desc.scale = float(scale)
    desc.causal = int(bool(causal))
    desc.dtype = DTYPE_F16 if et == torch.float16 else DTYPE_BF16
    desc.workspace = workspace.data_ptr()
    desc.workspace_bytes = workspace.numel() * workspace.element_size()
    desc.stream = _stream_handle(stream, q.device)
    _check(fa_bwd_ex_ptr(desc))
    return tuple(grads)


_autograd_fn = None


def _attention_function():
    """The torch.autograd.Function over fa_fwd_ex / fa_bwd_ex (built on first use,
    so that importing the package does not import torch)."""
    global _autograd_fn
    if _autograd_fn is None:
        import torch

        class FlashAttention(torch.autograd.Function):
            """out = softmax(scale * q k^T) v on the library's kernels; the
            backward recomputes P from the saved log-sum-exp."""

            @staticmethod
            def forward(ctx, q, k, v, causal, scale):
                out, lse = fa_fwd_ex(q, k, v, scale=scale, causal=causal)
                ctx.save_for_backward(q, k, v, out, lse)
                ctx.causal, ctx.scale = causal, scale
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, out, lse = ctx.saved_tensors
                dq, dk, dv = fa_bwd_ex(q, k, v, out, lse, dout.contiguous() if dout.stride(3) != 1 else dout,
                                       scale=ctx.scale, causal=ctx.causal)
                return dq, dk, dv, None, None

        _autograd_fn = FlashAttention
    return _autograd_fn


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """Differentiable attention on the library's kernels: ``q`` [B, H, Nq, d],
    ``k, v`` [B, H, Nk, d] views (bf16 or fp16 for gradients; any strides with a
    contiguous last dimension), causal masking top-left.  Returns ``out``; its
    backward computes dq, dk, dv with ``fa_bwd_ex`` from the saved output and
    log-sum-exp.  d is 32, 64 or 128 when gradients are needed."""
    import torch
    if scale is None:
        scale = float(torch.tensor(1.0 / math.sqrt(q.shape[-1]), dtype=torch.float32))
    return _attention_function().apply(q, k, v, bool(causal), float(scale))
