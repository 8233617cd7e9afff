"""CPU attention oracle: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library and never touches device
memory.  ``attention_rows`` wraps the fp64 C implementation in ``oracle.c``
(the plain definition, score rows materialised); ``online_softmax`` holds the
recurrence the pages derive, used only to check it against the definition.

Every function here is pinned by tests against values the pages print, closed
forms and brute force on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.oracle_attention_rows.restype = ctypes.c_int
            lib.oracle_attention_rows.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_attention_rows_qk.restype = ctypes.c_int
            lib.oracle_attention_rows_qk.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_attention_rows_dt.restype = ctypes.c_int
            lib.oracle_attention_rows_dt.argtypes = lib.oracle_attention_rows_qk.argtypes + [ctypes.c_int]
            lib.oracle_attention_rows_f32.restype = ctypes.c_int
            lib.oracle_attention_rows_f32.argtypes = lib.oracle_attention_rows_qk.argtypes
            lib.oracle_element_to_f64.restype = ctypes.c_double
            lib.oracle_element_to_f64.argtypes = [ctypes.c_uint16, ctypes.c_int]
            lib.oracle_attention_bwd.restype = ctypes.c_int
            lib.oracle_attention_bwd.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_attention_bwd_dt.restype = ctypes.c_int
            lib.oracle_attention_bwd_dt.argtypes = lib.oracle_attention_bwd.argtypes + [ctypes.c_int]
            lib.oracle_attention_bwd_qk.restype = ctypes.c_int
            lib.oracle_attention_bwd_qk.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            lib.oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


DTYPES = {"bf16": 0, "f16": 1}


def element_to_f64(bits: int, dtype: str = "bf16") -> float:
    """The oracle's own widening of one 16-bit pattern (exposed for pinning)."""
    return float(_load().oracle_element_to_f64(int(bits), DTYPES[dtype]))


def attention_rows(q, k, v, scale: float, causal: bool, rows=None, dtype: str = "bf16"):
    """Exact attention for selected query rows, in fp64.

    ``q``: uint16 bit array [B, H, Nq, d] of bfloat16 (``dtype="bf16"``) or fp16
    (``dtype="f16"``) values; ``k, v``: [B, H, Nk, d] (contiguous).  Causal masking is top-left (key j visible to query i iff
    j <= i).  ``scale``: the softmax scale (a Python float; pass the fp32 value
    the GPU receives, widened).  ``rows``: flat query row ids
    ``(b*H + h)*Nq + i``; ``None`` means every row.  Returns
    ``(out [nrows, d] float64, lse [nrows] float64)``.
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if rows is None:
        rows = np.arange(B * H * Nq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_attention_rows_dt(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
        rows.ctypes.data, rows.size, out.ctypes.data, lse.ctypes.data, DTYPES[dtype])
    if rc != 0:
        raise RuntimeError("oracle_attention_rows_dt failed with code %d" % rc)
    return out, lse


def attention_rows_f32(q, k, v, scale: float, causal: bool, rows=None):
    """``attention_rows`` for fp32 inputs: ``q`` float32 [B, H, Nq, d], ``k, v``
    float32 [B, H, Nk, d]."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.float32) for a in (q, k, v))
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if rows is None:
        rows = np.arange(B * H * Nq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = _load().oracle_attention_rows_f32(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
        rows.ctypes.data, rows.size, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_attention_rows_f32 failed with code %d" % rc)
    return out, lse


def attention_bwd(q, k, v, dout, scale: float, causal: bool, dtype: str = "bf16"):
    """Gradients (dq, dk, dv) of sum(dout * out) in fp64.

    ``q, dout``: uint16 bit arrays [B, H, Nq, d]; ``k, v``: [B, H, Nk, d]; of
    bfloat16 or (``dtype="f16"``) fp16 values.  Causal masking is top-left
    (key j permitted to query i iff j <= i).  Returns dq [B, H, Nq, d] and dk,
    dv [B, H, Nk, d].  Follows ``oracle_attention_bwd_qk`` in ``oracle.c``.
    """
    q, k, v, dout = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v, dout))
    if q.ndim != 4 or dout.shape != q.shape or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q, dout must share one [B, H, Nq, d] shape and k, v one [B, H, Nk, d] shape")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("q and k must agree on B, H and d")
    Nk = k.shape[2]
    dq = np.empty((B, H, Nq, d), dtype=np.float64)
    dk, dv = (np.empty((B, H, Nk, d), dtype=np.float64) for _ in range(2))
    rc = _load().oracle_attention_bwd_qk(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, B, H, Nq,
                                         Nk, d, float(scale), int(bool(causal)), dq.ctypes.data, dk.ctypes.data,
                                         dv.ctypes.data, DTYPES[dtype])
    if rc != 0:
        raise RuntimeError("oracle_attention_bwd_qk failed with code %d" % rc)
    return dq, dk, dv


def attention_f64(q, k, v, scale: float, causal: bool):
    """Convenience for tiny hand-made cases: fp64 arrays (q [Nq, d], k and v
    [N, d], Nq <= N) whose values are exactly representable in bfloat16
    (checked), one head.  Query rows beyond Nq are zero padding and are not
    returned; query row i is at position i for the causal rule."""
    from inputs import f64_to_bf16_bits, bf16_bits_to_f64  # seeded-input helpers only
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, n = q.shape[0], k.shape[0]
    if nq > n or k.shape != v.shape or q.shape[1] != k.shape[1]:
        raise ValueError("need q [Nq, d], k and v [N, d] with Nq <= N")
    qp = np.zeros_like(k)
    qp[:nq] = q
    arrs = []
    for a in (qp, k, v):
        bits = f64_to_bf16_bits(a)
        if not np.array_equal(bf16_bits_to_f64(bits), a):
            raise ValueError("value not exactly representable in bfloat16")
        arrs.append(bits.reshape(1, 1, *a.shape))
    return attention_rows(*arrs, scale=scale, causal=causal, rows=np.arange(nq))
