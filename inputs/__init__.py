"""Seeded synthetic inputs for the attention forward pass.

This module only draws numbers: it holds none of the attention arithmetic, and
both the CPU oracle (via the tests and the benchmark) and the HIP path consume
the same buffers it produces.

Recipe
------
* A counter-based SplitMix64 stream (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014): output ``i`` of the stream with
  seed ``s`` is ``mix64(s + (i + 1) * 0x9E3779B97F4A7C15)``.
* Two consecutive outputs ``(2p, 2p + 1)`` become uniforms
  ``u1 = (top53 + 1) * 2**-53`` in (0, 1] and ``u2 = top53 * 2**-53`` in [0, 1),
  and the Box-Muller transform (Box and Muller, 1958) turns them into the normal
  pair ``r cos(2 pi u2), r sin(2 pi u2)`` with ``r = sqrt(-2 ln u1)``; element
  ``2p`` takes the cosine, element ``2p + 1`` the sine.
* The fp64 normal is multiplied by ``sigma`` and rounded once, to nearest-even,
  straight to bfloat16 (no intermediate fp32 rounding).

Tensors are returned as ``uint16`` arrays holding bfloat16 bit patterns in the
contiguous ``[B, H, N, d]`` layout.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22  # elements per work item; keeps temporaries small

# Per-workload seeds: seed(c, t) = 0xFA2F0000 + 16 c + t, t = 0, 1, 2 for Q, K, V.
SEED_BASE = 0xFA2F0000


def workload_seed(config: int, tensor: int) -> int:
    """Seed of tensor ``tensor`` of workload number ``config``: 0 = Q, 1 = K, 2 = V,
    3 = the row sample of the CPU baseline, 4 = the upstream gradient dO."""
    return SEED_BASE + 16 * int(config) + int(tensor)


def splitmix64(seed: int, counters: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs for the given 0-based counters (uint64 array)."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (counters.astype(np.uint64) + np.uint64(1)) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _normals_f64(seed: int, start: int, count: int) -> np.ndarray:
    """Standard normals for element indices [start, start + count) (start even)."""
    assert start % 2 == 0
    npairs = (count + 1) // 2
    pair = np.arange(start // 2, start // 2 + npairs, dtype=np.uint64)
    a = splitmix64(seed, pair * np.uint64(2))
    b = splitmix64(seed, pair * np.uint64(2) + np.uint64(1))
    scale53 = 2.0 ** -53
    u1 = ((a >> np.uint64(11)).astype(np.float64) + 1.0) * scale53
    u2 = (b >> np.uint64(11)).astype(np.float64) * scale53
    r = np.sqrt(-2.0 * np.log(u1))
    theta = (2.0 * math.pi) * u2
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = r * np.cos(theta)
    out[1::2] = r * np.sin(theta)
    return out[:count]


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest-even, to bfloat16; returns the uint16 bits.

    Valid for finite values whose magnitude is 0 or at least 2**-126 (bf16 normal
    range); the generator never produces anything else (|x| >= ~1e-24 or 0), and
    this is asserted.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    ax = np.abs(x)
    if np.any((ax != 0.0) & (ax < 2.0 ** -126)):
        raise ValueError("value below the bfloat16 normal range")
    if np.any(ax >= 2.0 ** 128):
        raise ValueError("value beyond the bfloat16 range")
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    with np.errstate(over="ignore"):
        bits = (bits + (np.uint64((1 << 44) - 1) + lsb)) & np.uint64(~((1 << 45) - 1) & 0xFFFFFFFFFFFFFFFF)
    f32 = bits.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values once, to nearest-even, to IEEE fp16; returns the uint16 bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 bit patterns to fp64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bits_to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    return f16_bits_to_f64(bits) if dtype == "f16" else bf16_bits_to_f64(bits)


def normal_f16(seed: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """``count`` i.i.d. N(0, sigma^2) values rounded to fp16 (uint16 bits); the
    same normals as ``normal_bf16`` for the same seed."""
    out = np.empty(count, dtype=np.uint16)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = f64_to_f16_bits(_normals_f64(seed, s, n) * float(sigma))
    return out


def normal_f32(seed: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """``count`` i.i.d. N(0, sigma^2) values rounded to fp32 (the same draws as
    ``normal_bf16`` for the same seed)."""
    out = np.empty(count, dtype=np.float32)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = (_normals_f64(seed, s, n) * float(sigma)).astype(np.float32)
    return out


def normal_bits(seed: int, count: int, sigma: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """bf16 / f16: uint16 bit patterns; f32: float32 values."""
    if dtype == "f32":
        return normal_f32(seed, count, sigma)
    return normal_f16(seed, count, sigma) if dtype == "f16" else normal_bf16(seed, count, sigma)


def normal_bf16(seed: int, count: int, sigma: float = 1.0, threads: int | None = None) -> np.ndarray:
    """``count`` i.i.d. N(0, sigma^2) values rounded to bfloat16 (uint16 bits)."""
    out = np.empty(count, dtype=np.uint16)
    starts = list(range(0, count, _CHUNK))

    def work(s: int) -> None:
        n = min(_CHUNK, count - s)
        out[s:s + n] = f64_to_bf16_bits(_normals_f64(seed, s, n) * float(sigma))

    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        nthreads = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=nthreads) as pool:
            list(pool.map(work, starts))
    return out


# The five workloads the measurements and parity tests use.  Every one is square,
# dense and contiguous [B, H, N, d]; sigma_qk / sigma_v are the standard deviations.
WORKLOADS = {
    1: dict(name="B1-H1-N256-d64", B=1, H=1, N=256, d=64, modes=(0,), sigma_qk=1.0, sigma_v=1.0),
    2: dict(name="B1-H8-N1024-d64", B=1, H=8, N=1024, d=64, modes=(0, 1), sigma_qk=1.0, sigma_v=1.0),
    3: dict(name="B4-H8-N4096-d64", B=4, H=8, N=4096, d=64, modes=(0, 1), sigma_qk=1.0, sigma_v=1.0),
    4: dict(name="B1-H32-N32768-d128", B=1, H=32, N=32768, d=128, modes=(1,), sigma_qk=1.0, sigma_v=1.0),
    5: dict(name="B4-H32-N8192-d128-peaked", B=4, H=32, N=8192, d=128, modes=(0,), sigma_qk=4.0, sigma_v=1.0),
}


def default_scale(d: int) -> float:
    """The softmax scale the workloads use: the fp32 value of 1/sqrt(d)."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_qkv(config: int, B: int | None = None, H: int | None = None, N: int | None = None,
             d: int | None = None, sigma_qk: float | None = None, sigma_v: float | None = None,
             dtype: str = "bf16"):
    """Q, K, V bit arrays (bfloat16, or fp16 with ``dtype="f16"``) shaped
    [B, H, N, d] for workload ``config``.

    Shape and distribution default to the workload's own; overriding them keeps
    the workload's seeds (used by small parity cases).
    """
    w = WORKLOADS[config]
    B = w["B"] if B is None else B
    H = w["H"] if H is None else H
    N = w["N"] if N is None else N
    d = w["d"] if d is None else d
    sq = w["sigma_qk"] if sigma_qk is None else sigma_qk
    sv = w["sigma_v"] if sigma_v is None else sigma_v
    count = B * H * N * d
    q = normal_bits(workload_seed(config, 0), count, sq, dtype).reshape(B, H, N, d)
    k = normal_bits(workload_seed(config, 1), count, sq, dtype).reshape(B, H, N, d)
    v = normal_bits(workload_seed(config, 2), count, sv, dtype).reshape(B, H, N, d)
    return q, k, v


def random_qkv(seed: int, B: int, H: int, N: int, d: int, sigma_qk: float = 1.0, sigma_v: float = 1.0,
               dtype: str = "bf16"):
    """Q, K, V for an arbitrary seed (three consecutive sub-seeds), as bfloat16
    or fp16 bit patterns."""
    count = B * H * N * d
    q = normal_bits(seed * 3 + 0, count, sigma_qk, dtype).reshape(B, H, N, d)
    k = normal_bits(seed * 3 + 1, count, sigma_qk, dtype).reshape(B, H, N, d)
    v = normal_bits(seed * 3 + 2, count, sigma_v, dtype).reshape(B, H, N, d)
    return q, k, v


def sample_rows(config_seed: int, B: int, H: int, N: int, per_head: int = 64) -> np.ndarray:
    """Deterministic row sample: fixed edge rows plus seeded rows, per (b, h).

    Returns flat row ids ``(b * H + h) * N + i``, sorted and unique.
    """
    fixed = [0, 1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 256, N // 2 - 1, N // 2, N - 2, N - 1]
    rows = []
    for bh in range(B * H):
        base = [i for i in fixed if 0 <= i < N]
        extra = max(0, per_head - len(base))
        if extra:
            z = splitmix64(config_seed + 7919 * bh, np.arange(extra, dtype=np.uint64))
            base += [int(x) for x in (z % np.uint64(N))]
        rows.extend(bh * N + i for i in sorted(set(base)))
    return np.array(sorted(set(rows)), dtype=np.int64)
