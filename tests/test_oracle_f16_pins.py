"""Pins for the oracle's fp16 inputs: its element decoder against NumPy's own
IEEE binary16 conversion on every bit pattern, brute force on tiny fp16 cases,
and closed forms whose values are exactly representable in fp16.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from inputs import f16_bits_to_f64, f64_to_f16_bits, random_qkv


def test_decoder_matches_numpy_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.element_to_f64(int(b), "f16") for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, oracle.element_to_f64(0x8000, "f16")) == -1.0


def test_decoder_special_values():
    assert oracle.element_to_f64(0x3C00, "f16") == 1.0
    assert oracle.element_to_f64(0x0001, "f16") == 2.0 ** -24        # smallest subnormal
    assert oracle.element_to_f64(0x0400, "f16") == 2.0 ** -14        # smallest normal
    assert oracle.element_to_f64(0x7BFF, "f16") == 65504.0           # largest finite
    assert oracle.element_to_f64(0xC000, "f16") == -2.0
    assert oracle.element_to_f64(0x7C00, "f16") == math.inf
    # the same bits read as bfloat16 are a different number: the dtype is honoured
    assert oracle.element_to_f64(0x3C00, "bf16") == 2.0 ** -7


def brute_force_row(qi, K, V, scale, nkeys):
    e = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(qi, K[j]))) for j in range(nkeys)]
    tot = math.fsum(e)
    o = [math.fsum(e[j] * float(V[j, c]) for j in range(nkeys)) / tot for c in range(V.shape[1])]
    return np.array(o), math.log(tot)


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(1, 1, 7, 7, 8, False), (1, 2, 9, 9, 32, True),
                                                (2, 1, 5, 13, 16, True), (1, 1, 12, 12, 256, False)])
def test_brute_force_f16(B, H, Nq, Nk, d, causal):
    q, _, _ = random_qkv(500 + Nq + d, B, H, Nq, d, dtype="f16")
    _, k, v = random_qkv(600 + Nk + d, B, H, Nk, d, dtype="f16")
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = oracle.attention_rows(q, k, v, scale, causal, dtype="f16")
    qf = f16_bits_to_f64(q).reshape(B * H, Nq, d)
    kf, vf = (f16_bits_to_f64(a).reshape(B * H, Nk, d) for a in (k, v))
    for bh in range(B * H):
        for i in range(Nq):
            n = min(i + 1, Nk) if causal else Nk
            o, L = brute_force_row(qf[bh, i], kf[bh], vf[bh], scale, n)
            t = bh * Nq + i
            assert np.allclose(out[t], o, atol=1e-13, rtol=1e-12)
            assert abs(lse[t] - L) < 1e-12


def test_f16_identical_keys_and_fine_values():
    """Identical keys: every row is the plain mean of the visible value rows; the
    values use fp16's 10-bit fraction (not representable in bfloat16), so a
    decoder that read them as bfloat16 would fail."""
    rng = np.random.default_rng(11)
    N, d = 9, 32
    vals = 1.0 + rng.integers(0, 1024, size=(N, d)) / 1024.0     # exact in fp16, not in bfloat16
    kb = np.tile(f64_to_f16_bits(rng.standard_normal(d)), (N, 1)).reshape(1, 1, N, d)
    qb = f64_to_f16_bits(rng.standard_normal((N, d))).reshape(1, 1, N, d)
    vb = f64_to_f16_bits(vals).reshape(1, 1, N, d)
    assert np.array_equal(f16_bits_to_f64(vb)[0, 0], vals)
    out, _ = oracle.attention_rows(qb, kb, vb, 0.25, True, dtype="f16")
    for i in range(N):
        assert np.allclose(out[i], vals[: i + 1].mean(axis=0), atol=1e-14)


def test_same_normals_in_both_dtypes():
    """The fp16 and bfloat16 generators round the same N(0, 1) draws: they agree
    to within the coarser format's rounding."""
    from inputs import bf16_bits_to_f64, normal_bf16, normal_f16
    a = f16_bits_to_f64(normal_f16(77, 4096))
    b = bf16_bits_to_f64(normal_bf16(77, 4096))
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -8 + 2.0 ** -24)


# ---------------------------------------------------------------- fp32 inputs

@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(1, 1, 7, 7, 8, False), (1, 2, 9, 9, 64, True),
                                                (2, 1, 5, 13, 16, True), (1, 1, 12, 30, 128, False)])
def test_brute_force_f32(B, H, Nq, Nk, d, causal):
    """fp32 inputs carry 24-bit significands: the oracle reads them at full precision."""
    q, _, _ = random_qkv(700 + Nq + d, B, H, Nq, d, dtype="f32")
    _, k, v = random_qkv(710 + Nk + d, B, H, Nk, d, dtype="f32")
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = oracle.attention_rows_f32(q, k, v, scale, causal)
    qf = q.astype(np.float64).reshape(B * H, Nq, d)
    kf, vf = (a.astype(np.float64).reshape(B * H, Nk, d) for a in (k, v))
    for bh in range(B * H):
        for i in range(Nq):
            n = min(i + 1, Nk) if causal else Nk
            o, L = brute_force_row(qf[bh, i], kf[bh], vf[bh], scale, n)
            t = bh * Nq + i
            assert np.allclose(out[t], o, atol=1e-13, rtol=1e-12)
            assert abs(lse[t] - L) < 1e-12


def test_f32_values_are_not_rounded():
    """Identical keys: each row is the exact mean of the visible value rows, whose
    values need fp32's full significand (1 + 2^-20 steps), so any rounding to a
    16-bit format would show."""
    rng = np.random.default_rng(13)
    N, d = 6, 8
    vals = (1.0 + rng.integers(0, 1 << 20, size=(N, d)) * 2.0 ** -20).astype(np.float32)
    kk = np.tile(rng.standard_normal(d).astype(np.float32), (N, 1)).reshape(1, 1, N, d)
    qq = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    out, _ = oracle.attention_rows_f32(qq, kk, vals.reshape(1, 1, N, d), 0.5, True)
    for i in range(N):
        assert np.allclose(out[i], vals[: i + 1].astype(np.float64).mean(axis=0), atol=1e-15, rtol=1e-15)
