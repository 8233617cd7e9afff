"""Pins for the backward oracle (gradients of sum(dout * out)): central finite
differences of an independent NumPy fp64 forward, and invariants the softmax
fixes.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from inputs import bf16_bits_to_f64, random_qkv


def forward_np(q, k, v, scale, causal):
    """Plain fp64 attention of one head on float arrays (a different evaluation
    from the C oracle: whole score matrix, mask by -inf, numpy reductions)."""
    S = scale * (q @ k.T)
    if causal:
        S = np.where(np.tril(np.ones_like(S, dtype=bool)), S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return P @ v


@pytest.mark.parametrize("N,d,causal", [(1, 4, False), (5, 4, False), (5, 4, True), (7, 8, True), (9, 3, False)])
def test_gradients_match_finite_differences(N, d, causal):
    q, k, v = random_qkv(900 + N + d, 1, 1, N, d, sigma_qk=1.5)
    g, _, _ = random_qkv(950 + N, 1, 1, N, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    Q, K, V, G = (bf16_bits_to_f64(a)[0, 0] for a in (q, k, v, g))

    def f(Q_, K_, V_):
        return float(np.sum(G * forward_np(Q_, K_, V_, scale, causal)))

    eps = 1e-6
    for name, X, grad in (("q", Q, dq), ("k", K, dk), ("v", V, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = {"q": (Xp, K, V), "k": (Q, Xp, V), "v": (Q, K, Xp)}[name]
            args_m = {"q": (Xm, K, V), "k": (Q, Xm, V), "v": (Q, K, Xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert np.allclose(grad[0, 0], num, atol=1e-7, rtol=1e-6), name


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """Adding one vector to every key leaves every row's weights unchanged, so
    the key gradients sum to zero; adding one vector to every value adds it to
    every output, so the value gradients sum to the upstream gradients' sum.
    A causal row that sees one key has zero gradient with respect to q."""
    B, H, N, d = 1, 2, 40, 16
    q, k, v = random_qkv(990, B, H, N, d, sigma_qk=2.0)
    g, _, _ = random_qkv(991, B, H, N, d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.25, causal)
    G = bf16_bits_to_f64(g)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    assert np.allclose(dv.sum(axis=2), G.sum(axis=2), atol=1e-12)
    if causal:
        assert np.abs(dq[:, :, 0]).max() == 0.0


def test_zero_upstream_gradient_gives_zero():
    q, k, v = random_qkv(995, 1, 1, 12, 8)
    z = np.zeros_like(q)
    for grad in oracle.attention_bwd(q, k, v, z, 0.3, True):
        assert not np.any(grad)


@pytest.mark.parametrize("N,d,causal", [(6, 4, False), (7, 8, True)])
def test_f16_gradients_match_finite_differences(N, d, causal):
    """fp16 inputs: the oracle decodes them as IEEE binary16 (values a bfloat16
    reading would get wrong) and its gradients match central differences."""
    from inputs import f16_bits_to_f64
    q, k, v = random_qkv(1200 + N + d, 1, 1, N, d, sigma_qk=1.5, dtype="f16")
    g, _, _ = random_qkv(1250 + N, 1, 1, N, d, dtype="f16")
    scale = float(np.float32(1 / math.sqrt(d)))
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal, dtype="f16")
    Q, K, V, G = (f16_bits_to_f64(a)[0, 0] for a in (q, k, v, g))

    def f(Q_, K_, V_):
        return float(np.sum(G * forward_np(Q_, K_, V_, scale, causal)))

    eps = 1e-6
    for name, X, grad in (("q", Q, dq), ("k", K, dk), ("v", V, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = {"q": (Xp, K, V), "k": (Q, Xp, V), "v": (Q, K, Xp)}[name]
            args_m = {"q": (Xm, K, V), "k": (Q, Xm, V), "v": (Q, K, Xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert np.allclose(grad[0, 0], num, atol=1e-7, rtol=1e-6), name
