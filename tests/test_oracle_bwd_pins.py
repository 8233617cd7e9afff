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


@pytest.mark.parametrize("Nq,Nk,causal", [(3, 7, False), (3, 7, True), (8, 5, True), (6, 2, False)])
def test_non_square_gradients_match_finite_differences(Nq, Nk, causal):
    """Nq queries over Nk keys, causal top-left (j <= i): the oracle's gradients
    match central differences of the independent NumPy forward (np.tril of an
    Nq x Nk matrix keeps exactly j <= i)."""
    d = 4
    q, _, _ = random_qkv(1300 + Nq, 1, 1, Nq, d, sigma_qk=1.5)
    _, k, v = random_qkv(1350 + Nk, 1, 1, Nk, d, sigma_qk=1.5)
    g, _, _ = random_qkv(1400 + Nq + Nk, 1, 1, Nq, d)
    scale = float(np.float32(0.5))
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    assert dq.shape == (1, 1, Nq, d) and dk.shape == dv.shape == (1, 1, Nk, d)
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


def test_non_square_causal_keys_beyond_the_queries_get_no_gradient():
    """Causal top-left with Nq < Nk: keys j >= Nq are permitted to no query, so
    their dK and dV are exactly 0; the value gradients still sum to the
    upstream gradients' sum (each row's weights sum to 1)."""
    q, _, _ = random_qkv(1500, 1, 2, 10, 8)
    _, k, v = random_qkv(1501, 1, 2, 25, 8)
    g, _, _ = random_qkv(1502, 1, 2, 10, 8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.3, True)
    assert not np.any(dk[:, :, 10:]) and not np.any(dv[:, :, 10:])
    assert np.any(dk[:, :, :10]) and np.any(dv[:, :, :10])
    assert np.allclose(dv.sum(axis=2), bf16_bits_to_f64(g).sum(axis=2), atol=1e-12)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


def test_square_entry_points_agree():
    """The square entry points are the Nq = Nk case of the general one."""
    import ctypes
    q, k, v = random_qkv(1600, 1, 2, 9, 4)
    g, _, _ = random_qkv(1601, 1, 2, 9, 4)
    a = oracle.attention_bwd(q, k, v, g, 0.4, True)
    out = [np.empty((1, 2, 9, 4)) for _ in range(3)]
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, g)]
    rc = oracle._load().oracle_attention_bwd(*(x.ctypes.data for x in arrs), 1, 2, 9, 4, ctypes.c_double(0.4), 1,
                                             *(o.ctypes.data for o in out))
    assert rc == 0
    for x, y in zip(a, out):
        assert np.array_equal(x, y)
