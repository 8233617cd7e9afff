"""Pins for the CPU oracle: printed worked examples, closed forms, invariants and
brute force on tiny inputs.  None of these re-run the oracle's own formula; each
is chosen so that a plausible slip in the oracle (a dropped scale, a wrong sign,
a transposed operand, a causal off-by-one, the wrong log base, a missing max
subtraction) fails at least one of them.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import online_softmax as osm
from inputs import bf16_bits_to_f64, f64_to_bf16_bits, random_qkv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def num(x):
    if isinstance(x, str):
        if x == "ln2":
            return math.log(2.0)
        if "/" in x:
            a, b = x.split("/")
            return float(a) / float(b)
        return float(x)
    return float(x)


def f32(x):
    return float(np.float32(x))


def pad(rows, width):
    a = np.zeros((len(rows), width))
    for i, r in enumerate(rows):
        a[i, :len(r)] = r
    return a


# ---------------------------------------------------------------- printed examples

def test_four_token_table_4_2_output_and_weights():
    """Table 4.2: weights and output as printed (3 decimals) and in closed form."""
    g = load("four_token_attention.json")
    scale = f32(1.0 / math.sqrt(g["head_dim"]))
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-9
    # value rows as the page gives them -> printed output
    q = pad([g["q"]], 2)
    K = pad(g["K"], 2)
    V = pad(g["V"], 2)
    out, lse = oracle.attention_f64(q, K, V, scale, causal=False)
    assert np.allclose(out[0], g["printed"]["output"], atol=tol, rtol=0)
    # identity value rows turn the output into the weights themselves
    qw = pad([g["q"]], 4)
    Kw = pad(g["K"], 4)
    out_w, lse_w = oracle.attention_f64(qw, Kw, np.eye(4), scale, causal=False)
    assert np.allclose(out_w[0], g["printed"]["weights"], atol=tol, rtol=0)
    assert np.allclose(np.exp(lse_w[0] + np.log(out_w[0])), g["printed"]["exponentials"], atol=tol)
    assert abs(math.exp(lse[0]) - g["printed"]["sum"]) <= tol
    # closed form: output = [sigmoid(c), 1/2] with c = scale; LSE = ln(2 e^c + 2)
    c = scale
    assert abs(out[0, 0] - 1.0 / (1.0 + math.exp(-c))) < 1e-14
    assert abs(out[0, 1] - 0.5) < 1e-15
    assert abs(lse[0] - math.log(2.0 * math.exp(c) + 2.0)) < 1e-14


def test_two_block_online_softmax_states():
    """Section 4.8 worked example: every printed state of the recurrence."""
    g = load("online_softmax_two_blocks.json")
    s = [num(x) for x in g["scores"]]
    V = np.array(g["V"], dtype=float)
    o, L, st = osm.attend_row(s, V, g["blocks"])
    b1, b2 = st.trace
    p1, p2 = g["printed"]["after_block_1"], g["printed"]["after_block_2"]
    for got, want in ((b1, p1), (b2, p2)):
        assert got["m"] == pytest.approx(num(want["m"]), abs=1e-15)
        assert got["alpha"] == pytest.approx(want["alpha"], abs=1e-15)
        assert got["w"] == pytest.approx(want["w"], abs=1e-15)
        assert got["l"] == pytest.approx(want["l"], abs=1e-15)
        assert np.allclose(got["o"], want["o"], atol=1e-15)
    assert np.allclose(o, g["printed"]["output"], atol=1e-15)
    # the definition, through the C oracle: scores [0, 0, ln2, ln2] come from
    # q = e1, k = [0, 0, e1, e1] and scale = fp32(ln 2)
    scale = f32(math.log(2.0))
    q = np.array([[1.0, 0.0]])
    K = np.array([[0.0, 0.0], [0.0, 0.0], [1.0, 0.0], [1.0, 0.0]])
    out, lse = oracle.attention_f64(q, K, V, scale, causal=False)
    w = np.array([1.0, 1.0, math.exp(scale), math.exp(scale)])
    assert np.allclose(out[0], (w / w.sum()) @ V, atol=1e-15)
    assert np.allclose(out[0], g["printed"]["output"], atol=1e-8)
    full = [num(x) for x in g["printed"]["full_row_weights"]]
    assert np.allclose(w / w.sum(), full, atol=1e-8)


def test_online_max_sum_four_values():
    """x = [2, 1, 5, 3]: running max 5 and sum 1.2034, one element at a time."""
    g = load("online_max_sum_four.json")
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-9
    m, l = osm.online_max_sum(g["x"])
    assert m == g["printed"]["m"]
    assert abs(l - g["printed"]["l"]) <= tol
    assert np.allclose([math.exp(x - m) for x in g["x"]], g["printed"]["terms"], atol=tol)
    # the C oracle on the same scores (d = 1, q = 1, k_j = x_j, scale = 1): LSE = m + ln l
    x = np.array(g["x"], dtype=float)[:, None]
    _, lse = oracle.attention_f64(np.ones((1, 1)), x, np.ones((4, 1)), 1.0, causal=False)
    assert abs(math.exp(lse[0] - 5.0) - g["printed"]["l"]) <= tol


def test_eight_scores_whole_row_and_tiles():
    """Section 2.7: whole-row P and l, and the two-tile walk with its repair factor."""
    g = load("eight_scores_two_tiles.json")
    p = g["printed"]
    tol = 0.5 * 10 ** -g["printed_decimals"] + 1e-9
    s = np.array(g["s"], dtype=float)
    # C oracle with identity value rows: O = P
    q = np.zeros((1, 8)); q[0, 0] = 1.0
    K = np.zeros((8, 8)); K[:, 0] = s
    out, lse = oracle.attention_f64(q, K, np.eye(8), 1.0, causal=False)
    assert np.allclose(out[0], p["P"], atol=tol)
    assert abs(math.exp(lse[0] - p["m"]) - p["l"]) <= tol
    assert abs(out[0].sum() - 1.0) < 1e-14
    # recurrence in two tiles of four
    o, L, st = osm.attend_row(list(s), np.eye(8), 4)
    t1, t2 = st.trace
    assert t1["m"] == p["tile_1"]["m"]
    assert abs(t1["l"] - p["tile_1"]["l"]) <= tol
    assert np.allclose(t1["w"], p["tile_1"]["terms"], atol=tol)
    assert abs(t2["alpha"] - p["repair_factor"]) <= 0.5e-3
    assert t2["m"] == p["m"]
    assert abs(t2["l"] - p["l"]) <= tol
    assert np.allclose(o, p["P"], atol=tol)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_values(causal):
    """All keys equal: every permitted score of a row is the same, so the weights
    are uniform; O_i = mean of the permitted v_j and LSE_i = s_i + ln(count)."""
    rng = np.random.default_rng(1)
    N, d = 37, 16
    scale = f32(1 / math.sqrt(d))
    q = bf16_bits_to_f64(f64_to_bf16_bits(rng.standard_normal((N, d))))
    kv = bf16_bits_to_f64(f64_to_bf16_bits(rng.standard_normal(d)))
    K = np.tile(kv, (N, 1))
    V = bf16_bits_to_f64(f64_to_bf16_bits(rng.standard_normal((N, d))))
    out, lse = oracle.attention_f64(q, K, V, scale, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.allclose(out[i], V[:n].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - (scale * float(q[i] @ kv) + math.log(n))) < 1e-12


def test_one_dominant_key_selects_its_value():
    """k_j* = c q with c large and the other keys small: O ~ v_j*, within the bound
    sum_{j != j*} P_j |v_j - v_j*| computed from closed-form P."""
    rng = np.random.default_rng(2)
    N, d = 50, 8
    q = np.zeros(d); q[:4] = [1, -1, 0.5, 2]
    K = bf16_bits_to_f64(f64_to_bf16_bits(0.01 * rng.standard_normal((N, d))))
    jstar = 31
    K[jstar] = 8.0 * q
    V = bf16_bits_to_f64(f64_to_bf16_bits(rng.standard_normal((N, d))))
    out, _ = oracle.attention_f64(q[None, :], K, V, 1.0, causal=False)
    s = K @ q
    bound = 0.0
    for j in range(N):
        if j != jstar:
            bound += math.exp(s[j] - s[jstar]) * np.abs(V[j] - V[jstar]).max()
    assert bound < 1e-10
    assert np.abs(out[0] - V[jstar]).max() <= bound + 1e-15


def test_causal_row_zero_is_first_value_row():
    """Row 0 may only see key 0: O_0 = v_0 exactly, LSE_0 = scale q_0 . k_0."""
    q, k, v = random_qkv(11, 2, 3, 20, 32)
    scale = f32(1 / math.sqrt(32))
    rows = np.array([bh * 20 for bh in range(6)])
    out, lse = oracle.attention_rows(q, k, v, scale, True, rows)
    qf, kf, vf = (bf16_bits_to_f64(a).reshape(6, 20, 32) for a in (q, k, v))
    for t in range(6):
        assert np.array_equal(out[t], vf[t, 0])
        assert lse[t] == pytest.approx(scale * float(qf[t, 0] @ kf[t, 0]), abs=1e-13)


def test_causal_row_ignores_future_keys():
    """Changing keys and values after position i leaves row i unchanged (exactly),
    and changing any key before or at i changes it."""
    q, k, v = random_qkv(12, 1, 1, 30, 16)
    scale = f32(0.25)
    o1, l1 = oracle.attention_rows(q, k, v, scale, True)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 20:] ^= 0x0040
    v2[0, 0, 20:] ^= 0x0040
    o2, l2 = oracle.attention_rows(q, k2, v2, scale, True)
    assert np.array_equal(o1[:20], o2[:20]) and np.array_equal(l1[:20], l2[:20])
    assert not np.allclose(o1[20:], o2[20:])
    # non-causal rows all see the change
    o3, _ = oracle.attention_rows(q, k, v, scale, False)
    o4, _ = oracle.attention_rows(q, k2, v2, scale, False)
    assert np.all(np.abs(o3 - o4).max(axis=1) > 0)


def test_value_rows_of_ones_give_ones():
    """Rows of P sum to 1, so V = 1 gives O = 1 (both modes)."""
    q, k, _ = random_qkv(13, 1, 2, 45, 8, sigma_qk=3.0)
    v = np.full_like(q, f64_to_bf16_bits(np.array([1.0]))[0])
    for causal in (False, True):
        out, _ = oracle.attention_rows(q, k, v, 0.5, causal)
        assert np.abs(out - 1.0).max() < 1e-13


def test_large_scores_stay_finite_and_shift_invariant():
    """Scores near 1000 (exp overflows fp64 without the max subtraction) give the
    same O as the same scores shifted down, and LSE shifted by the same amount."""
    d = 4
    base = np.array([[0.0, 1.0, 2.0, 0.5, -1.0]]).T  # five keys
    q = np.array([[1.0, 1.0, 0.0, 0.0]])
    K0 = np.hstack([base, np.zeros((5, 1)), np.zeros((5, 2))])
    K1 = K0.copy(); K1[:, 1] = 1000.0        # every score + 1000
    V = np.arange(20, dtype=float).reshape(5, 4)
    o0, l0 = oracle.attention_f64(q, K0, V, 1.0, False)
    o1, l1 = oracle.attention_f64(q, K1, V, 1.0, False)
    assert np.all(np.isfinite(o1)) and np.isfinite(l1[0])
    assert np.allclose(o0, o1, atol=1e-12)
    assert l1[0] - l0[0] == pytest.approx(1000.0, abs=1e-9)
    ref = softmax(base[:, 0]) @ V
    assert np.allclose(o0[0], ref, atol=1e-13)
    assert l0[0] == pytest.approx(logsumexp(base[:, 0]), abs=1e-13)


# ---------------------------------------------------------------- brute force

def brute_force_row(qi, K, V, scale, nkeys):
    """Unshifted softmax with Python floats and math.fsum (a different evaluation
    from the oracle's shifted one; valid for the small scores used here)."""
    e = [math.exp(scale * math.fsum(float(a) * float(b) for a, b in zip(qi, K[j]))) for j in range(nkeys)]
    tot = math.fsum(e)
    o = [math.fsum(e[j] * float(V[j, c]) for j in range(nkeys)) / tot for c in range(V.shape[1])]
    return np.array(o), math.log(tot)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 1, 1, 4, False), (1, 1, 1, 4, True), (1, 2, 7, 8, False),
                                            (2, 1, 13, 16, True), (1, 1, 33, 64, False),
                                            (1, 1, 33, 64, True), (1, 1, 20, 128, True)])
def test_brute_force_tiny(B, H, N, d, causal):
    q, k, v = random_qkv(100 + N + d, B, H, N, d)
    scale = f32(1 / math.sqrt(d))
    out, lse = oracle.attention_rows(q, k, v, scale, causal)
    qf, kf, vf = (bf16_bits_to_f64(a).reshape(B * H, N, d) for a in (q, k, v))
    for bh in range(B * H):
        for i in range(N):
            o, L = brute_force_row(qf[bh, i], kf[bh], vf[bh], scale, i + 1 if causal else N)
            t = bh * N + i
            assert np.allclose(out[t], o, atol=1e-13, rtol=1e-12)
            assert abs(lse[t] - L) < 1e-12


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal", [(1, 1, 5, 17, 8, False), (1, 1, 5, 17, 8, True),
                                                (2, 1, 19, 6, 16, True), (1, 2, 19, 6, 16, False),
                                                (1, 1, 1, 40, 64, True), (1, 1, 40, 1, 64, True)])
def test_brute_force_nonsquare(B, H, Nq, Nk, d, causal):
    """Nq queries over Nk keys; causal is top-left: query i sees keys 0..min(i, Nk-1)
    ("How to profile and optimise kernels", Round 4: the non-square causal check
    against an explicit top-left mask)."""
    q, _, _ = random_qkv(300 + Nq, B, H, Nq, d)
    _, k, v = random_qkv(400 + Nk, B, H, Nk, d)
    scale = f32(1 / math.sqrt(d))
    out, lse = oracle.attention_rows(q, k, v, scale, causal)
    qf = bf16_bits_to_f64(q).reshape(B * H, Nq, d)
    kf, vf = (bf16_bits_to_f64(a).reshape(B * H, Nk, d) for a in (k, v))
    for bh in range(B * H):
        for i in range(Nq):
            n = min(i + 1, Nk) if causal else Nk
            o, L = brute_force_row(qf[bh, i], kf[bh], vf[bh], scale, n)
            t = bh * Nq + i
            assert np.allclose(out[t], o, atol=1e-13, rtol=1e-12)
            assert abs(lse[t] - L) < 1e-12


def test_nonsquare_identical_keys():
    """Identical keys, more queries than keys, causal: row i averages the first
    min(i+1, Nk) value rows exactly and LSE = s + ln(count)."""
    rng = np.random.default_rng(5)
    Nq, Nk, d = 12, 5, 16
    scale = f32(0.25)
    qb = f64_to_bf16_bits(rng.standard_normal((Nq, d))).reshape(1, 1, Nq, d)
    kv = f64_to_bf16_bits(rng.standard_normal(d))
    kb = np.tile(kv, (Nk, 1)).reshape(1, 1, Nk, d)
    vb = f64_to_bf16_bits(rng.standard_normal((Nk, d))).reshape(1, 1, Nk, d)
    out, lse = oracle.attention_rows(qb, kb, vb, scale, True)
    qf, kf, vf = bf16_bits_to_f64(qb)[0, 0], bf16_bits_to_f64(kv), bf16_bits_to_f64(vb)[0, 0]
    for i in range(Nq):
        n = min(i + 1, Nk)
        assert np.allclose(out[i], vf[:n].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - (scale * float(qf[i] @ kf) + math.log(n))) < 1e-12


def test_library_softmax_on_asymmetric_case():
    """scipy's softmax/logsumexp on Q K^T (not K Q^T): catches a transposed
    operand, since Q != K here."""
    q, k, v = random_qkv(21, 1, 1, 24, 16, sigma_qk=2.0)
    scale = f32(0.25)
    qf, kf, vf = (bf16_bits_to_f64(a)[0, 0] for a in (q, k, v))
    S = scale * (qf @ kf.T)
    for causal in (False, True):
        out, lse = oracle.attention_rows(q, k, v, scale, causal)
        for i in range(24):
            n = i + 1 if causal else 24
            assert np.allclose(out[i], softmax(S[i, :n]) @ vf[:n], atol=1e-12)
            assert lse[i] == pytest.approx(logsumexp(S[i, :n]), abs=1e-12)
        # the transposed reading disagrees
        assert not np.allclose(out[5], softmax(S[:24 if not causal else 6, 5]) @ vf[:24 if not causal else 6])


def test_sampled_rows_match_full_rows():
    """Asking for a subset of rows (any order) gives the same values as the full run."""
    q, k, v = random_qkv(22, 2, 2, 40, 32)
    full_o, full_l = oracle.attention_rows(q, k, v, 0.2, True)
    rows = np.array([159, 0, 77, 40, 3, 120])
    o, l = oracle.attention_rows(q, k, v, 0.2, True, rows)
    assert np.array_equal(o, full_o[rows]) and np.array_equal(l, full_l[rows])


# ---------------------------------------------------------------- recurrence vs definition

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_recurrence_equals_definition_any_tiling(seed):
    """The online recurrence reaches the two-pass result for every tiling
    (the induction argument), including uneven chunks and a maximum that only
    arrives in the last block."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(50, 300))
    d = 8
    q, k, v = random_qkv(300 + seed, 1, 1, N, d, sigma_qk=2.0)
    qf, kf, vf = (bf16_bits_to_f64(a)[0, 0] for a in (q, k, v))
    scale = f32(1 / math.sqrt(d))
    # plant the row maximum in the last key of row 0's sweep
    kf[-1] = 4.0 * qf[0]
    k2 = f64_to_bf16_bits(kf).reshape(1, 1, N, d)
    kf = bf16_bits_to_f64(k2)[0, 0]
    rows = [0, 1, N // 2, N - 1]
    out, lse = oracle.attention_rows(q, k2, v, scale, False, np.array(rows))
    for t, i in enumerate(rows):
        s = [scale * float(qf[i] @ kf[j]) for j in range(N)]
        tilings = [1, 2, 3, 4, 7, 16, 64, N]
        cuts = sorted(set(int(x) for x in rng.integers(1, N, size=6)))
        tilings.append([b - a for a, b in zip([0] + cuts, cuts + [N])])  # 7 uneven chunks
        for tiling in tilings:
            o, L, _ = osm.attend_row(s, vf, tiling)
            assert np.allclose(o, out[t], atol=1e-12, rtol=1e-12)
            assert abs(L - lse[t]) < 1e-12


def test_forgetting_the_rescale_is_caught():
    """Dropping alpha (the page's 'forget the rescale' failure) changes the result
    when the maximum arrives late, so the recurrence test above has teeth."""
    s = [0.0, 1.0, 0.5, 6.0]
    V = np.eye(4)
    o_ok, _, _ = osm.attend_row(s, V, 2)
    # hand-run the recurrence without alpha
    m, l, o = -math.inf, 0.0, np.zeros(4)
    for blk in ([0, 1], [2, 3]):
        m_new = max(m, max(s[j] for j in blk))
        w = [math.exp(s[j] - m_new) for j in blk]
        l = l + sum(w)
        o = o + sum(wj * V[j] for wj, j in zip(w, blk))
        m = m_new
    assert not np.allclose(o / l, o_ok, atol=1e-3)
    assert np.allclose(o_ok, softmax(s), atol=1e-15)


def test_first_block_alpha_is_zero_not_nan():
    st = osm.RowState()
    osm.update(st, [3.0, -2.0], np.eye(2))
    assert st.trace[0]["alpha"] == 0.0
    assert np.all(np.isfinite(st.o))


def test_whole_head_recurrence_matches_oracle():
    q, k, v = random_qkv(31, 1, 1, 48, 16)
    qf, kf, vf = (bf16_bits_to_f64(a)[0, 0] for a in (q, k, v))
    for causal in (False, True):
        o_ref, l_ref = oracle.attention_rows(q, k, v, 0.25, causal)
        o, l = osm.attention_recurrence(qf, kf, vf, 0.25, causal, block=16)
        assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)


# ---------------------------------------------------------------- merge of partial states

def test_merge_reproduces_the_two_block_example():
    """The state of block 1 merged with the state block 2 has on its own is the
    printed state after block 2 (m = ln 2, l = 3, o = [1.5, 1.5]) and O = [1/2, 1/2]
    ("4 Triton and Custom Kernels", section 4.8 worked example)."""
    g = load("online_softmax_two_blocks.json")
    s = [num(x) for x in g["scores"]]
    V = np.array(g["V"], dtype=float)
    a = osm.update(osm.RowState(), s[:2], V[:2])
    b = osm.update(osm.RowState(), s[2:], V[2:])
    mg = osm.merge(a, b)
    after = g["printed"]["after_block_2"]
    assert mg.m == pytest.approx(num(after["m"]), abs=1e-15)
    assert mg.l == pytest.approx(after["l"], abs=1e-15)
    assert np.allclose(mg.o, after["o"], atol=1e-15)
    assert np.allclose(mg.o / mg.l, g["printed"]["output"], atol=1e-15)


def test_merge_of_any_split_equals_the_whole_row():
    """Key splits of any sizes, each run through the recurrence and then merged in
    any order, give the definition's O and LSE; the empty state is the identity."""
    rng = np.random.default_rng(9)
    for trial in range(20):
        n = int(rng.integers(2, 200))
        s = list(rng.standard_normal(n) * 4.0)
        V = rng.standard_normal((n, 8))
        w = np.exp(np.array(s) - max(s))
        ref_o, ref_l = (w @ V) / w.sum(), max(s) + math.log(w.sum())
        cuts = sorted(set(int(c) for c in rng.integers(1, n, size=int(rng.integers(1, 6)))))
        parts = [(a, b) for a, b in zip([0] + cuts, cuts + [n]) if b > a]
        states = [osm.update(osm.RowState(), s[a:b], V[a:b]) for a, b in parts]
        rng.shuffle(states)
        acc = osm.RowState()
        for st in states:
            acc = osm.merge(acc, st)
        assert np.allclose(acc.o / acc.l, ref_o, atol=1e-12)
        assert acc.m + math.log(acc.l) == pytest.approx(ref_l, abs=1e-12)


def test_merge_with_empty_state_is_identity():
    a = osm.update(osm.RowState(), [0.5, -1.0], np.eye(2))
    for m in (osm.merge(a, osm.RowState()), osm.merge(osm.RowState(), a)):
        assert m.m == a.m and m.l == a.l and np.array_equal(m.o, a.o)


def _lazy_row(scores, values, block, margin):
    """The recurrence with a lazy reference maximum (the GPU kernel's variant):
    the reference m moves to a block's maximum only when that maximum exceeds m
    by more than `margin`; O / l and m + ln l are then used as usual."""
    m, l, o = -math.inf, 0.0, np.zeros(values.shape[1])
    for a in range(0, len(scores), block):
        s = np.asarray(scores[a:a + block])
        bm = s.max()
        m_new = bm if bm > m + margin else m
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        p = np.exp(s - m_new)
        l = alpha * l + p.sum()
        o = alpha * o + p @ values[a:a + block]
        m = m_new
    return o / l, m + math.log(l)


@pytest.mark.parametrize("margin", [0.0, 8.0 * math.log(2.0), 30.0])
def test_lazy_reference_maximum_equals_definition(margin):
    """O = sum P V / sum P and LSE = m + ln l hold for any reference m, so a
    maximum that lags the true one by up to the margin gives the definition's
    result (here against the oracle, with an increasing score sequence that
    forces the reference to move, and a late maximum)."""
    rng = np.random.default_rng(9)
    N, d = 300, 8
    q, k, v = random_qkv(900, 1, 1, N, d, sigma_qk=2.0)
    qf, kf, vf = (bf16_bits_to_f64(a)[0, 0] for a in (q, k, v))
    scale = f32(1 / math.sqrt(d))
    kf = kf * np.linspace(0.2, 3.0, N)[:, None]          # scores of row 0 drift upward
    k2 = f64_to_bf16_bits(kf).reshape(1, 1, N, d)
    kf = bf16_bits_to_f64(k2)[0, 0]
    rows = np.array([0, 7, N - 1])
    out, lse = oracle.attention_rows(q, k2, v, scale, False, rows)
    for t, i in enumerate(rows):
        s = [scale * float(qf[i] @ kf[j]) for j in range(N)]
        for block in (16, 64):
            o, L = _lazy_row(s, vf, block, margin)
            assert np.allclose(o, out[t], atol=1e-11, rtol=1e-11)
            assert abs(L - lse[t]) < 1e-11
