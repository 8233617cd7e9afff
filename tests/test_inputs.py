"""Seeded input generator: determinism, rounding and distribution. CPU only."""
import math

import numpy as np
import torch

import inputs


def test_splitmix64_matches_scalar_definition():
    """Vectorised outputs equal a scalar run of the published SplitMix64 steps."""
    mask = (1 << 64) - 1

    def scalar(seed, i):
        z = (seed + (i + 1) * 0x9E3779B97F4A7C15) & mask
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        return z ^ (z >> 31)

    seed = 0xFA2F0031
    got = inputs.splitmix64(seed, np.arange(64, dtype=np.uint64))
    assert [int(x) for x in got] == [scalar(seed, i) for i in range(64)]


def test_generator_is_deterministic_and_chunk_independent():
    a = inputs.normal_bf16(5, 3 * (1 << 22) + 17)
    b = inputs.normal_bf16(5, 3 * (1 << 22) + 17, threads=1)
    assert np.array_equal(a, b)
    c = inputs.normal_bf16(5, 1001)
    assert np.array_equal(a[:1001], c)
    assert not np.array_equal(inputs.normal_bf16(6, 1001), c)


def test_bf16_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7
    cases = [
        (one, 0x3F80),
        (one + ulp / 2, 0x3F80),                 # tie -> even (mantissa 0)
        (one + 1.5 * ulp, 0x3F82),               # tie -> even (mantissa 2)
        (one + ulp / 2 + 2.0 ** -40, 0x3F81),    # just above the tie (fp64-only bits)
        (-(one + ulp / 2 + 2.0 ** -40), 0xBF81),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.0, 0x4040),
    ]
    got = inputs.f64_to_bf16_bits(np.array([x for x, _ in cases]))
    assert [int(x) for x in got] == [b for _, b in cases]


def test_bf16_rounding_matches_torch_on_fp32_values():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32)
    ours = inputs.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_normal_moments():
    x = inputs.bf16_bits_to_f64(inputs.normal_bf16(9, 1 << 20, sigma=4.0))
    assert abs(x.mean()) < 0.02
    assert abs(x.std() - 4.0) < 0.02
    assert abs(((x / 4.0) ** 4).mean() - 3.0) < 0.05


def test_workload_shapes_and_seeds():
    q, k, v = inputs.make_qkv(1)
    assert q.shape == (1, 1, 256, 64) and q.dtype == np.uint16
    assert not np.array_equal(q, k) and not np.array_equal(k, v)
    q2, _, _ = inputs.make_qkv(1)
    assert np.array_equal(q, q2)
    assert inputs.workload_seed(3, 2) == 0xFA2F0000 + 48 + 2
    assert inputs.default_scale(64) == 0.125
    assert inputs.default_scale(128) == float(np.float32(1 / math.sqrt(128)))


def test_sample_rows():
    r = inputs.sample_rows(1234, 2, 3, 4096, per_head=64)
    assert r.dtype == np.int64 and np.all(np.diff(r) > 0)
    heads = r // 4096
    assert set(heads.tolist()) == set(range(6))
    for bh in range(6):
        rows = r[heads == bh] % 4096
        assert {0, 1, 4094, 4095, 2047, 2048}.issubset(set(rows.tolist()))
        assert 16 <= rows.size <= 64
