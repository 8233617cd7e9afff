"""GPU parity of the backward (fa_bwd, through the C ABI) against the fp64 CPU
oracle's gradients: ragged lengths, both head dims and masks, the degenerate
one-token head, determinism, a reused workspace, and the B4-H8-N4096 d64
workload on a sample of heads."""
import numpy as np
import pytest

import oracle
from inputs import normal_bf16, random_qkv
from parity import compare_grad, fp32_scale, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_fa2_amd as fa
    fa.load_library()
    return torch.device("cuda:0")


def bits_of(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def problem(seed, B, H, N, d):
    q, k, v = random_qkv(seed, B, H, N, d)
    dout = normal_bf16(seed + 3, B * H * N * d).reshape(B, H, N, d)
    return q, k, v, dout


def gpu_grads(q, k, v, dout, scale, causal, workspace=None):
    import torch
    import flashattention_forward_fa2_amd as fa
    tq, tk, tv, tg = (to_device(a) for a in (q, k, v, dout))
    out, lse = fa.fa_fwd(tq, tk, tv, scale=scale, causal=bool(causal))
    dq, dk, dv = fa.fa_bwd(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal), workspace=workspace)
    torch.cuda.synchronize()
    return bits_of(dq), bits_of(dk), bits_of(dv)


def check(seed, B, H, N, d, causal, heads=None):
    q, k, v, dout = problem(seed, B, H, N, d)
    scale = fp32_scale(d)
    got = gpu_grads(q, k, v, dout, scale, causal)
    if heads is not None:  # the oracle on a sample of (b, h) pairs: heads are independent
        sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
        got = tuple(sel(g.reshape(B, H, N, d)) for g in got)
        q, k, v, dout = (sel(a) for a in (q, k, v, dout))
    ref = oracle.attention_bwd(q, k, v, dout, scale, causal)
    label = "bwd B%d H%d N%d d%d c%d" % (B, H, N, d, causal)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        compare_grad(g, r, label="%s %s" % (label, name))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,H,N", [(1, 2, 256), (2, 2, 300), (1, 3, 77), (1, 2, 1000)])
def test_bwd_matches_oracle(B, H, N, d, causal):
    check(9000 + N + d + causal, B, H, N, d, causal)


@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_b1_h8_n1024(causal):
    check(9100 + causal, 1, 8, 1024, 64, causal)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_single_token_head(d):
    """N = 1: P = 1, so dv = dout and dq = dk = 0 up to the rounding of dP - D."""
    q, k, v, dout = problem(9200 + d, 2, 2, 1, d)
    dq, dk, dv = gpu_grads(q, k, v, dout, fp32_scale(d), 0)
    assert np.array_equal(dv, dout)
    from inputs import bf16_bits_to_f64
    assert np.abs(bf16_bits_to_f64(dq)).max() < 1e-4
    assert np.abs(bf16_bits_to_f64(dk)).max() < 1e-4


def test_deterministic_and_workspace_reuse():
    """No atomics: two calls give the same bits; one workspace serves two shapes."""
    import torch
    import flashattention_forward_fa2_amd as fa
    ws = torch.empty(fa.bwd_workspace_bytes(2, 4, 700, 128), dtype=torch.uint8, device="cuda")
    for seed, (N, d) in enumerate([(700, 128), (333, 64)]):
        q, k, v, dout = problem(9300 + seed, 2, 4, N, d)
        a = gpu_grads(q, k, v, dout, fp32_scale(d), 1, workspace=ws)
        b = gpu_grads(q, k, v, dout, fp32_scale(d), 1, workspace=ws)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        ref = oracle.attention_bwd(q, k, v, dout, fp32_scale(d), True)
        for name, g, r in zip(("dq", "dk", "dv"), a, ref):
            compare_grad(g, r, label="ws N%d d%d %s" % (N, d, name))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_bwd_b4_h8_n4096_sampled_heads(causal, d):
    """The B4-H8-N4096 workload on the GPU (d = 64; d = 32 and 128, whose causal
    launches keep several workgroups per CU and reorder co-resident layers);
    the oracle on one head per batch."""
    check(9400 + causal + d, 4, 8, 4096, d, causal, heads=[(0, 0), (1, 3), (2, 5), (3, 7)])
