"""GPU parity of the split-key path (fa_fwd_splitkv: per-split partial results,
then the merge kernel) against the fp64 CPU oracle, and against fa_fwd_ex."""
import numpy as np
import pytest

import oracle
from inputs import random_qkv
from parity import compare, fp32_scale, to_device

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


def qkv(seed, B, H, Nq, Nk, d):
    q, _, _ = random_qkv(seed, B, H, Nq, d)
    _, k, v = random_qkv(seed + 1, B, H, Nk, d)
    return q, k, v


@pytest.mark.parametrize("B,H,Nq,Nk,d,causal,S", [
    (1, 8, 1024, 1024, 64, 0, 0), (1, 8, 1024, 1024, 64, 1, 0),   # the B1-H8-N1024 workload, default splits
    (1, 1, 256, 256, 64, 0, 4),                                  # the B1-H1-N256 workload, 4 splits
    (1, 4, 1, 8192, 128, 0, 16), (1, 4, 1, 8192, 128, 1, 16),    # one query over a long key range
    (1, 2, 37, 3000, 64, 1, 5), (2, 2, 300, 777, 128, 1, 3),
    (1, 1, 5, 100, 64, 0, 16),                                    # more splits asked than key tiles
    (2, 3, 7, 2000, 32, 1, 0), (1, 2, 1, 5000, 32, 0, 0),         # d = 32, default splits
    (1, 2, 32, 3000, 128, 1, 0),                                  # a full 32-query block, default splits
])
def test_splitkv_matches_oracle(B, H, Nq, Nk, d, causal, S):
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(7000 + Nq + Nk + S, B, H, Nq, Nk, d)
    out, lse = fa.fa_fwd_splitkv(to_device(q), to_device(k), to_device(v), scale=fp32_scale(d), causal=bool(causal),
                                 num_splits=S)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), causal)
    compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref,
            label="splitkv B%d H%d Nq=%d Nk=%d d=%d c=%d S=%d" % (B, H, Nq, Nk, d, causal, S))


@pytest.mark.parametrize("causal", [0, 1])
def test_one_split_is_bit_identical_to_fa_fwd_ex(causal):
    """With one split the merge divides by exp(0) = 1: same bits as the direct path
    launched with the split path's tile (for Nq = 300 the default 8-wavefront
    tile; the direct path's own choice on this small grid is the key-split tile)."""
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(7100 + causal, 2, 3, 300, 500, 64)
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    o1, l1 = fa.fa_fwd_ex(tq, tk, tv, causal=bool(causal), cfg=(1, 8, 64))
    o2, l2 = fa.fa_fwd_splitkv(tq, tk, tv, causal=bool(causal), num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_strided_layout_and_reused_workspace():
    """[B, N, H, d] views through the split path; one workspace serves two calls
    of different shapes in a row (its contents are scratch)."""
    import torch
    import flashattention_forward_fa2_amd as fa
    d = 128
    ws = torch.empty(fa.splitkv_workspace_bytes(2, 3, 200, 2500, d, 6), dtype=torch.uint8, device="cuda")
    for seed, (Nq, Nk, S) in enumerate([(200, 2500, 6), (50, 900, 3)]):
        q, k, v = qkv(7200 + seed, 2, 3, Nq, Nk, d)
        tq, tk, tv = (to_device(a).permute(0, 2, 1, 3).contiguous().transpose(1, 2) for a in (q, k, v))
        out, lse = fa.fa_fwd_splitkv(tq, tk, tv, scale=fp32_scale(d), causal=True, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), True)
        compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref, label="splitkv bnhd Nq=%d Nk=%d" % (Nq, Nk))
