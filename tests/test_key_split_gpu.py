"""GPU parity of the key-split tile (fa_tile_cfg (1, 4, 32, ksplit 4): four
wavefronts share each block of 32 queries, sweep every fourth key tile each and
merge their partial softmax states inside the workgroup) against the fp64 CPU
oracle, through the C ABI: Nq queries over Nk keys with the top-left causal mask
(including query blocks past the last key and sweeps in which some wavefronts
get no key tile), [B, N, H, d] strided views, fp16, and peaked scores whose
partial maxima differ widely between the wavefronts of a block; every row is
compared.  Also: the default launch of a short workload is this tile and is
bit-identical to naming it."""
import numpy as np
import pytest

import oracle
from inputs import random_qkv
from parity import compare, fp32_scale, to_device

pytestmark = pytest.mark.gpu

KS = (1, 4, 32, 4)


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


def run(q, k, v, d, causal, dtype="bf16", bnhd=False, cfg=KS):
    import torch
    import flashattention_forward_fa2_amd as fa
    tq, tk, tv = (to_device(a, dtype=dtype) for a in (q, k, v))
    if bnhd:  # stored [B, N, H, d]; the kernel sees [B, H, N, d] views with row stride H*d
        tq, tk, tv = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (tq, tk, tv))
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=fp32_scale(d), causal=causal, cfg=cfg)  # cfg None: the default
    torch.cuda.synchronize()
    return out, lse


def check(q, k, v, d, causal, label, dtype="bf16", **kw):
    out, lse = run(q, k, v, d, causal, dtype=dtype, **kw)
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), causal, dtype=dtype)
    tol = dict(o_max=4e-3, o_mean=3e-4) if dtype == "f16" else {}
    compare(bits_of(out), lse.contiguous().cpu().numpy(), o_ref, l_ref, label=label, dtype=dtype, **tol)
    return out, lse


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (5, 40), (40, 5), (33, 97), (200, 64), (64, 200), (300, 1000),
                                   (1000, 300), (257, 257)])
def test_lengths(Nq, Nk, d, causal):
    """Nk = 1 .. 1000: one to 32 key tiles, so a block's four wavefronts get from
    zero to eight tiles each; causal blocks past the last key see all of them."""
    q, _, _ = random_qkv(8100 + Nq, 1, 2, Nq, d)
    _, k, v = random_qkv(8200 + Nk, 1, 2, Nk, d)
    check(q, k, v, d, causal, "key split Nq=%d Nk=%d d=%d causal=%d" % (Nq, Nk, d, causal))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_peaked_scores(d, causal):
    """Q, K ~ N(0, 4^2): each wavefront's reference maximum moves often and the
    four partial maxima of a row differ by many units, so the merge weights
    2^(m_w - M) span a wide range."""
    q, k, v = random_qkv(8300 + d, 2, 3, 777, d, sigma_qk=4.0)
    check(q, k, v, d, causal, "key split peaked d=%d causal=%d" % (d, causal))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_strided_and_fp16(d, dtype):
    """[B, N, H, d] views (the strided instantiation) in bf16 and fp16, both masks,
    and bit-identity with the contiguous launch of the same tile."""
    import torch
    for causal in (0, 1):
        q, k, v = random_qkv(8400 + d + causal, 2, 3, 450, d, dtype=dtype)
        out, lse = check(q, k, v, d, causal, "key split bnhd %s d=%d causal=%d" % (dtype, d, causal), dtype=dtype,
                         bnhd=True)
        o2, l2 = run(q, k, v, d, causal, dtype=dtype)
        assert torch.equal(out.contiguous().view(torch.int16), o2.view(torch.int16))
        assert torch.equal(lse.contiguous(), l2)


@pytest.mark.parametrize("causal", [0, 1])
def test_default_short_workload_uses_the_tile(causal):
    """B1 H8 N1024 d64 (the short multi-head workload) launches the key-split
    tile by default on a 256-CU device, bit-identical to naming it."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N, d = 1, 8, 1024, 64
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert fa.launch_cfg(B, H, N, d, bool(causal)) == KS
    q, k, v = (to_device(a) for a in random_qkv(8500 + causal, B, H, N, d))
    o1, l1 = fa.fa_fwd(q, k, v, scale=fp32_scale(d), causal=bool(causal))
    o2, l2 = fa.fa_fwd(q, k, v, scale=fp32_scale(d), causal=bool(causal), cfg=fa.launch_cfg(B, H, N, d, bool(causal)))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128])
def test_long_key_range(d):
    """100 queries over 2^20 + 17 keys (the default tile on this small grid):
    each wavefront sweeps 8192 key tiles, whose byte offsets inside the head
    reach 2^28 (d = 128), the last tile ragged; every row, both masks (causal
    top-left: query i sees keys 0..i only)."""
    import flashattention_forward_fa2_amd as fa
    Nq, Nk = 100, (1 << 20) + 17
    assert fa.launch_cfg(1, 1, Nq, d, False) == KS and fa.launch_cfg(1, 1, Nq, d, True) == KS
    q, _, _ = random_qkv(8600 + d, 1, 1, Nq, d)
    _, k, v = random_qkv(8700 + d, 1, 1, Nk, d)
    for causal in (0, 1):
        check(q, k, v, d, causal, "key split long Nk=%d d=%d causal=%d" % (Nk, d, causal), cfg=None)
