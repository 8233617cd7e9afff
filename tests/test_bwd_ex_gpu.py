"""GPU parity of the descriptor backward (fa_bwd_ex, through the C ABI): fp16
inputs against the fp64 oracle on fp16-decoded values, [B, N, H, d] and packed
QKV / dQKV layouts against the oracle, and bit-identity of the strided kernels
with the contiguous ones on the same values."""
import numpy as np
import pytest

import oracle
from inputs import normal_bits, random_qkv
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


def problem(seed, B, H, N, d, dtype):
    q, k, v = random_qkv(seed, B, H, N, d, dtype=dtype)
    dout = normal_bits(seed + 3, B * H * N * d, dtype=dtype).reshape(B, H, N, d)
    return q, k, v, dout


def bnhd_view(bits, dtype):
    """A [B, H, N, d] device view whose memory is [B, N, H, d] (a transpose)."""
    t = to_device(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), dtype=dtype)
    return t.transpose(1, 2)


def oracle_check(got, q, k, v, dout, scale, causal, dtype, label):
    ref = oracle.attention_bwd(q, k, v, dout, scale, causal, dtype=dtype)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        compare_grad(g, r, label="%s %s" % (label, name), dtype=dtype)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("B,H,N", [(1, 2, 300), (2, 1, 77), (1, 1, 1000)])
def test_f16_matches_oracle(B, H, N, d, causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v, dout = problem(9300 + N + d + causal, B, H, N, d, "f16")
    scale = fp32_scale(d)
    tq, tk, tv, tg = (to_device(a, dtype="f16") for a in (q, k, v, dout))
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal))
    grads = fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal))
    torch.cuda.synchronize()
    oracle_check([bits_of(g) for g in grads], q, k, v, dout, scale, causal, "f16",
                 "bwd f16 B%d H%d N%d d%d c%d" % (B, H, N, d, causal))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_bnhd_layout_matches_oracle(dtype, d, causal):
    """Every tensor in [B, N, H, d] memory, lse in a padded [B, H, N + 40] buffer."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N = 2, 3, 200
    q, k, v, dout = problem(9400 + d + causal, B, H, N, d, dtype)
    scale = fp32_scale(d)
    tq, tk, tv, tg = (bnhd_view(a, dtype) for a in (q, k, v, dout))
    et = tq.dtype
    out = torch.empty((B, N, H, d), dtype=et, device=tq.device).transpose(1, 2)
    lse = torch.full((B, H, N + 40), float("nan"), dtype=torch.float32, device=tq.device)[:, :, :N]
    fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal), out=out, lse=lse)
    grads = [torch.full((B, N, H, d), float("nan"), dtype=et, device=tq.device).transpose(1, 2) for _ in range(3)]
    fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal), dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    oracle_check([bits_of(g) for g in grads], q, k, v, dout, scale, causal, dtype,
                 "bwd %s [B,N,H,d] d%d c%d" % (dtype, d, causal))


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 64, 1), ("f16", 128, 0)])
def test_packed_qkv_and_dqkv(dtype, d, causal):
    """q, k, v read from one [B, N, 3, H, d] tensor and dq, dk, dv written
    interleaved into another: the layout of a fused QKV projection."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N = 1, 4, 333
    q, k, v, dout = problem(9500 + d, B, H, N, d, dtype)
    scale = fp32_scale(d)
    qkv_bits = np.stack([a.transpose(0, 2, 1, 3) for a in (q, k, v)], axis=2)  # [B, N, 3, H, d]
    qkv = to_device(np.ascontiguousarray(qkv_bits), dtype=dtype)
    tq, tk, tv = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    tg = bnhd_view(dout, dtype)
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal))
    dqkv = torch.full((B, N, 3, H, d), float("nan"), dtype=qkv.dtype, device=qkv.device)
    views = [dqkv[:, :, i].transpose(1, 2) for i in range(3)]
    fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal), dq=views[0], dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    oracle_check([bits_of(g) for g in views], q, k, v, dout, scale, causal, dtype,
                 "bwd %s packed d%d c%d" % (dtype, d, causal))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_strided_bit_identical_to_contiguous(d, causal):
    """Same values, different addressing: the strided kernels do the same
    arithmetic in the same order, so every gradient bit agrees with fa_bwd."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N = 2, 2, 517
    q, k, v, dout = problem(9600 + d + causal, B, H, N, d, "bf16")
    scale = fp32_scale(d)
    cq, ck, cv, cg = (to_device(a) for a in (q, k, v, dout))
    out, lse = fa.fa_fwd(cq, ck, cv, scale=scale, causal=bool(causal))
    ref = fa.fa_bwd(cq, ck, cv, out, lse, cg, scale=scale, causal=bool(causal))
    again = fa.fa_bwd_ex(cq, ck, cv, out, lse, cg, scale=scale, causal=bool(causal))  # contiguous descriptor
    sq, sk, sv, sg = (bnhd_view(a, "bf16") for a in (q, k, v, dout))
    so = torch.empty((B, N, H, d), dtype=out.dtype, device=out.device).transpose(1, 2)
    so.copy_(out)
    sl = torch.empty((B, H, N + 8), dtype=torch.float32, device=out.device)[:, :, :N]
    sl.copy_(lse)
    strided = fa.fa_bwd_ex(sq, sk, sv, so, sl, sg, scale=scale, causal=bool(causal),
                           dq=torch.empty((B, N, H, d), dtype=out.dtype, device=out.device).transpose(1, 2),
                           dk=torch.empty((B, N, H, d), dtype=out.dtype, device=out.device).transpose(1, 2),
                           dv=torch.empty((B, N, H, d), dtype=out.dtype, device=out.device).transpose(1, 2))
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv"), ref, again, strided):
        assert np.array_equal(bits_of(a), bits_of(b)), name
        assert np.array_equal(bits_of(a), bits_of(c)), name


def test_f16_single_token_head():
    """N = 1: P = 1 exactly, so dv = dout bit for bit and dq = dk = 0 to rounding."""
    import torch
    import flashattention_forward_fa2_amd as fa
    from inputs import f16_bits_to_f64
    q, k, v, dout = problem(9700, 2, 2, 1, 64, "f16")
    tq, tk, tv, tg = (to_device(a, dtype="f16") for a in (q, k, v, dout))
    out, lse = fa.fa_fwd_ex(tq, tk, tv)
    dq, dk, dv = fa.fa_bwd_ex(tq, tk, tv, out, lse, tg)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(dv), dout)
    assert np.abs(f16_bits_to_f64(bits_of(dq))).max() < 1e-4
    assert np.abs(f16_bits_to_f64(bits_of(dk))).max() < 1e-4


@pytest.mark.parametrize("N,d,causal", [(2048, 64, 0), (2048, 128, 1)])
def test_f16_long_head_matches_oracle(N, d, causal):
    """fp16 over long heads (eight 256-key tiles): one whole head per case against the oracle."""
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v, dout = problem(9800 + d, 1, 1, N, d, "f16")
    scale = fp32_scale(d)
    tq, tk, tv, tg = (to_device(a, dtype="f16") for a in (q, k, v, dout))
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal))
    grads = fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal))
    torch.cuda.synchronize()
    oracle_check([bits_of(g) for g in grads], q, k, v, dout, scale, causal, "f16",
                 "bwd f16 N%d d%d c%d" % (N, d, causal))


def problem_qk(seed, B, H, Nq, Nk, d, dtype):
    q, _, _ = random_qkv(seed, B, H, Nq, d, dtype=dtype)
    _, k, v = random_qkv(seed + 1, B, H, Nk, d, dtype=dtype)
    dout = normal_bits(seed + 3, B * H * Nq * d, dtype=dtype).reshape(B, H, Nq, d)
    return q, k, v, dout


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Nq,Nk", [(100, 300), (300, 100), (1, 517), (517, 33), (64, 600)])
def test_non_square_matches_oracle(Nq, Nk, d, causal):
    """Nq queries over Nk keys (top-left causal), against the oracle; with
    causal and Nq < Nk the keys j >= Nq are seen by no query and their dk, dv
    rows must be exactly zero."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H = 1, 2
    q, k, v, dout = problem_qk(9900 + Nq + Nk + d + causal, B, H, Nq, Nk, d, "bf16")
    scale = fp32_scale(d)
    tq, tk, tv, tg = (to_device(a) for a in (q, k, v, dout))
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal))
    grads = fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal))
    torch.cuda.synchronize()
    got = [bits_of(g) for g in grads]
    assert got[0].shape == (B, H, Nq, d) and got[1].shape == got[2].shape == (B, H, Nk, d)
    oracle_check(got, q, k, v, dout, scale, causal, "bf16", "bwd Nq%d Nk%d d%d c%d" % (Nq, Nk, d, causal))
    if causal and Nq < Nk:
        assert not np.any(got[1][:, :, Nq:]) and not np.any(got[2][:, :, Nq:])


@pytest.mark.parametrize("causal", [0, 1])
def test_non_square_strided_f16(causal):
    """fp16, [B, N, H, d] memory for every tensor, 200 queries over 77 keys."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, Nq, Nk, d = 2, 3, 200, 77, 64
    q, k, v, dout = problem_qk(9950 + causal, B, H, Nq, Nk, d, "f16")
    scale = fp32_scale(d)
    tq, tk, tv, tg = (bnhd_view(a, "f16") for a in (q, k, v, dout))
    out = torch.empty((B, Nq, H, d), dtype=torch.float16, device=tq.device).transpose(1, 2)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=tq.device)
    fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=bool(causal), out=out, lse=lse)
    dq = torch.full((B, Nq, H, d), float("nan"), dtype=torch.float16, device=tq.device).transpose(1, 2)
    dk, dv = (torch.full((B, Nk, H, d), float("nan"), dtype=torch.float16, device=tq.device).transpose(1, 2)
              for _ in range(2))
    fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=bool(causal), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    oracle_check([bits_of(g) for g in (dq, dk, dv)], q, k, v, dout, scale, causal, "f16",
                 "bwd f16 [B,N,H,d] Nq%d Nk%d c%d" % (Nq, Nk, causal))
