"""fa.attention as a torch.autograd function: its gradients are the backward
kernels' (bit for bit) and match the oracle; [B, N, H, d] views and Nq != Nk
work through autograd; and a few SGD steps through it reduce a loss."""
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
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d,causal", [(32, True), (64, False), (128, True)])
def test_gradients_are_the_kernels_and_match_the_oracle(d, causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N = 1, 2, 300
    q, k, v = random_qkv(7100 + d, B, H, N, d)
    g = normal_bits(7150 + d, B * H * N * d).reshape(B, H, N, d)
    tq, tk, tv = (to_device(a).requires_grad_() for a in (q, k, v))
    tg = to_device(g)
    out = fa.attention(tq, tk, tv, causal=causal)
    (out * tg).sum().backward()          # d loss / d out = g, in out's dtype
    torch.cuda.synchronize()
    o2, lse = fa.fa_fwd_ex(tq.detach(), tk.detach(), tv.detach(), scale=fp32_scale(d), causal=causal)
    ref_kernels = fa.fa_bwd_ex(tq.detach(), tk.detach(), tv.detach(), o2, lse, tg, scale=fp32_scale(d), causal=causal)
    for t, r in zip((tq, tk, tv), ref_kernels):
        assert torch.equal(t.grad.view(torch.int16), r.view(torch.int16))
    ref = oracle.attention_bwd(q, k, v, g, fp32_scale(d), causal)
    for name, t, r in zip(("dq", "dk", "dv"), (tq, tk, tv), ref):
        compare_grad(bits_of(t.grad), r, label="autograd d%d c%d %s" % (d, causal, name))


def test_bnhd_views_and_non_square():
    """Leaves stored [B, N, H, d]; the kernels see transposed views, and autograd
    hands each leaf its gradient in the leaf's own layout."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, Nq, Nk, d = 2, 2, 100, 260, 64
    q, _, _ = random_qkv(7200, B, H, Nq, d)
    _, k, v = random_qkv(7201, B, H, Nk, d)
    g = normal_bits(7202, B * H * Nq * d).reshape(B, H, Nq, d)
    leaves = [to_device(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).requires_grad_() for a in (q, k, v)]
    out = fa.attention(*(t.transpose(1, 2) for t in leaves), causal=True)
    (out * to_device(g)).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, g, fp32_scale(d), True)
    for name, t, r in zip(("dq", "dk", "dv"), leaves, ref):
        assert t.grad.shape == t.shape
        compare_grad(bits_of(t.grad.transpose(1, 2)), r, label="autograd [B,N,H,d] %s" % name)


def test_sgd_through_attention_reduces_the_loss():
    import torch
    import flashattention_forward_fa2_amd as fa
    torch.manual_seed(0)
    dev = torch.device("cuda:0")
    B, H, N, d = 1, 4, 256, 64
    x = (torch.randn(B, H, N, d, device=dev) * 0.5).to(torch.bfloat16)
    target = torch.randn(B, H, N, d, device=dev).to(torch.bfloat16)
    wq = torch.randn(d, d, device=dev, requires_grad=True)
    wk = torch.randn(d, d, device=dev, requires_grad=True)
    losses = []
    for _ in range(20):
        q = (x.float() @ wq).to(torch.bfloat16)
        k = (x.float() @ wk).to(torch.bfloat16)
        out = fa.attention(q, k, x, causal=True)
        loss = ((out.float() - target.float()) ** 2).mean()
        losses.append(float(loss.detach()))
        wq.grad = wk.grad = None
        loss.backward()
        with torch.no_grad():
            wq -= 0.5 * wq.grad
            wk -= 0.5 * wk.grad
    assert all(np.isfinite(losses)) and losses[-1] < losses[0]
