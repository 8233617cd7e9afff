"""Grouped-query attention through strides alone: H query heads over Hkv key /
value heads (G = H / Hkv query heads per key head).  The query heads of one
group become one "batch" entry over a single key head with head stride 0;
the forward matches the oracle on K, V repeated to every query head, and the
backward's per-query-head dK, dV summed over each group match the oracle's
gradients of the shared heads."""
import numpy as np
import pytest

import oracle
from inputs import normal_bits, random_qkv
from parity import compare, compare_grad, fp32_scale, to_device

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


@pytest.mark.parametrize("Hkv,G,causal", [(2, 4, True), (1, 6, False), (3, 2, True)])
def test_grouped_query_attention(Hkv, G, causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    B, N, Nk, d = 2, 200, 333, 64
    H = Hkv * G
    q, _, _ = random_qkv(7300 + G, B, H, N, d)
    _, k, v = random_qkv(7301 + Hkv, B, Hkv, Nk, d)
    g = normal_bits(7302 + H, B * H * N * d).reshape(B, H, N, d)
    scale = fp32_scale(d)
    tq, tk, tv, tg = (to_device(a) for a in (q, k, v, g))
    # [B, H, N, d] queries as [B*Hkv, G, N, d]; keys [B, Hkv, Nk, d] as [B*Hkv, G (stride 0), Nk, d]
    q5, g5 = tq.view(B * Hkv, G, N, d), tg.view(B * Hkv, G, N, d)
    k5 = tk.view(B * Hkv, 1, Nk, d).expand(B * Hkv, G, Nk, d)
    v5 = tv.view(B * Hkv, 1, Nk, d).expand(B * Hkv, G, Nk, d)
    assert k5.stride(1) == 0
    out, lse = fa.fa_fwd_ex(q5, k5, v5, scale=scale, causal=causal)
    dq, dk_h, dv_h = fa.fa_bwd_ex(q5, k5, v5, out, lse, g5, scale=scale, causal=causal,
                                  dk=torch.empty((B * Hkv, G, Nk, d), dtype=tq.dtype, device=tq.device),
                                  dv=torch.empty((B * Hkv, G, Nk, d), dtype=tq.dtype, device=tq.device))
    dk = dk_h.float().sum(dim=1).view(B, Hkv, Nk, d)     # the group's sum (fp32, outside the kernels)
    dv = dv_h.float().sum(dim=1).view(B, Hkv, Nk, d)
    torch.cuda.synchronize()
    k_rep, v_rep = (np.repeat(a, G, axis=1) for a in (k, v))  # key head h // G for query head h
    o_ref, l_ref = oracle.attention_rows(q, k_rep, v_rep, scale, causal)
    compare(bits_of(out.view(B, H, N, d)), lse.view(B, H, N).cpu().numpy(), o_ref, l_ref,
            label="gqa Hkv%d G%d c%d" % (Hkv, G, causal))
    rq, rk, rv = oracle.attention_bwd(q, k_rep, v_rep, g, scale, causal)
    compare_grad(bits_of(dq.view(B, H, N, d)), rq, label="gqa dq")
    for name, got, r in (("dk", dk, rk), ("dv", dv, rv)):
        ref = r.reshape(B, Hkv, G, Nk, d).sum(axis=2)
        err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
        # a sum of G bf16-rounded per-head gradients: at most G times the per-head
        # bound in the worst case, sqrt(G) times in rms (independent roundings)
        assert err.max() <= G * 1e-2 * np.abs(r).max(), (name, err.max(), np.abs(r).max())
        assert np.sqrt(np.mean(err ** 2)) <= np.sqrt(G) * 4e-3 * np.sqrt(np.mean(r ** 2)), name
