"""GPU parity of the general-layout entry point (fa_fwd_ex, through the C ABI)
against the fp64 CPU oracle: Nq queries over Nk keys with the top-left causal
mask, [B, N, H, d] strides, q/k/v as views of one packed tensor, outputs written
into strided views with untouched padding, and bit-identity with fa_fwd on the
square contiguous case."""
import numpy as np
import pytest

import oracle
from inputs import bf16_bits_to_f64, random_qkv
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


def qkv_nonsquare(seed, B, H, Nq, Nk, d, sigma_qk=1.0):
    q, _, _ = random_qkv(seed, B, H, Nq, d, sigma_qk=sigma_qk)
    _, k, v = random_qkv(seed + 1, B, H, Nk, d, sigma_qk=sigma_qk)
    return q, k, v


def run_ex(q, k, v, scale, causal, out=None, lse=None):
    import torch
    import flashattention_forward_fa2_amd as fa
    out, lse = fa.fa_fwd_ex(q, k, v, scale=scale, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Nq,Nk", [(1, 4096), (7, 300), (100, 333), (333, 100), (640, 64), (257, 1000),
                                   (1000, 1), (512, 512)])
def test_nonsquare_lengths(Nq, Nk, d, causal):
    q, k, v = qkv_nonsquare(5000 + Nq + Nk, 1, 2, Nq, Nk, d)
    scale = fp32_scale(d)
    out, lse = run_ex(to_device(q), to_device(k), to_device(v), scale, causal)
    o_ref, l_ref = oracle.attention_rows(q, k, v, scale, causal)
    compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref,
            label="Nq=%d Nk=%d d=%d causal=%d" % (Nq, Nk, d, causal))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_bnhd_layout_and_strided_outputs(d, causal):
    """q, k, v, out stored [B, N, H, d]; lse a padded [B, H, Nq] view."""
    import torch
    B, H, N = 2, 3, 300
    q, k, v = random_qkv(6100 + d + causal, B, H, N, d)
    tq, tk, tv = (to_device(a).permute(0, 2, 1, 3).contiguous() for a in (q, k, v))  # [B, N, H, d]
    out_store = torch.full((B, N, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_store = torch.full((B, H, N + 5), -3.0, dtype=torch.float32, device="cuda")
    out, lse = run_ex(tq.transpose(1, 2), tk.transpose(1, 2), tv.transpose(1, 2), fp32_scale(d), causal,
                      out=out_store.transpose(1, 2), lse=lse_store[:, :, :N])
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), causal)
    compare(bits_of(out), lse.contiguous().cpu().numpy(), o_ref, l_ref,
            label="bnhd d=%d causal=%d" % (d, causal))
    assert torch.all(lse_store[:, :, N:] == -3.0)


def test_packed_qkv_views():
    """q, k, v as three interleaved views of one [B, N, 3, H, d] tensor."""
    import torch
    B, H, N, d = 2, 4, 200, 64
    q, k, v = random_qkv(6200, B, H, N, d)
    packed = torch.empty((B, N, 3, H, d), dtype=torch.bfloat16, device="cuda")
    for i, a in enumerate((q, k, v)):
        packed[:, :, i] = to_device(a).permute(0, 2, 1, 3)
    out, lse = run_ex(packed[:, :, 0].transpose(1, 2), packed[:, :, 1].transpose(1, 2),
                      packed[:, :, 2].transpose(1, 2), fp32_scale(d), True)
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), True)
    compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref, label="packed qkv")


def test_padding_between_output_rows_is_untouched():
    """out with a row stride of d + 64 elements: the 64 padding elements of every
    row keep their sentinel."""
    import torch
    B, H, N, d = 1, 2, 260, 128
    q, k, v = random_qkv(6300, B, H, N, d)
    store = torch.full((B, H, N, d + 64), 5.0, dtype=torch.bfloat16, device="cuda")
    out, lse = run_ex(to_device(q), to_device(k), to_device(v), fp32_scale(d), False, out=store[..., :d])
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), False)
    compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref, label="padded out rows")
    assert torch.all(store[..., d:] == 5.0)


@pytest.mark.parametrize("causal", [0, 1])
def test_ex_is_bit_identical_to_fa_fwd(causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v = random_qkv(6400 + causal, 2, 2, 777, 64)
    tq, tk, tv = (to_device(a) for a in (q, k, v))
    o1, l1 = fa.fa_fwd(tq, tk, tv, causal=bool(causal))
    o2, l2 = fa.fa_fwd_ex(tq, tk, tv, causal=bool(causal))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_single_query_over_long_keys_equals_last_row():
    """One query (the decode shape) over N keys, causal top-left, sees only key 0;
    non-causal it matches row 0 of the square problem with that query."""
    import torch
    B, H, N, d = 1, 4, 2048, 128
    q, k, v = random_qkv(6500, B, H, N, d)
    q1 = np.ascontiguousarray(q[:, :, :1])
    tq, tk, tv = to_device(q1), to_device(k), to_device(v)
    out_c, _ = run_ex(tq, tk, tv, fp32_scale(d), True)
    vf = bf16_bits_to_f64(v)[:, :, 0]
    assert np.array_equal(bf16_bits_to_f64(bits_of(out_c))[:, :, 0], vf)
    out_n, lse_n = run_ex(tq, tk, tv, fp32_scale(d), False)
    o_ref, l_ref = oracle.attention_rows(q1, k, v, fp32_scale(d), False)
    compare(bits_of(out_n), lse_n.cpu().numpy(), o_ref, l_ref, label="decode Nq=1")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,tile", [(3072, (1, 12, 64)), (4096, (1, 8, 32))])
def test_bnhd_on_the_default_non_causal_tiles(N, tile, dtype):
    """[B, N, H, d] views at non-causal shapes whose default tiles on a 256-CU
    device are the 12-wavefront one (B4 H8 N3072 d64: 256 workgroups of 384
    queries) and the 32-key 8-wavefront one (B4 H8 N4096 d64: 512 workgroups of
    256 queries, two per CU), so the strided instantiations of those tiles run;
    sampled rows (every query tile's edges and the last row) against the oracle,
    and bit-identity with the contiguous launch of the same tile."""
    import torch
    import flashattention_forward_fa2_amd as fa
    from inputs import sample_rows
    B, H, d = 4, 8, 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cfg = fa.launch_cfg(B, H, N, d, False, dtype)
    if cus == 256:
        assert cfg == tile
    q, k, v = random_qkv(6600 + N, B, H, N, d, dtype=dtype)
    tq, tk, tv = (to_device(a, dtype=dtype).permute(0, 2, 1, 3).contiguous() for a in (q, k, v))  # [B, N, H, d]
    out, lse = run_ex(tq.transpose(1, 2), tk.transpose(1, 2), tv.transpose(1, 2), fp32_scale(d), False)
    rows = sample_rows(6600 + N, B, H, N, per_head=24)
    bq = 32 * cfg[0] * cfg[1]
    edges = sorted({i for t in range(0, N, bq) for i in (t, min(t + bq, N) - 1)})
    extra = np.array([bh * N + i for bh in range(B * H) for i in edges[:4] + edges[-2:]])
    rows = np.unique(np.concatenate([rows, extra]))
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), False, rows=rows, dtype=dtype)
    tol = dict(o_max=4e-3, o_mean=3e-4) if dtype == "f16" else {}
    compare(bits_of(out), lse.contiguous().cpu().numpy(), o_ref, l_ref, rows=rows, dtype=dtype,
            label="bnhd tile %s N=%d %s" % (cfg, N, dtype), **tol)
    o2, l2 = fa.fa_fwd_ex(to_device(q, dtype=dtype), to_device(k, dtype=dtype), to_device(v, dtype=dtype),
                          scale=fp32_scale(d), causal=False, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
