"""GPU parity of the other element types and head dims (fp16 inputs; d = 32 and
256; fp32 inputs on the fp32 kernel) against the fp64 CPU oracle, through
fa_fwd_ex (desc.dtype) and the split path; fa_fwd (bfloat16) at d = 32 and 256."""
import numpy as np
import pytest

import oracle
from inputs import random_qkv
from parity import compare, fp32_scale, to_device

pytestmark = pytest.mark.gpu

# fp16 keeps 11 significant bits against bfloat16's 8: its outputs, and the P
# operand of the P.V product, round 8x finer, so the same error budget shrinks
# accordingly (the pages put fp16 attention at about 1e-3 agreement).
F16_MAX, F16_MEAN = 4e-3, 3e-4


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


def qkv(seed, B, H, Nq, Nk, d, dtype, sigma=1.0):
    q, _, _ = random_qkv(seed, B, H, Nq, d, sigma_qk=sigma, dtype=dtype)
    _, k, v = random_qkv(seed + 1, B, H, Nk, d, sigma_qk=sigma, dtype=dtype)
    return q, k, v


def check(q, k, v, causal, dtype, label, run):
    import torch
    d = q.shape[-1]
    out, lse = run(*(to_device(a, dtype=dtype) for a in (q, k, v)))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), causal, dtype=dtype)
    tol = dict(o_max=F16_MAX, o_mean=F16_MEAN) if dtype == "f16" else {}
    return compare(bits_of(out), lse.contiguous().cpu().numpy(), o_ref, l_ref, label=label, dtype=dtype, **tol)


# bf16 at d = 64 and 128 has suites of its own.
@pytest.mark.parametrize("dtype,d", [("f16", 32), ("f16", 64), ("f16", 128), ("f16", 256), ("bf16", 32), ("bf16", 256)])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Nq,Nk", [(300, 300), (1, 777), (200, 77)])
def test_dtype_and_head_dim(dtype, d, causal, Nq, Nk):
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(8000 + d + Nq + causal, 2, 2, Nq, Nk, d, dtype)
    run = lambda a, b, c: fa.fa_fwd_ex(a, b, c, scale=fp32_scale(d), causal=bool(causal))
    check(q, k, v, causal, dtype, "%s d=%d c=%d Nq=%d Nk=%d" % (dtype, d, causal, Nq, Nk), run)


def f16_variants():
    import flashattention_forward_fa2_amd as fa
    try:
        return fa.variants("f16")
    except Exception:
        return []


@pytest.mark.parametrize("variant", f16_variants(), ids=lambda v: "d%d-c%d-%s" % (v[0], v[1], "-".join(map(str, v[2]))))
def test_every_compiled_f16_variant(variant):
    """Each fp16 tile configuration, named explicitly, on a head of several ragged tiles."""
    import flashattention_forward_fa2_amd as fa
    d, causal, cfg = variant
    q, k, v = qkv(8300 + d + causal, 2, 3, 600, 600, d, "f16", sigma=2.0)
    run = lambda a, b, c: fa.fa_fwd_ex(a, b, c, scale=fp32_scale(d), causal=bool(causal), cfg=cfg)
    check(q, k, v, causal, "f16", "f16 variant d=%d c=%d %s" % (d, causal, cfg), run)


@pytest.mark.parametrize("d", [32, 256])
@pytest.mark.parametrize("causal", [0, 1])
def test_fa_fwd_bf16_new_head_dims(d, causal):
    """The square contiguous entry point at d = 32 and 256, a head of several tiles."""
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(8100 + d + causal, 1, 4, 1000, 1000, d, "bf16")
    run = lambda a, b, c: fa.fa_fwd(a, b, c, scale=fp32_scale(d), causal=bool(causal))
    check(q, k, v, causal, "bf16", "fa_fwd bf16 d=%d c=%d" % (d, causal), run)


@pytest.mark.parametrize("dtype,d", [("f16", 64), ("f16", 128), ("f16", 256), ("bf16", 32)])
def test_strided_and_split_paths(dtype, d):
    """[B, N, H, d] views, then the split-key path with a short query range."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, N = 2, 3, 500
    q, k, v = qkv(8200 + d, B, H, N, N, d, dtype)
    def strided(a, b, c):
        a, b, c = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (a, b, c))
        return fa.fa_fwd_ex(a, b, c, scale=fp32_scale(d), causal=True)
    check(q, k, v, 1, dtype, "strided %s d=%d" % (dtype, d), strided)
    qs = np.ascontiguousarray(q[:, :, :40])
    split = lambda a, b, c: fa.fa_fwd_splitkv(a, b, c, scale=fp32_scale(d), causal=False, num_splits=4)
    check(qs, k, v, 0, dtype, "split %s d=%d" % (dtype, d), split)


def test_f16_peaked_scores_and_large_values():
    """fp16 inputs with scaled scores of sigma 16 and values near the top of the
    fp16 range: scores and statistics stay fp32, the output stays finite."""
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(8300, 1, 2, 600, 600, 128, "f16", sigma=4.0)
    vbig = (v.view(np.float16).astype(np.float64) * 4000.0).astype(np.float16).view(np.uint16)  # |v| up to ~2e4
    run = lambda a, b, c: fa.fa_fwd_ex(a, b, c, scale=fp32_scale(128), causal=False)
    import torch
    out, lse = run(*(to_device(a, dtype="f16") for a in (q, k, vbig)))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_rows(q, k, vbig, fp32_scale(128), False, dtype="f16")
    o = bits_of(out).view(np.float16).astype(np.float64).reshape(-1, 128)
    assert np.all(np.isfinite(o))
    rel = np.abs(o - o_ref).max() / np.abs(o_ref).max()
    assert rel <= F16_MAX, rel


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_d256_longer_head(dtype):
    """d = 256 over several 128-query and 32-key tiles, causal."""
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(8400, 1, 2, 2048, 2048, 256, dtype)
    run = lambda a, b, c: fa.fa_fwd_ex(a, b, c, scale=fp32_scale(256), causal=True)
    check(q, k, v, 1, dtype, "%s d=256 N=2048 causal" % dtype, run)


# ---------------------------------------------------------------- fp32 inputs
# fp32 products and sums: scores carry about sqrt(d) * 2^-24 * |s| of error,
# O about sqrt(N) * 2^-24 * |O| more, and v_exp_f32 about 1 ulp: below 1e-5 for
# these inputs.  Bars: max |dO| <= 1e-4, mean <= 1e-5, LSE 1e-5 relative.
F32_MAX, F32_MEAN, F32_LSE = 1e-4, 1e-5, 1e-5


def f32_device(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def check_f32(q, k, v, causal, label, run):
    import torch
    d = q.shape[-1]
    out, lse = run(f32_device(q), f32_device(k), f32_device(v))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_rows_f32(q, k, v, fp32_scale(d), causal)
    o = out.contiguous().cpu().numpy().astype(np.float64).reshape(-1, d)
    L = lse.contiguous().cpu().numpy().astype(np.float64).reshape(-1)
    err = np.abs(o - o_ref)
    lerr = (np.abs(L - l_ref) / np.maximum(1.0, np.abs(l_ref))).max()
    import sys
    print("[parity] %s max|dO|=%.3e mean|dO|=%.3e lse=%.3e" % (label, err.max(), err.mean(), lerr),
          file=sys.stderr, flush=True)
    assert np.all(np.isfinite(o))
    assert err.max() <= F32_MAX and err.mean() <= F32_MEAN and lerr <= F32_LSE, (err.max(), err.mean(), lerr)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("Nq,Nk", [(300, 300), (1, 777), (200, 77), (1000, 1000)])
def test_f32_inputs(d, causal, Nq, Nk):
    import flashattention_forward_fa2_amd as fa
    q, k, v = qkv(8500 + d + Nq + causal, 2, 2, Nq, Nk, d, "f32")
    run = lambda a, b, c: fa.fa_fwd_ex(a, b, c, scale=fp32_scale(d), causal=bool(causal))
    check_f32(q, k, v, causal, "f32 d=%d c=%d Nq=%d Nk=%d" % (d, causal, Nq, Nk), run)


def test_f32_strided_views_and_peaked_scores():
    """[B, N, H, d] fp32 views with scaled scores of sigma 16."""
    import flashattention_forward_fa2_amd as fa
    d = 128
    q, k, v = qkv(8600, 2, 3, 400, 400, d, "f32", sigma=4.0)
    def run(a, b, c):
        a, b, c = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (a, b, c))
        return fa.fa_fwd_ex(a, b, c, scale=fp32_scale(d), causal=True)
    check_f32(q, k, v, 1, "f32 strided peaked", run)


def test_f32_long_head_sampled_rows():
    """B1-H4-N4096 d128 causal in fp32, every row of two heads."""
    import torch
    import flashattention_forward_fa2_amd as fa
    d = 128
    q, k, v = qkv(8700, 1, 4, 4096, 4096, d, "f32")
    out, lse = fa.fa_fwd_ex(f32_device(q), f32_device(k), f32_device(v), scale=fp32_scale(d), causal=True)
    torch.cuda.synchronize()
    rows = np.arange(2 * 4096, dtype=np.int64)
    o_ref, l_ref = oracle.attention_rows_f32(q, k, v, fp32_scale(d), True, rows)
    o = out.cpu().numpy().astype(np.float64).reshape(-1, d)[rows]
    assert np.abs(o - o_ref).max() <= F32_MAX
    assert (np.abs(lse.cpu().numpy().reshape(-1)[rows] - l_ref) / np.maximum(1, np.abs(l_ref))).max() <= F32_LSE
