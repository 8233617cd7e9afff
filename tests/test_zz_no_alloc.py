"""fa_fwd_splitkv_noalloc (partial results in the library's static per-GPU
scratch) against fa_fwd_splitkv with a caller workspace, through the C ABI: two
calls in a row, the second smaller, each bit-identical to the workspace path
and within the oracle tolerances; a request beyond the scratch is refused."""
import ctypes

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


def run_both(B, H, Nq, Nk, d, causal, S, seed):
    """One call through each entry point on the same inputs; returns their
    outputs, the inputs' bits and the workspace size the shape needs."""
    import torch
    import flashattention_forward_fa2_amd as fa
    q, _, _ = random_qkv(seed, B, H, Nq, d)
    _, k, v = random_qkv(seed + 1, B, H, Nk, d)
    tq, tk, tv = to_device(q), to_device(k), to_device(v)
    scale = fp32_scale(d)
    lib = fa.load_library()
    stream = torch.cuda.current_stream()
    outs = []
    for noalloc in (True, False):
        out = torch.full_like(tq, float("nan"))
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
        desc, out, lse = fa._make_desc(tq, tk, tv, scale, causal, out, lse, stream)
        if noalloc:
            st = lib.fa_fwd_splitkv_noalloc(ctypes.byref(desc), S)
        else:
            need = fa.splitkv_workspace_bytes(B, H, Nq, Nk, d, S)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            st = lib.fa_fwd_splitkv(ctypes.byref(desc), S, ctypes.c_void_p(ws.data_ptr()), ctypes.c_longlong(need))
        assert st == 0, fa.strerror(st)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs, (q, k, v), fa.splitkv_workspace_bytes(B, H, Nq, Nk, d, S)


@pytest.mark.parametrize("causal", [0, 1])
def test_noalloc_matches_workspace_path_twice(causal):
    """A large call, then a smaller one: the second reads the scratch the first
    left behind and must still equal the workspace path bit for bit."""
    import torch
    import flashattention_forward_fa2_amd as fa
    for i, (B, H, Nq, Nk, d, S) in enumerate([(2, 8, 64, 3000, 128, 12), (1, 3, 7, 500, 64, 4)]):
        (a, b), (q, k, v), need = run_both(B, H, Nq, Nk, d, causal, S, 7300 + 10 * i + causal)
        assert 0 < need <= fa.SPLITKV_NOALLOC_MAX_BYTES
        assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), "out differs (call %d)" % i
        assert torch.equal(a[1], b[1]), "lse differs (call %d)" % i
        o_ref, l_ref = oracle.attention_rows(q, k, v, fp32_scale(d), bool(causal))
        compare(bits_of(a[0]), a[1].cpu().numpy(), o_ref, l_ref,
                label="noalloc B%d H%d Nq=%d Nk=%d d=%d c=%d S=%d" % (B, H, Nq, Nk, d, causal, S))


def test_noalloc_refuses_more_than_the_scratch():
    """A split count whose partial results exceed the scratch returns
    FA_ERR_SCRATCH and leaves the outputs untouched."""
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H, Nq, Nk, d, S = 4, 32, 512, 8192, 128, 8
    assert fa.splitkv_workspace_bytes(B, H, Nq, Nk, d, S) > fa.SPLITKV_NOALLOC_MAX_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device="cuda")
    desc, out, lse = fa._make_desc(q, k, k, None, False, out, lse, torch.cuda.current_stream())
    assert fa.load_library().fa_fwd_splitkv_noalloc(ctypes.byref(desc), S) == 13  # FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
