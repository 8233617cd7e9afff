"""A seeded sweep of random problems through the descriptor entry points:
lengths, head dims, element types, masks and memory layouts drawn together,
forward (every row) and, where d allows, backward (every gradient element)
against the oracle."""
import numpy as np
import pytest

import oracle
from inputs import normal_bits, random_qkv
from parity import compare, compare_grad, fp32_scale, to_device

pytestmark = pytest.mark.gpu

F16_MAX, F16_MEAN = 4e-3, 3e-4


@pytest.fixture(scope="module", autouse=True)
def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_fa2_amd as fa
    fa.load_library()
    return torch.device("cuda:0")


def draw(i):
    rng = np.random.default_rng(20000 + i)
    d = int(rng.choice([32, 64, 128, 256]))
    return dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), Nq=int(rng.integers(1, 700)),
                Nk=int(rng.integers(1, 700)), d=d, dtype=str(rng.choice(["bf16", "f16"])),
                causal=bool(rng.integers(0, 2)), layout=str(rng.choice(["bhnd", "bnhd", "padded"])), seed=20000 + i)


def place(bits, layout, dtype):
    """A [B, H, N, d] device view of `bits` stored in the given layout."""
    import torch
    B, H, N, d = bits.shape
    if layout == "bhnd":
        return to_device(bits, dtype=dtype)
    if layout == "bnhd":
        return to_device(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)), dtype=dtype).transpose(1, 2)
    # rows padded to d + 16 elements, garbage in the padding
    buf = np.full((B, H, N, d + 16), 0x7E00 if dtype == "f16" else 0x7FC0, dtype=np.uint16)
    buf[..., :d] = bits
    return to_device(buf, dtype=dtype)[..., :d]


def empty_like_layout(shape, layout, dtype_t, dev):
    import torch
    B, H, N, d = shape
    if layout == "bnhd":
        return torch.empty((B, N, H, d), dtype=dtype_t, device=dev).transpose(1, 2)
    if layout == "padded":
        return torch.empty((B, H, N, d + 16), dtype=dtype_t, device=dev)[..., :d]
    return torch.empty(shape, dtype=dtype_t, device=dev)


def bits_of(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("i", range(24))
def test_random_problem(i):
    import torch
    import flashattention_forward_fa2_amd as fa
    p = draw(i)
    B, H, Nq, Nk, d, dt, causal, layout = (p[k] for k in ("B", "H", "Nq", "Nk", "d", "dtype", "causal", "layout"))
    label = "random %d: B%d H%d Nq%d Nk%d d%d %s c%d %s" % (i, B, H, Nq, Nk, d, dt, causal, layout)
    print(label, flush=True)
    q, _, _ = random_qkv(p["seed"], B, H, Nq, d, dtype=dt)
    _, k, v = random_qkv(p["seed"] + 1, B, H, Nk, d, dtype=dt)
    scale = fp32_scale(d)
    tq, tk, tv = place(q, layout, dt), place(k, layout, dt), place(v, layout, dt)
    out = empty_like_layout((B, H, Nq, d), layout, tq.dtype, tq.device)
    out, lse = fa.fa_fwd_ex(tq, tk, tv, scale=scale, causal=causal, out=out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_rows(q, k, v, scale, causal, dtype=dt)
    tol = dict(o_max=F16_MAX, o_mean=F16_MEAN) if dt == "f16" else {}
    compare(bits_of(out), lse.cpu().numpy(), o_ref, l_ref, label=label, dtype=dt, **tol)
    if d not in (32, 64, 128):
        return
    g = normal_bits(p["seed"] + 3, B * H * Nq * d, dtype=dt).reshape(B, H, Nq, d)
    tg = place(g, layout, dt)
    grads = [empty_like_layout(s, layout, tq.dtype, tq.device) for s in ((B, H, Nq, d), (B, H, Nk, d), (B, H, Nk, d))]
    fa.fa_bwd_ex(tq, tk, tv, out, lse, tg, scale=scale, causal=causal, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(q, k, v, g, scale, causal, dtype=dt)
    for name, t, r in zip(("dq", "dk", "dv"), grads, ref):
        compare_grad(bits_of(t), r, label="%s %s" % (label, name), dtype=dt)
