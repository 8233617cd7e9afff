"""The tile fa_fwd picks on its own (fa_launch_cfg): 8-wavefront tiles when the
grid fills the GPU; when it would not, at d = 32, 64 and 128 the key-split tile
(four wavefronts sharing each 32-query block) if causal or if 4-wavefront tiles
too would leave compute units idle, else 4-wavefront tiles; on non-causal grids
that fill the GPU, the 8-, 12- or 4-wavefront tile that leaves the busiest
compute unit the least work; and the default launch is bit-identical to the
explicit launch of the configuration it names."""
import numpy as np
import pytest

from inputs import random_qkv
from parity import fp32_scale, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_fa2_amd as fa
    fa.load_library()
    return torch.device("cuda:0")


def test_choice_follows_the_grid():
    import torch
    import flashattention_forward_fa2_amd as fa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ks = (1, 4, 32, 4)
    assert fa.launch_cfg(4, 8, 4096, 64, False) == (1, 8, 64)          # 512 workgroups of 256 queries
    assert fa.launch_cfg(1, 8, 4096, 64, False) == (1, 4, 64)          # 128 of them; 256 of 128 queries
    assert fa.launch_cfg(1, 8, 4096, 64, True) == ks                   # causal: key split below the CU count
    assert fa.launch_cfg(1, 8, 4096, 128, True) == ks
    assert fa.launch_cfg(1, 8, 1024, 64, True) == ks                   # 32, then 64: fewer than the CUs
    assert fa.launch_cfg(1, 8, 1024, 64, False, "f16") == ks
    assert fa.launch_cfg(1, 1, 256, 64, False) == ks
    assert fa.launch_cfg(1, 8, 1024, 128, False, "f16") == ks
    assert fa.launch_cfg(1, 8, 1024, 32, False) == ks
    assert fa.launch_cfg(1, 8, 4096, 32, False) == (1, 4, 64)          # the 4-wave grid fills the CUs
    assert fa.launch_cfg(1, 8, 1024, 256, False) == (1, 4, 32)         # d = 256 has the 4-wave tile only
    assert fa.launch_cfg(1, 8, 1024, 64, False, "f32") == (1, 4, 32)
    n = 256 * ((cus + 7) // 8)                                         # 8 heads x n/256 tiles >= cus
    assert fa.launch_cfg(1, 8, n, 64, False) == (1, 8, 64)
    assert fa.launch_cfg(1, 8, n, 64, True) == (1, 8, 64)
    assert fa.launch_cfg(1, 8, n - 256, 64, False) == (1, 4, 64)      # 8 * (ceil(cus / 8) - 1) < cus
    assert fa.launch_cfg(1, 8, n - 256, 64, True) == ks
    m = 128 * ((cus + 7) // 8)                                         # 4-wave grid just fills the CUs
    assert fa.launch_cfg(1, 8, m, 64, False) == (1, 4, 64)
    assert fa.launch_cfg(1, 8, m - 128, 64, False) == ks


def balanced(B, H, N, waves, permille, cus):
    n = B * H * -(-N // (32 * waves))
    return -(-n // cus) * waves * permille


@pytest.mark.parametrize("B,H,N,d", [(4, 8, 4096, 64), (4, 8, 3072, 64), (4, 8, 6144, 64), (4, 12, 2048, 64),
                                     (2, 16, 5000, 64), (1, 64, 3000, 64), (4, 32, 8192, 128),
                                     (4, 8, 3072, 128), (2, 16, 5000, 128), (4, 16, 4096, 128),
                                     (4, 8, 4096, 32), (4, 8, 3072, 32), (2, 16, 5000, 32), (4, 8, 6144, 32)])
def test_non_causal_tile_balances_the_compute_units(B, H, N, d):
    import torch
    import flashattention_forward_fa2_amd as fa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if B * H * -(-N // 256) < cus:
        pytest.skip("grid smaller than the device: the small-grid rule applies")
    opts = [((1, 8, 64), 1000), ((1, 12, 64), 975), ((1, 4, 64), {32: 1025, 64: 1030, 128: 1050}[d])]
    if d != 64:
        opts.pop(1)
    want = min(opts, key=lambda o: (balanced(B, H, N, o[0][1], o[1], cus), o[0] != (1, 8, 64)))[0]
    for dt in ("bf16", "f16"):
        assert fa.launch_cfg(B, H, N, d, False, dt) == want
    assert fa.launch_cfg(B, H, N, d, True) in ((1, 8, 64),)                 # causal keeps the 8-wave tile
    if cus == 256:                                                         # the measured choices on MI355X
        assert dict([((4, 8, 4096, 64), (1, 8, 64)), ((4, 8, 3072, 64), (1, 12, 64)),
                     ((4, 8, 6144, 64), (1, 12, 64)), ((4, 12, 2048, 64), (1, 4, 64)),
                     ((2, 16, 5000, 64), (1, 4, 64)), ((1, 64, 3000, 64), (1, 12, 64)),
                     ((4, 32, 8192, 128), (1, 8, 64)), ((4, 8, 3072, 128), (1, 4, 64)),
                     ((2, 16, 5000, 128), (1, 4, 64)), ((4, 16, 4096, 128), (1, 8, 64)),
                     ((4, 8, 4096, 32), (1, 8, 64)), ((4, 8, 3072, 32), (1, 4, 64)),
                     ((2, 16, 5000, 32), (1, 4, 64)), ((4, 8, 6144, 32), (1, 8, 64))])[(B, H, N, d)] == want


@pytest.mark.parametrize("N,causal", [(1024, True), (1024, False), (4096, False), (300, True), (3072, False)])
def test_default_launch_equals_the_named_configuration(N, causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H = (4, 8) if N == 3072 else (1, 8)
    d = 128 if N == 300 else 64
    q, k, v = (to_device(a) for a in random_qkv(7700 + N, B, H, N, d))
    scale = fp32_scale(d)
    o1, l1 = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    cfg = fa.launch_cfg(B, H, N, d, causal)
    o2, l2 = fa.fa_fwd(q, k, v, scale=scale, causal=causal, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
