"""The tile fa_fwd picks on its own (fa_launch_cfg), at d = 32, 64 and 128.
Non-causal: the key-split tile (four wavefronts sharing each 32-query block)
while twice the 4-wavefront grid fits the compute units, the 4-wavefront tile
while that grid does (at d = 32 while the 8-wavefront grid does), and beyond
the 8-, 12- or 4-wavefront tile or the 32-key 8-wavefront tile, whichever leaves
the busiest compute unit the least work.  Causal: the key split on grids of
fewer 8-wavefront workgroups than compute units (at d = 128 only while the
4-wavefront grid is smaller, or just fills them with rows of 2048 or more; at
d = 32 up to 1.5 times the compute units); beyond, the 4-wavefront tile where the
8-wavefront tile's launch order loads the compute units unevenly (unless its own
is worse), and where both are even the 8-wavefront tile, except from four layers
on at d = 64 (and at d = 32 for rows up to 4096).  The rule is checked
against a Python restatement of it (its own replay of the causal launch order)
and against the choices tile sweeps measured on MI355X; the default launch is
bit-identical to the explicit launch of the configuration it names."""
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


def test_choice_follows_the_grid():
    import torch
    import flashattention_forward_fa2_amd as fa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ks = (1, 4, 32, 4)
    assert fa.launch_cfg(4, 8, 4096, 64, False) == (1, 8, 32)          # 512 workgroups of 256 queries, two per CU
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
    assert fa.launch_cfg(1, 8, 4 * n, 64, True) == (1, 4, 64)          # four layers: three 4-wave tiles per CU
    assert fa.launch_cfg(1, 8, 4 * n, 128, True) == (1, 8, 64)         # ... at d = 128 two, as many as 8-wave ones
    assert fa.launch_cfg(1, 8, n - 256, 64, False) == (1, 8, 64)      # 8-wave grid < cus < 4-wave grid
    assert fa.launch_cfg(1, 8, n - 256, 64, True) == ks
    m = 128 * ((cus + 7) // 8)                                         # 4-wave grid just fills the CUs
    assert fa.launch_cfg(1, 8, m, 64, False) == (1, 4, 64)
    assert fa.launch_cfg(1, 8, m // 2, 64, False) == ks                # ... or fills half of them
    if cus == 256:
        assert fa.launch_cfg(1, 8, n, 64, True) == (1, 4, 64)          # one layer: the longest tile sets the time
        assert fa.launch_cfg(1, 8, m - 128, 64, False) == (1, 4, 64)
        assert fa.launch_cfg(4, 8, 2048, 32, False) == (1, 4, 64)      # d = 32: one layer of 8-wave tiles
        assert fa.launch_cfg(4, 8, 512, 128, False) == (1, 4, 64)      # d = 128: two key-split layers of short rows
        assert fa.launch_cfg(1, 8, 2048, 128, False) == ks             # ... of long rows
        assert fa.launch_cfg(4, 8, 2048, 64, False) == (1, 8, 64)


# ---- a restatement of the causal rule ---------------------------------------
FA_CAUSAL_GROUP = 2


def causal_order(i, total, BH, nqt, res, cus):
    """(head, query tile) of causal workgroup i: heads grouped per XCD, longest
    tile first within groups of two heads, odd co-resident layers reversed."""
    if BH % 8 == 0:
        t = (i & 7) * (total >> 3) + (i >> 3)
        per, hpx = total >> 3, BH >> 3
        chunk, j = divmod(t, per)
        cpx = cus >> 3
        if res > 1 and cpx > 0 and cus % 8 == 0:
            l, p = divmod(j, cpx)
            if l % 2 == 1 and l < res and (l + 1) * cpx <= per:
                j = l * cpx + (cpx - 1 - p)
        gs = FA_CAUSAL_GROUP if hpx % FA_CAUSAL_GROUP == 0 else hpx
        grp, r = divmod(j, gs * nqt)
        return chunk * hpx + grp * gs + r % gs, nqt - 1 - r // gs
    u = i
    if res > 1 and cus > 0:
        l, p = divmod(u, cus)
        if l % 2 == 1 and l < res and (l + 1) * cus <= total:
            u = l * cus + (cus - 1 - p)
    return u % BH, nqt - 1 - u // BH


def causal_balance(BH, N, rows, res, cus):
    """Mean over largest per-CU count of visited 64-key tiles, per XCD: the first
    res layers round-robin, then each workgroup on the least loaded CU."""
    nqt = -(-N // rows)
    total = BH * nqt
    cpx = max(1, cus // 8)
    worst = 1.0
    for x in ([0] if BH % 8 == 0 and cus % 8 == 0 else range(8)):
        work = [0] * cpx
        for k, i in enumerate(range(x, total, 8)):
            _, qt = causal_order(i, total, BH, nqt, res, cus)
            c = k % cpx if k < cpx * res else work.index(min(work))
            work[c] += -(-min(qt * rows + rows, N) // 64)
        if max(work) > 0:
            worst = min(worst, sum(work) / cpx / max(work))
    return worst


# Workgroups per CU of the causal 8- and 4-wavefront kernels (register and LDS
# limits of the gfx950 build): d = 32 two and four, d = 64 one and three,
# d = 128 one and two.
RESIDENT = {32: (2, 4), 64: (1, 3), 128: (1, 2)}


def causal_rule(B, H, N, d, cus):
    w8, w4 = B * H * -(-N // 256), B * H * -(-N // 128)
    if (d <= 64 or w4 < cus or (w4 == cus and N >= 2048)) if w8 < cus else (d == 32 and 2 * w8 <= 3 * cus):
        return (1, 4, 32, 4)
    r8, r4 = RESIDENT[d]
    replay = w8 <= 16 * cus
    b8 = 0.0 if w8 < cus else causal_balance(B * H, N, 256, r8, cus) if replay else 1.0
    b4 = causal_balance(B * H, N, 128, r4, cus) if replay else 1.0
    if b4 < b8:
        return (1, 8, 64)
    if b8 < 0.97:
        return (1, 4, 64)
    long_grid = w8 >= 4 * cus
    return (1, 4, 64) if long_grid and (d == 64 or (d == 32 and N <= 4096)) else (1, 8, 64)


CAUSAL_SHAPES = [(4, 8, 2048), (2, 8, 4096), (1, 16, 4096), (1, 8, 8192), (3, 8, 4096), (4, 8, 3072), (4, 8, 4096),
                 (2, 8, 8192), (8, 8, 2048), (5, 8, 4096), (6, 8, 4096), (4, 16, 4096), (8, 8, 1024), (16, 8, 512),
                 (1, 32, 2048), (1, 24, 2048), (6, 8, 1024), (2, 12, 3000), (3, 5, 4096), (1, 32, 32768)]


@pytest.mark.parametrize("d", [32, 64, 128])
def test_causal_rule_matches_its_statement(d):
    import torch
    import flashattention_forward_fa2_amd as fa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("the occupancy table above is MI355X's")
    for B, H, N in CAUSAL_SHAPES:
        want = causal_rule(B, H, N, d, cus)
        for dt in ("bf16", "f16"):
            assert fa.launch_cfg(B, H, N, d, True, dt) == want, (B, H, N, d, dt)


def test_causal_choices_measured_on_mi355x():
    """Where the tile sweeps put each causal shape (HIP events, best of the 8- and
    4-wavefront tiles and the key split): the 8-wavefront tile only where its
    order pairs long tiles with short ones on every CU."""
    import torch
    import flashattention_forward_fa2_amd as fa
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("measured on a 256-CU MI355X")
    best = {(4, 8, 2048, 64): (1, 4, 64), (2, 8, 4096, 64): (1, 4, 64), (1, 8, 8192, 64): (1, 4, 64),
            (3, 8, 4096, 64): (1, 4, 64), (4, 8, 3072, 64): (1, 8, 64), (4, 8, 4096, 64): (1, 8, 64),
            (2, 8, 8192, 64): (1, 8, 64), (8, 8, 2048, 64): (1, 4, 64), (5, 8, 4096, 64): (1, 4, 64),
            (6, 8, 4096, 64): (1, 4, 64), (16, 8, 512, 64): (1, 4, 64), (6, 8, 1024, 64): (1, 4, 32, 4),
            (4, 8, 2048, 128): (1, 4, 64), (4, 8, 4096, 128): (1, 8, 64), (2, 8, 8192, 128): (1, 8, 64),
            (8, 8, 1024, 128): (1, 4, 64), (1, 24, 2048, 128): (1, 4, 64), (1, 8, 4096, 128): (1, 4, 32, 4),
            (4, 8, 1024, 128): (1, 4, 64), (1, 4, 8192, 128): (1, 4, 32, 4), (4, 8, 512, 128): (1, 4, 32, 4),
            (1, 32, 32768, 128): (1, 8, 64), (4, 8, 2048, 32): (1, 4, 32, 4), (4, 8, 3072, 32): (1, 4, 32, 4),
            (2, 16, 3072, 32): (1, 4, 32, 4), (8, 8, 2048, 32): (1, 8, 64), (4, 8, 4096, 32): (1, 8, 64),
            (8, 16, 2048, 64): (1, 4, 64), (4, 32, 4096, 64): (1, 4, 64), (2, 16, 8192, 64): (1, 4, 64),
            (1, 32, 32768, 64): (1, 4, 64), (16, 16, 2048, 64): (1, 4, 64), (8, 16, 2048, 128): (1, 4, 64),
            (16, 16, 2048, 128): (1, 4, 64), (2, 16, 8192, 128): (1, 8, 64), (8, 8, 4096, 32): (1, 4, 64),
            (4, 16, 8192, 32): (1, 8, 64), (16, 16, 2048, 32): (1, 4, 64), (1, 32, 32768, 32): (1, 8, 64)}
    for (B, H, N, d), t in best.items():
        assert fa.launch_cfg(B, H, N, d, True) == t == causal_rule(B, H, N, d, cus), (B, H, N, d)


def test_rule_answers_do_not_depend_on_call_order():
    """The causal answers are remembered (eight per host thread): asking for more
    shapes than that, in one order, in reverse and again, with both element
    types interleaved, gives the same tiles every time."""
    import flashattention_forward_fa2_amd as fa
    shapes = [(B, H, N, d) for (B, H, N) in CAUSAL_SHAPES[:12] for d in (64, 128)]
    first = {(sh, dt): fa.launch_cfg(*sh, True, dt) for sh in shapes for dt in ("bf16", "f16")}
    for order in (shapes[::-1], shapes[::3] + shapes[1::3] + shapes[2::3]):
        for sh in order:
            for dt in ("f16", "bf16"):
                assert fa.launch_cfg(*sh, True, dt) == first[(sh, dt)], (sh, dt)
    assert all(first[(sh, "bf16")] == first[(sh, "f16")] for sh in shapes)


def balanced(B, H, N, waves, permille, cus):
    """Work of the busiest compute unit, weighed per mille; permille is a pair
    (the tile's weight once some CU gets two workgroups, and before)."""
    n = B * H * -(-N // (32 * waves))
    return -(-n // cus) * waves * permille[0 if n > cus else 1]


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
    p4 = {32: 1025, 64: 1030, 128: 1050}[d]
    opts = [((1, 8, 64), (1000, 1000)), ((1, 8, 32), (970, 1075)), ((1, 12, 64), (975, 975)), ((1, 4, 64), (p4, p4))]
    if d != 64:
        opts = [opts[0], opts[3]]
    want = min(opts, key=lambda o: (balanced(B, H, N, o[0][1], o[1], cus), o[0] != (1, 8, 64)))[0]
    for dt in ("bf16", "f16"):
        assert fa.launch_cfg(B, H, N, d, False, dt) == want
    if cus == 256:
        assert fa.launch_cfg(B, H, N, d, True) == causal_rule(B, H, N, d, cus)
    if cus == 256:                                                         # the measured choices on MI355X
        assert dict([((4, 8, 4096, 64), (1, 8, 32)), ((4, 8, 3072, 64), (1, 12, 64)),
                     ((4, 8, 6144, 64), (1, 8, 32)), ((4, 12, 2048, 64), (1, 4, 64)),
                     ((2, 16, 5000, 64), (1, 4, 64)), ((1, 64, 3000, 64), (1, 8, 32)),
                     ((4, 32, 8192, 128), (1, 8, 64)), ((4, 8, 3072, 128), (1, 4, 64)),
                     ((2, 16, 5000, 128), (1, 4, 64)), ((4, 16, 4096, 128), (1, 8, 64)),
                     ((4, 8, 4096, 32), (1, 8, 64)), ((4, 8, 3072, 32), (1, 4, 64)),
                     ((2, 16, 5000, 32), (1, 4, 64)), ((4, 8, 6144, 32), (1, 8, 64))])[(B, H, N, d)] == want


@pytest.mark.parametrize("N,causal", [(1024, True), (1024, False), (4096, False), (300, True), (3072, False),
                                      (2048, True)])
def test_default_launch_equals_the_named_configuration(N, causal):
    import torch
    import flashattention_forward_fa2_amd as fa
    B, H = (4, 8) if N in (3072, 2048) else (1, 8)
    d = 128 if N == 300 else 64
    qb, kb, vb = random_qkv(7700 + N, B, H, N, d)
    q, k, v = (to_device(a) for a in (qb, kb, vb))
    scale = fp32_scale(d)
    o1, l1 = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    cfg = fa.launch_cfg(B, H, N, d, causal)
    o2, l2 = fa.fa_fwd(q, k, v, scale=scale, causal=causal, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    # and the default launch against the oracle on every 13th row (and the last)
    rows = np.append(np.arange(0, B * H * N, 13), B * H * N - 1)
    o_ref, l_ref = oracle.attention_rows(qb, kb, vb, scale, causal, rows=rows)
    compare(o1.view(torch.int16).cpu().numpy().view(np.uint16), l1.cpu().numpy(), o_ref, l_ref, rows=rows,
            label="default launch N=%d causal=%d cfg=%s" % (N, causal, cfg))
