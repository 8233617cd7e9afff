"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call.  CPU only (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import flashattention_forward_fa2_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("fa_fwd.h", "fa_bwd.h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB):
        fa.build()
    return fa.load_library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^(?:int|long long|const char \*)\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


def test_header_declares_what_the_binding_lists():
    assert declared_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_exported_symbols_have_c_linkage():
    out = os.popen("nm -D --defined-only %s" % fa.LIB).read()
    syms = set(re.findall(r"\bT (fa_\w+)$", out, re.M))
    assert set(declared_functions()) <= syms


def test_strerror_and_version(lib):
    assert fa.version() >= 100
    for code in range(13):
        assert fa.strerror(code)
    assert fa.strerror(99) == "unknown status"


def test_variant_table(lib):
    for dtype in ("bf16", "f16"):
        vs = fa.variants(dtype)
        for d in (32, 64, 128, 256):
            for causal in (0, 1):
                assert (d, causal, fa.default_cfg(4096, d, causal)) in vs, (dtype, d, causal)
    assert lib.fa_variant_dtype(-1) < 0 and lib.fa_variant_dtype(lib.fa_num_variants()) < 0
    assert len(fa.variants("bf16")) + len(fa.variants("f16")) + len(fa.variants("f32")) == lib.fa_num_variants()
    assert sorted(v[:2] for v in fa.variants("f32")) == [(64, 0), (64, 1), (128, 0), (128, 1)]


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: checks fail before any HIP call


def call(q=FAKE, k=2 * FAKE, v=3 * FAKE, out=4 * FAKE, lse=5 * FAKE, B=1, H=1, N=64, d=64, scale=0.125,
         causal=0, cfg=None):
    return fa.fa_fwd_ptr(q, k, v, out, lse, B, H, N, d, scale, causal, 0, cfg)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(out=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2),
    (dict(B=1 << 12, H=1 << 12, N=1 << 10), 2),
    (dict(N=1 << 24, d=128), 2),
    (dict(d=16), 3), (dict(d=96), 3), (dict(d=512), 3),
    (dict(scale=0.0), 4), (dict(scale=-0.1), 4), (dict(scale=float("inf")), 4), (dict(scale=float("nan")), 4),
    (dict(causal=2), 5), (dict(causal=-1), 5),
    (dict(q=FAKE + 8), 6), (dict(out=4 * FAKE + 4), 6), (dict(lse=5 * FAKE + 2), 6),
    (dict(out=FAKE), 7), (dict(out=FAKE + 16), 7), (dict(lse=3 * FAKE + 64), 7), (dict(lse=4 * FAKE + 1024), 7),
])
def test_argument_errors_return_codes(lib, kw, code):
    assert call(**kw) == code


def test_head_extent_limit_edge(lib):
    """(N + 256) * d must stay below 2^30 (one head's bytes within the 32-bit
    offsets of a buffer resource): the first N that reaches it is refused, the
    one below passes every host check (and stops at the device check on a host
    without a gfx950).  The tensors are 2 GiB apart, so they do not overlap."""
    d, far = 64, 1 << 32
    N = (1 << 30) // d - 256
    assert call(N=N, d=d, q=far, k=2 * far, v=3 * far, out=4 * far, lse=5 * far) == 2
    assert call(N=N - 1, d=d, q=far, k=2 * far, v=3 * far, out=4 * far, lse=5 * far) in (0, 8)


def test_inputs_may_alias_each_other(lib):
    # q = k = v is a legal self-attention call: it passes validation (and then
    # stops at the device check on a host without a gfx950).
    st = call(q=FAKE, k=FAKE, v=FAKE)
    assert st in (0, 8)


def test_unknown_tile_config_is_rejected(lib):
    assert call(cfg=(3, 4, 64)) == 5
    assert call(cfg=(1, 4, 48)) == 5


def test_no_device_on_cpu_host(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == 8


def test_no_undefined_kernel_launch_stubs():
    """Every kernel variant's host launch stub is defined in the library (a
    template body the host pass cannot instantiate leaves it undefined)."""
    out = os.popen("nm -D %s" % fa.LIB).read()
    assert not re.findall(r"\bU \S*device_stub\S*", out)


# ---------------------------------------------------------------- general-layout entry point

def test_desc_layout_matches_the_header(tmp_path):
    """The ctypes mirror of fa_fwd_desc has the C struct's size and offsets."""
    src = tmp_path / "sz.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"fa_fwd.h\"\n"
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(fa_fwd_desc),"
        " offsetof(fa_fwd_desc, B), offsetof(fa_fwd_desc, q_stride), offsetof(fa_fwd_desc, lse_stride),"
        " offsetof(fa_fwd_desc, scale), offsetof(fa_fwd_desc, stream), offsetof(fa_fwd_desc, dtype)); return 0;}\n")
    exe = tmp_path / "sz"
    assert os.system("gcc -I %s -o %s %s" % (os.path.join(ROOT, "include"), exe, src)) == 0
    got = [int(x) for x in os.popen(str(exe)).read().split()]
    D = fa.FwdDesc
    assert got == [ctypes.sizeof(D), D.B.offset, D.q_stride.offset, D.lse_stride.offset, D.scale.offset,
                   D.stream.offset, D.dtype.offset]


def test_tile_cfg_layout_matches_the_header(tmp_path):
    """The ctypes mirror of fa_tile_cfg (four ints since version 600) has the C
    struct's size and offsets."""
    src = tmp_path / "tc.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"fa_fwd.h\"\n"
        "int main(void){printf(\"%zu %zu %zu\\n\", sizeof(fa_tile_cfg), offsetof(fa_tile_cfg, bk),"
        " offsetof(fa_tile_cfg, ksplit)); return 0;}\n")
    exe = tmp_path / "tc"
    assert os.system("gcc -I %s -o %s %s" % (os.path.join(ROOT, "include"), exe, src)) == 0
    got = [int(x) for x in os.popen(str(exe)).read().split()]
    T = fa.TileCfg
    assert got == [ctypes.sizeof(T), T.bk.offset, T.ksplit.offset]
    assert fa.version() >= 600


def test_key_split_variants(lib):
    """The key-split tile (1, 4, 32, ksplit 4) is compiled at d = 32, 64 and 128
    for bf16 and fp16, both masks; other key-split shapes, and d = 256, are
    refused before any device call (FA_ERR_ARG), while a compiled one gets as far
    as the device check."""
    for dtype in ("bf16", "f16"):
        vs = fa.variants(dtype)
        for d in (32, 64, 128):
            for causal in (0, 1):
                assert (d, causal, (1, 4, 32, 4)) in vs
        assert not any(len(v[2]) == 4 for v in vs if v[0] == 256)
    assert not any(len(v[2]) == 4 for v in fa.variants("f32"))
    assert call(d=256, cfg=(1, 4, 32, 4)) == 5
    assert call(d=64, cfg=(1, 4, 32, 3)) == 5
    assert call(d=64, cfg=(1, 4, 64, 4)) == 5
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert call(d=64, cfg=(1, 4, 32, 4)) == 8
        assert call(d=32, cfg=(1, 4, 32, 4)) == 8
        assert call(d=128, causal=1, cfg=(1, 4, 32, 4)) == 8
    assert call(d=64, cfg=(1, 4, 32, 0)) == call(d=64, cfg=(1, 4, 32))  # ksplit 0 is ksplit 1


def desc(**kw):
    """A valid square contiguous descriptor on fake pointers, then overrides."""
    B, H, Nq, Nk, d = kw.pop("B", 1), kw.pop("H", 2), kw.pop("Nq", 64), kw.pop("Nk", 64), kw.pop("d", 64)
    a = fa.FwdDesc()
    a.q, a.k, a.v, a.out, a.lse = FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE
    a.B, a.H, a.Nq, a.Nk, a.d = B, H, Nq, Nk, d
    a.q_stride = (ctypes.c_longlong * 3)(H * Nq * d, Nq * d, d)
    a.o_stride = (ctypes.c_longlong * 3)(H * Nq * d, Nq * d, d)
    a.k_stride = (ctypes.c_longlong * 3)(H * Nk * d, Nk * d, d)
    a.v_stride = (ctypes.c_longlong * 3)(H * Nk * d, Nk * d, d)
    a.lse_stride = (ctypes.c_longlong * 2)(H * Nq, Nq)
    a.scale, a.causal, a.stream = 0.125, 0, None
    for key, val in kw.items():
        if key.endswith("stride"):
            val = (ctypes.c_longlong * len(val))(*val)
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(lse=None), 1),
    (dict(Nq=0), 2), (dict(Nk=0), 2), (dict(B=0), 2),
    (dict(d=96), 3),
    (dict(q_stride=(8192, 4096, 32)), 11),            # row stride shorter than a row
    (dict(k_stride=(8192, 4096, 68)), 11),            # not a multiple of 8 elements
    (dict(v_stride=(8192, -4096, 64)), 11),           # negative
    (dict(o_stride=(8192, 4096, 1 << 24)), 11),       # a head beyond 32-bit offsets
    (dict(lse_stride=(-1, 64)), 11),
    (dict(scale=0.0), 4), (dict(causal=3), 5), (dict(dtype=3), 5), (dict(dtype=-1), 5),
    (dict(dtype=2, d=32, q_stride=(4096, 2048, 32), k_stride=(4096, 2048, 32), v_stride=(4096, 2048, 32),
          o_stride=(4096, 2048, 32)), 3),                                   # fp32 takes d = 64 and 128
    (dict(dtype=2, q_stride=(8192, 4096, 66)), 11),                         # fp32 rows: whole 16-byte units
    (dict(dtype=2, k_stride=(8192, 4096, 1 << 23)), 11),                    # fp32 head beyond 2^31 bytes
    (dict(d=48), 3),
    (dict(k=2 * FAKE + 8), 6), (dict(lse=5 * FAKE + 2), 6),
    (dict(out=3 * FAKE), 7), (dict(lse=FAKE + 256), 7),
])
def test_desc_argument_errors(lib, kw, code):
    assert fa.fa_fwd_ex_ptr(desc(**kw)) == code


def test_desc_null_and_unknown_cfg(lib):
    assert lib.fa_fwd_ex(None) == 1
    assert fa.fa_fwd_ex_ptr(desc(), cfg=(3, 4, 64)) == 5


def test_desc_valid_layouts_reach_the_device_check(lib):
    """Legal descriptors pass validation and stop at the device check here:
    non-square, [B, N, H, d] strides, and q, k, v as views of one packed tensor."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    B, H, N, d = 2, 4, 128, 64
    bnhd = (N * H * d, d, H * d)
    assert fa.fa_fwd_ex_ptr(desc(Nq=17, Nk=300)) == 8
    for d in (32, 256):                                     # the other head dims, both element types
        for dt in (0, 1):
            assert fa.fa_fwd_ex_ptr(desc(d=d, dtype=dt)) == 8
    for d in (64, 128):                                     # fp32; a 4-element (16-byte) row pitch is legal
        st = (2 * 64 * (d + 4), 64 * (d + 4), d + 4)
        assert fa.fa_fwd_ex_ptr(desc(d=d, dtype=2, q_stride=st, k_stride=st, v_stride=st, o_stride=st,
                                     out=8 * FAKE)) == 8
    assert fa.fa_fwd_ex_ptr(desc(B=B, H=H, Nq=N, Nk=N, q_stride=bnhd, k_stride=bnhd, v_stride=bnhd,
                                 o_stride=bnhd, out=8 * FAKE)) == 8
    packed = (N * 3 * H * d, d, 3 * H * d)  # [B, N, 3, H, d]: q, k, v interleaved
    assert fa.fa_fwd_ex_ptr(desc(B=B, H=H, Nq=N, Nk=N, q=FAKE, k=FAKE + 2 * H * d, v=FAKE + 4 * H * d,
                                 q_stride=packed, k_stride=packed, v_stride=packed, out=16 * FAKE,
                                 lse=24 * FAKE)) == 8


# ---------------------------------------------------------------- split keys

def test_splitkv_workspace_and_default_splits(lib):
    assert fa.splitkv_workspace_bytes(1, 8, 1024, 1024, 64, 4) == 4 * 8 * 1024 * 65 * 4
    # chunk = ceil(1000 / 3) = 334 -> 384 keys, so 3 splits are used
    assert fa.splitkv_workspace_bytes(1, 1, 10, 1000, 128, 3) == 3 * 10 * 129 * 4
    # 16 requested over 100 keys: chunk 64, 2 splits used
    assert fa.splitkv_workspace_bytes(1, 1, 1, 100, 64, 16) == 2 * 65 * 4
    assert fa.splitkv_default_splits(1, 8, 1024, 1024, 64) == 4      # 32 workgroups, >= 256 keys per split
    # decoding (Nq <= 32): key-split workgroups of one 32-query block, about 256 of them
    assert fa.splitkv_default_splits(1, 32, 1, 32768, 128) == 8      # 32 workgroups -> 8 splits
    assert fa.splitkv_default_splits(4, 32, 1, 8192, 128) == 2       # 128 workgroups -> 2 splits
    assert fa.splitkv_default_splits(8, 32, 1, 4096, 128) == 1       # 256 workgroups already
    assert fa.splitkv_default_splits(4, 8, 1, 4096, 64) == 8         # 32 workgroups, 512 keys per split
    assert fa.splitkv_default_splits(1, 1, 1, 1000, 64) == 1         # >= 512 keys per split
    assert fa.splitkv_default_splits(4, 8, 4096, 4096, 64) == 1      # 512 workgroups already
    with pytest.raises(fa.FaError):
        fa.splitkv_workspace_bytes(1, 1, 1, 1, 96, 1)


WS = 64 * FAKE  # 256-byte aligned, far from the tensors


def test_splitkv_rejects_fp32(lib):
    d = desc(dtype=2)
    assert lib.fa_fwd_splitkv(ctypes.byref(d), 2, ctypes.c_void_p(WS), ctypes.c_longlong(1 << 30)) == 5


@pytest.mark.parametrize("args,code", [
    (dict(ws=None), 12), (dict(ws=WS + 16), 12), (dict(nbytes=100), 12),
    (dict(splits=-1), 5), (dict(splits=2000), 5),
    (dict(ws=FAKE), 7),                       # the workspace overlaps q
])
def test_splitkv_argument_errors(lib, args, code):
    d = desc()
    ws = args.get("ws", WS)
    nbytes = args.get("nbytes", 1 << 30)
    st = lib.fa_fwd_splitkv(ctypes.byref(d), args.get("splits", 2), None if ws is None else ctypes.c_void_p(ws),
                            ctypes.c_longlong(nbytes))
    assert st == code


def test_splitkv_valid_call_reaches_the_device_check(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = desc(Nq=1, Nk=4096)
    assert lib.fa_fwd_splitkv(ctypes.byref(d), 0, ctypes.c_void_p(WS), ctypes.c_longlong(1 << 30)) == 8


def test_splitkv_noalloc_host_checks(lib):
    """The static-scratch entry point: NULL descriptor, the descriptor checks,
    FA_ERR_SCRATCH (13) when the partial results exceed the scratch, decided on
    the host before any device call, and the header's limit equals the
    binding's."""
    assert lib.fa_fwd_splitkv_noalloc(None, 0) == 1
    assert lib.fa_fwd_splitkv_noalloc(ctypes.byref(desc(d=96)), 0) == 3
    assert lib.fa_fwd_splitkv_noalloc(ctypes.byref(desc()), 2000) == 5
    assert lib.fa_fwd_splitkv_noalloc(ctypes.byref(desc(dtype=2)), 2) == 5
    far = 1 << 32  # tensors of 268 MB: keep the fake pointers apart
    big = desc(B=4, H=32, Nq=512, Nk=8192, d=128, q=far, k=2 * far, v=3 * far, out=4 * far, lse=5 * far)
    assert fa.splitkv_workspace_bytes(4, 32, 512, 8192, 128, 8) > fa.SPLITKV_NOALLOC_MAX_BYTES
    assert lib.fa_fwd_splitkv_noalloc(ctypes.byref(big), 8) == 13
    text = open(HEADERS[0]).read()
    m = re.search(r"#define FA_SPLITKV_NOALLOC_MAX_BYTES \((\d+)LL << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.SPLITKV_NOALLOC_MAX_BYTES
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert lib.fa_fwd_splitkv_noalloc(ctypes.byref(desc(Nq=1, Nk=4096)), 0) == 8


# ---------------------------------------------------------------- backward

def bwd_call(**kw):
    a = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, out=4 * FAKE, lse=5 * FAKE, dout=6 * FAKE, dq=7 * FAKE, dk=8 * FAKE,
             dv=9 * FAKE, B=1, H=2, N=64, d=64, scale=0.125, causal=0, ws=WS, nbytes=1 << 30)
    a.update(kw)
    return fa.fa_bwd_ptr(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["B"],
                         a["H"], a["N"], a["d"], a["scale"], a["causal"], a["ws"], a["nbytes"], 0)


def test_bwd_header_compiles_as_c99(tmp_path):
    src = tmp_path / "b.c"
    src.write_text("#include \"fa_bwd.h\"\nint main(void){return fa_bwd_workspace_bytes(1,1,1,64) > 0 ? 0 : 1;}\n")
    assert os.system("gcc -std=c99 -fsyntax-only -I %s %s" % (os.path.join(ROOT, "include"), src)) == 0


def test_bwd_workspace_bytes(lib):
    assert fa.bwd_workspace_bytes(4, 8, 4096, 64) == 8 * 4 * 8 * 4096
    assert fa.bwd_workspace_bytes(1, 1, 1, 128) == 8
    assert fa.bwd_workspace_bytes(2, 1, 5, 32) == 80
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 256) == -3
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 96) == -3
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64) == -2


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(dout=0), 1), (dict(dv=0), 1), (dict(ws=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(N=1 << 24, d=128), 2), (dict(d=256), 3), (dict(d=96), 3),
    (dict(scale=0.0), 4), (dict(scale=float("nan")), 4), (dict(causal=2), 5),
    (dict(dout=6 * FAKE + 8), 6), (dict(dk=8 * FAKE + 2), 6), (dict(lse=5 * FAKE + 1), 6),
    (dict(ws=WS + 64), 12), (dict(nbytes=8 * 2 * 64 - 1), 12),
    (dict(dq=FAKE), 7),                 # dq overwrites q
    (dict(dk=7 * FAKE + 64), 7),        # dk overlaps dq
    (dict(dv=5 * FAKE), 7),             # dv overlaps lse
    (dict(ws=6 * FAKE), 7),             # the workspace overlaps dout
])
def test_bwd_argument_errors(lib, kw, code):
    assert bwd_call(**kw) == code


def test_bwd_valid_call_reaches_the_device_check(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bwd_call() == 8
    assert bwd_call(q=FAKE, k=FAKE, v=FAKE, nbytes=8 * 2 * 64) == 8  # inputs may alias; exact workspace size


# ------------------------------------------------- backward, descriptor form

def bwd_desc(**kw):
    """A valid contiguous bf16 backward descriptor on fake pointers, then overrides
    (stride fields take 3-tuples)."""
    B, H, N, d = kw.pop("B", 1), kw.pop("H", 2), kw.pop("N", 64), kw.pop("d", 64)
    a = fa.BwdDesc()
    a.q, a.k, a.v, a.out, a.lse, a.dout = FAKE, 2 * FAKE, 3 * FAKE, 4 * FAKE, 5 * FAKE, 6 * FAKE
    a.dq, a.dk, a.dv = 7 * FAKE, 8 * FAKE, 9 * FAKE
    a.B, a.H, a.N, a.d = B, H, N, d
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        setattr(a, name + "_stride", (ctypes.c_longlong * 3)(H * N * d, N * d, d))
    a.lse_stride = (ctypes.c_longlong * 2)(H * N, N)
    a.scale, a.causal, a.dtype = 0.125, 0, 0
    a.workspace, a.workspace_bytes, a.stream = WS, 1 << 30, None
    for key, val in kw.items():
        if key.endswith("_stride"):
            val = (ctypes.c_longlong * len(val))(*val)
        setattr(a, key, val)
    return a


def bwd_ex(lib, **kw):
    a = bwd_desc(**kw)
    return lib.fa_bwd_ex(ctypes.byref(a))


def packed(base, B, N, H, d, slot, slots=3):
    """Pointer and strides of slot `slot` of a [B, N, slots, H, d] 16-bit buffer."""
    return base + slot * H * d * 2, (N * slots * H * d, d, slots * H * d)


def test_bwd_ex_null_descriptor(lib):
    assert lib.fa_bwd_ex(None) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(dq=0), 1), (dict(workspace=0), 1),
    (dict(N=0), 2), (dict(B=1 << 12, H=1 << 10, N=1 << 9), 2), (dict(d=256), 3), (dict(d=16), 3),
    (dict(q_stride=(8192, 4096, 68)), 11),          # row stride not a multiple of 8 elements
    (dict(dv_stride=(8192, 4096, 56)), 11),         # row stride < d
    (dict(k_stride=(-8192, 4096, 64)), 11),
    (dict(do_stride=(8192, 4096, 1 << 22)), 11),    # (N + 256) * row stride >= 2^30
    (dict(lse_stride=(-1, 64)), 11),
    (dict(scale=-1.0), 4), (dict(causal=3), 5), (dict(dtype=2), 5), (dict(dtype=7), 5),
    (dict(out=4 * FAKE + 8), 6), (dict(lse=5 * FAKE + 2), 6),
    (dict(workspace=WS + 128), 12), (dict(workspace_bytes=8 * 2 * 64 - 1), 12),
    (dict(dk=7 * FAKE), 7),                         # dk is dq
    (dict(dq=6 * FAKE + 4096), 7),                  # dq inside dout
    (dict(workspace=9 * FAKE), 7),                  # the workspace overlaps dv
])
def test_bwd_ex_argument_errors(lib, kw, code):
    assert bwd_ex(lib, **kw) == code


def test_bwd_ex_interleaved_alias_rule(lib):
    """dq, dk, dv interleaved in one packed [B, N, 3, H, d] buffer are disjoint
    although their extents overlap; shifting one of them by 8 elements makes two
    of them share bytes, and that is rejected."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    B, N, H, d = 2, 64, 2, 64
    P = 16 * FAKE
    g = [packed(P, B, N, H, d, s) for s in range(3)]
    ok = dict(B=B, N=N, H=H, d=d, dq=g[0][0], dq_stride=g[0][1], dk=g[1][0], dk_stride=g[1][1], dv=g[2][0],
              dv_stride=g[2][1], workspace_bytes=8 * B * H * N)
    assert bwd_ex(lib, **ok) == 8  # valid: reaches the device check
    bad = dict(ok, dk=g[1][0] - 16)
    assert bwd_ex(lib, **bad) == 7
    # q, k, v read from a packed buffer, dq beside them in the same rows: a
    # [B, N, 4, H, d] buffer whose slot 3 is written.
    Q = 32 * FAKE
    r = [packed(Q, B, N, H, d, s, slots=4) for s in range(4)]
    mixed = dict(ok, q=r[0][0], q_stride=r[0][1], k=r[1][0], k_stride=r[1][1], v=r[2][0], v_stride=r[2][1],
                 dq=r[3][0], dq_stride=r[3][1])
    assert bwd_ex(lib, **mixed) == 8
    assert bwd_ex(lib, **dict(mixed, dq=r[2][0], dq_stride=r[2][1])) == 7  # dq would overwrite v


def test_bwd_ex_valid_layouts_reach_the_device_check(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    B, N, H, d = 1, 64, 2, 128
    bnhd = (N * H * d, d, H * d)
    assert bwd_ex(lib, B=B, N=N, H=H, d=d, q_stride=bnhd, k_stride=bnhd, v_stride=bnhd, o_stride=bnhd,
                  do_stride=bnhd, dq_stride=bnhd, dk_stride=bnhd, dv_stride=bnhd, lse_stride=(2 * N * H, 2 * N),
                  dtype=1) == 8


@pytest.mark.parametrize("kw,code", [
    (dict(Nk=-1), 2),
    (dict(Nk=1 << 30), 2),                                            # B*H*Nk = 2^31
    # (Nk + 256) * row stride * 2 bytes >= 2^31 for k, although fine for N = 64 rows
    (dict(Nk=1 << 20, k_stride=(1 << 31, 1 << 30, 1024)), 11),
])
def test_bwd_ex_key_length_errors(lib, kw, code):
    assert bwd_ex(lib, **kw) == code


def test_bwd_ex_non_square_reaches_the_device_check(lib):
    """Nq = 64 queries over Nk = 300 keys: k, v, dk, dv take Nk rows; the alias
    check uses each tensor's own extent (dk placed right after a 64-row dq is
    fine, right after a 300-row dq it would not be)."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    H, N, Nk, d = 2, 64, 300, 64
    qs, ks = (H * N * d, N * d, d), (H * Nk * d, Nk * d, d)
    kw = dict(N=N, Nk=Nk, H=H, d=d, q_stride=qs, o_stride=qs, do_stride=qs, dq_stride=qs, k_stride=ks,
              v_stride=ks, dk_stride=ks, dv_stride=ks, lse_stride=(H * N, N))
    assert bwd_ex(lib, **kw) == 8
    assert bwd_ex(lib, **dict(kw, dk=7 * FAKE + H * N * d * 2)) == 8      # just after dq's extent
    assert bwd_ex(lib, **dict(kw, dk=7 * FAKE + H * N * d * 2 - 16)) == 7  # overlaps dq's last row


@pytest.mark.parametrize("args,code", [
    ((0, 1, 64, 64, 0, 0), 2), ((1, 1, 0, 64, 0, 0), 2), ((1, 1, 64, 96, 0, 0), 3), ((1, 1, 64, 32, 0, 2), 3),
    ((1, 1, 64, 64, 2, 0), 5), ((1, 1, 64, 64, 0, 3), 5),
])
def test_launch_cfg_argument_errors(lib, args, code):
    c = fa.TileCfg()
    assert lib.fa_launch_cfg(*args, ctypes.byref(c)) == code


def test_launch_cfg_needs_a_device(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    c = fa.TileCfg()
    assert lib.fa_launch_cfg(4, 8, 4096, 64, 0, 0, ctypes.byref(c)) == 8
    assert lib.fa_launch_cfg(4, 8, 4096, 64, 0, 0, None) == 1


def test_written_tensors_must_not_overlap_themselves(lib):
    """A zero or too-small stride on a written tensor would have two lanes store
    one element: refused with FA_ERR_ALIAS (inputs may still share rows)."""
    d = desc(o_stride=(8192, 0, 64))                        # every head's output on one head
    assert lib.fa_fwd_ex(ctypes.byref(d)) == 7
    d = desc(o_stride=(8192, 64 * 32, 64))                  # heads 32 rows apart, 64 rows each
    assert lib.fa_fwd_ex(ctypes.byref(d)) == 7
    d = desc(lse_stride=(128, 32))                          # lse rows of 64 entries 32 apart
    assert lib.fa_fwd_ex(ctypes.byref(d)) == 7
    assert bwd_ex(lib, dk_stride=(8192, 0, 64)) == 7
    assert bwd_ex(lib, dv_stride=(0, 4096, 64), B=2, workspace_bytes=8 * 2 * 2 * 64) == 7


def test_shared_key_heads_are_valid_inputs(lib):
    """k, v with head stride 0 (one key head for every query head, as in
    multi-query attention) pass the checks; the call reaches the device check."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = desc(k_stride=(4096, 0, 64), v_stride=(4096, 0, 64))
    assert lib.fa_fwd_ex(ctypes.byref(d)) == 8
    assert bwd_ex(lib, k_stride=(4096, 0, 64), v_stride=(4096, 0, 64)) == 8
