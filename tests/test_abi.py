"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call.  CPU only (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import flashattention_forward_fa2_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB):
        fa.build()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


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
    for code in range(11):
        assert fa.strerror(code)
    assert fa.strerror(99) == "unknown status"


def test_variant_table(lib):
    vs = fa.variants()
    assert len(vs) >= 4  # both head dims x both modes
    for d in (64, 128):
        for causal in (0, 1):
            assert any(v[0] == d and v[1] == causal for v in vs)
            assert (d, causal, fa.default_cfg(4096, d, causal)) in vs


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: checks fail before any HIP call


def call(q=FAKE, k=2 * FAKE, v=3 * FAKE, out=4 * FAKE, lse=5 * FAKE, B=1, H=1, N=64, d=64, scale=0.125,
         causal=0, cfg=None):
    return fa.fa_fwd_ptr(q, k, v, out, lse, B, H, N, d, scale, causal, 0, cfg)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(out=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2),
    (dict(B=1 << 12, H=1 << 12, N=1 << 10), 2),
    (dict(N=1 << 24, d=128), 2),
    (dict(d=32), 3), (dict(d=96), 3), (dict(d=256), 3),
    (dict(scale=0.0), 4), (dict(scale=-0.1), 4), (dict(scale=float("inf")), 4), (dict(scale=float("nan")), 4),
    (dict(causal=2), 5), (dict(causal=-1), 5),
    (dict(q=FAKE + 8), 6), (dict(out=4 * FAKE + 4), 6), (dict(lse=5 * FAKE + 2), 6),
    (dict(out=FAKE), 7), (dict(out=FAKE + 16), 7), (dict(lse=3 * FAKE + 64), 7), (dict(lse=4 * FAKE + 1024), 7),
])
def test_argument_errors_return_codes(lib, kw, code):
    assert call(**kw) == code


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
