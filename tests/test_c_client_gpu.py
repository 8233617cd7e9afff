"""The C ABI from a plain C program: gcc builds tests/c/abi_demo.c against
include/fa_fwd.h, libfa_fwd.so and the HIP runtime's C API (no torch, no
Python in the compute path); it runs fa_fwd and fa_fwd_ex on device memory it
allocates itself and checks every output element against the CPU oracle."""
import os
import subprocess
import sys

import pytest

import oracle
import flashattention_forward_fa2_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_demo(tmp_path):
    exe = str(tmp_path / "abi_demo")
    oracle.build(force=False)
    libdir, oradir = os.path.dirname(fa.LIB), os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c", "abi_demo.c"), "-o", exe,
           "-L", libdir, "-lfa_fwd", "-L", oradir, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + libdir, "-Wl,-rpath," + oradir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_builds(tmp_path):
    """CPU: the client compiles and links as plain C."""
    if not os.path.exists(fa.LIB):
        pytest.skip("library not built")
    build_demo(tmp_path)


@pytest.mark.gpu
def test_c_client_runs_on_the_gpu(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build_demo(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    print(r.stdout, r.stderr, file=sys.stderr, flush=True)
    assert r.returncode == 0 and "ABI_DEMO OK" in r.stdout, (r.returncode, r.stdout, r.stderr)
