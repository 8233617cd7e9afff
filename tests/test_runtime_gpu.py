"""The library shares torch's HIP runtime whatever the import order: loading it
(e.g. by listing its variants) before torch is imported still gives a working
call.  Run in a fresh interpreter, since the order is per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, %r)
import flashattention_forward_fa2_amd as fa
fa.variants()                       # loads the library before the script imports torch
import torch
assert torch.cuda.is_available()
maps = open("/proc/self/maps").read()
runtimes = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
q = torch.randn(1, 2, 256, 64, device="cuda", dtype=torch.bfloat16)
out, lse = fa.fa_fwd(q, q, q, causal=True)
torch.cuda.synchronize()
assert torch.isfinite(out.float()).all()
print("RUNTIMES", len(runtimes), sorted(runtimes))
"""


def test_library_loaded_before_torch_still_works():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, "-c", SCRIPT % ROOT], capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], file=sys.stderr, flush=True)
    assert r.returncode == 0, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("RUNTIMES")][0]
    assert line.split()[1] == "1", line  # one HIP runtime in the process
