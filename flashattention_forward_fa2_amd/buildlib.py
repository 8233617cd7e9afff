"""Build libfa_fwd.so (HIP, gfx950 only; forward and backward) in-tree with hipcc."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_fwd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # MFMA accumulators in VGPRs: no AGPR<->VGPR copies around the rescale
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def source_digest(names=("fa_fwd_kernel.hpp", "fa_fwd_f32_kernel.hpp", "fa_fwd.hip")) -> str:
    """sha256 over kernel sources and the device flags: identifies the compiled
    kernels, so that measurements taken on one build are not reported for
    another.  The default covers the forward; pass ``BWD_SOURCES`` for the
    backward."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(DEVICE_FLAGS).encode())
    return h.hexdigest()


SOURCES = ("fa_fwd.hip", "fa_bwd.hip")
BWD_SOURCES = ("fa_fwd_kernel.hpp", "fa_bwd_kernel.hpp", "fa_bwd.hip")


def build(verbose: bool = False, extra=()) -> str:
    """Compile the forward and backward sources into one shared library."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *extra,
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def resource_usage() -> list[dict]:
    """Per-kernel resources of the device code as the library builds it (the
    compiler's kernel-resource-usage remarks): one dict per kernel with its
    demangled name, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD and
    LDS bytes per workgroup."""
    import re
    fields = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "waves", "LDS Size [bytes/block]": "lds"}
    out = []
    for src in SOURCES:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "--cuda-device-only", "-c",
               "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
               "-o", os.devnull, os.path.join(CSRC, src)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, res.stderr[-2000:]))
        cur = None
        for line in res.stderr.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = {"mangled": m.group(1), "source": src}
                out.append(cur)
                continue
            for label, key in fields.items():
                m = re.search(re.escape(label) + r": (\d+)", line)
                if m and cur is not None:
                    cur[key] = int(m.group(1))
    names = subprocess.run(["c++filt"], input="\n".join(k["mangled"] for k in out), capture_output=True,
                           text=True).stdout.splitlines()
    for k, n in zip(out, names):
        k["name"] = n.replace("fa::", "").replace("(fa::Params)", "").replace("(fa::BwdParams)", "")
    return out


if __name__ == "__main__":
    if sys.argv[1:] == ["--resources"]:
        print("| kernel | VGPR | AGPR | scratch B/lane | waves/SIMD | LDS B |")
        print("|---|---|---|---|---|---|")
        for k in resource_usage():
            print("| `%s` | %d | %d | %d | %d | %d |" % (k["name"], k.get("vgpr", 0), k.get("agpr", 0),
                                                        k.get("scratch", 0), k.get("waves", 0), k.get("lds", 0)))
    else:
        print(build(verbose=True))
