"""Shared helpers of the GPU parity tests: move seeded bf16 inputs to the device,
run the HIP path through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import math
import sys

import numpy as np

from inputs import bits_to_f64

# Tolerances on bf16 outputs against the fp64 oracle (element by element over
# every compared row): max |dO| <= 2e-2, mean |dO| <= 2e-3; LSE: |dLSE| <=
# 1e-4 * max(1, |LSE|) (a pure relative bound is ill-posed where LSE ~ 0).
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_REL = 1e-4


def to_device(bits: np.ndarray, device="cuda:0", dtype: str = "bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).to(device)


def gpu_forward(q_bits, k_bits, v_bits, scale, causal, cfg=None, device="cuda:0"):
    import torch
    import flashattention_forward_fa2_amd as fa
    q, k, v = (to_device(a, device) for a in (q_bits, k_bits, v_bits))
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal, cfg=cfg)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return o, lse.cpu().numpy()


def compare(o_gpu_bits, lse_gpu, o_ref, lse_ref, rows=None, label="", dtype="bf16", o_max=None, o_mean=None):
    """Element-wise comparison; returns the error summary, raises on failure."""
    d = o_ref.shape[-1]
    o = bits_to_f64(o_gpu_bits, dtype).reshape(-1, d)
    L = np.asarray(lse_gpu, dtype=np.float64).reshape(-1)
    if rows is not None:
        o = o[rows]
        L = L[rows]
    err = np.abs(o - o_ref)
    lerr = np.abs(L - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    s = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_rel=float(lerr.max()),
             finite=bool(np.all(np.isfinite(o)) and np.all(np.isfinite(L))), rows=int(o.shape[0]))
    print("[parity] %s max|dO|=%.3e mean|dO|=%.3e max dLSE/max(1,|LSE|)=%.3e rows=%d"
          % (label, s["max_abs"], s["mean_abs"], s["lse_rel"], s["rows"]), file=sys.stderr, flush=True)
    assert s["finite"], "non-finite output"
    assert s["max_abs"] <= (O_MAX_ABS if o_max is None else o_max), s
    assert s["mean_abs"] <= (O_MEAN_ABS if o_mean is None else o_mean), s
    assert s["lse_rel"] <= LSE_REL, s
    return s


def fp32_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


# Backward: each gradient tensor is compared as a whole against the fp64 oracle,
# relative to its own scale (gradients have no fixed magnitude):
# max |dG| <= GRAD_MAX_REL * max |G| and rms(dG) <= GRAD_RMS_REL * rms(G).
# With u = 2^-8 (bf16 unit roundoff), rounding the outputs alone gives errors up
# to u |G| with rms about u / sqrt(3) ~ 2.3e-3 of rms(G); the bf16 operands P and
# dS and the bf16 O inside D add less than that again.  Bounds: 2.5 u and 1.8 u/sqrt(3).
GRAD_MAX_REL = 1e-2
GRAD_RMS_REL = 4e-3
# fp16 (u = 2^-11) by the same rule: 2.56 u and 1.77 u / sqrt(3).
GRAD_F16_MAX_REL = 1.25e-3
GRAD_F16_RMS_REL = 5e-4


# A gradient the oracle finds identically zero (every row that reaches it sees
# a single key: P = 1 so dS = P (dP - D) = 0) has no scale to be relative to;
# it is held to the rounding of dP - D instead, absolutely.
GRAD_ZERO_ABS = 1e-4


def compare_grad(g_gpu_bits, g_ref, label="", dtype="bf16"):
    g = bits_to_f64(np.asarray(g_gpu_bits), dtype).reshape(g_ref.shape)
    err = np.abs(g - g_ref)
    if not np.any(g_ref):
        print("[parity] %s reference identically 0, max|dG|=%.3e" % (label, float(err.max())), file=sys.stderr,
              flush=True)
        assert np.all(np.isfinite(g)), "non-finite gradient"
        assert float(err.max()) <= GRAD_ZERO_ABS, float(err.max())
        return dict(max_abs=float(err.max()))
    scale_max = max(float(np.abs(g_ref).max()), 1e-30)
    scale_rms = max(float(np.sqrt(np.mean(g_ref ** 2))), 1e-30)
    s = dict(max_rel=float(err.max()) / scale_max, rms_rel=float(np.sqrt(np.mean(err ** 2))) / scale_rms,
             ref_max=scale_max, finite=bool(np.all(np.isfinite(g))))
    print("[parity] %s max|dG|/max|G|=%.3e rms(dG)/rms(G)=%.3e max|G|=%.3e"
          % (label, s["max_rel"], s["rms_rel"], s["ref_max"]), file=sys.stderr, flush=True)
    max_rel, rms_rel = (GRAD_F16_MAX_REL, GRAD_F16_RMS_REL) if dtype == "f16" else (GRAD_MAX_REL, GRAD_RMS_REL)
    assert s["finite"], "non-finite gradient"
    assert s["max_rel"] <= max_rel, s
    assert s["rms_rel"] <= rms_rel, s
    return s
