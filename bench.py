"""Throughput of the gfx950 FlashAttention-2 forward on one MI355X.

One step = one non-causal and one causal forward pass over the B=4, H=8,
N=4096, d=64 bf16 workload (the shape the article "How to profile and optimise
kernels" benchmarks, section "Where the last article left off" and Round 5),
inputs already resident in HBM.  Prints ONE JSON line:

  value      TFLOP/s of the whole step, FLOPs = 4*B*H*N^2*d per mode, halved
             for causal;
  roofline   the dominant (non-causal) kernel against the bf16 dense MFMA peak,
             its duration taken from HIP events on the launch stream;
  cpu_baseline  the fp64 CPU oracle on a bounded row sample of the same
             workload, on this host's cores (a baseline, not a target), with
             the parity of those rows against the GPU output.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3|4|5]
       python bench.py --bwd ...   (the backward pass instead; its own JSON line)
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (fp16 the same)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s (bf16, causal + non-causal) and % of bf16 MFMA peak"
# The pages' figures for this exact workload (RTX 4070 SUPER, Triton): 1.954 ms
# non-causal and 1.077 ms causal, i.e. 206.16 GFLOP in 3.031 ms.
PAGES_STEP_TFLOPS = (4 * 32 * 4096 ** 2 * 64 * 1.5) / 3.031e-3 / 1e12


def flops(B, H, N, d, causal, Nk=None):
    """4*B*H*N^2*d, halved for causal (the pages' convention); with Nq != Nk
    the exact count of visible (query, key) pairs times 4*d."""
    if Nk is None or Nk == N:
        f = 4.0 * B * H * N * N * d
        return f / 2 if causal else f
    if not causal:
        return 4.0 * B * H * N * Nk * d
    m = min(N, Nk)
    pairs = m * (m + 1) / 2 + (N - m) * Nk  # row i sees min(i + 1, Nk) keys
    return 4.0 * B * H * pairs * d


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cfg", type=str, default=None, help="force a tile variant: qb,waves,bk[,ksplit]")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows-per-head", type=int, default=None)
    ap.add_argument("--ramp-seconds", type=float, default=1.0,
                    help="extra back-to-back launches before timing, so clocks ramp up")
    ap.add_argument("--only", choices=["noncausal", "causal"], default=None,
                    help="run one mode only (counter collection)")
    ap.add_argument("--layout", choices=["bhnd", "bnhd"], default="bhnd",
                    help="bnhd: q, k, v, out stored [B, N, H, d] and passed as strided views (fa_fwd_ex)")
    ap.add_argument("--nq", type=int, default=None,
                    help="use only the first NQ query rows (Nq != Nk, through fa_fwd_ex)")
    ap.add_argument("--splitkv", type=int, default=None, metavar="S",
                    help="run through fa_fwd_splitkv with S key splits (0: the library's default)")
    ap.add_argument("--flush-reps", type=int, default=10,
                    help="launches per mode timed again with caches flushed before each (0: skip)")
    ap.add_argument("--no-gemm", action="store_true", help="skip the attainable-GEMM reference")
    ap.add_argument("--dtype", choices=["bf16", "f16", "f32"], default="bf16",
                    help="element type of q, k, v, out (f16 and f32 run through fa_fwd_ex)")
    ap.add_argument("--headdim", type=int, default=None, choices=[32, 64, 128, 256],
                    help="override the workload's head dimension (same B, H, N and distributions)")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="override the workload's sequence length N (same B, H, d and distributions)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward (fa_bwd: dQ, dK, dV from the forward's out and LSE) instead")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (4 and 5: the long-context targets; 1 and 2: the short ones)")
    ap.add_argument("--extra-steps", type=int, default=10, help="timed launches per mode of workloads 4 and 5")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device copy of MIB MiB (calibrates byte counters)")
    ap.add_argument("--gemm-only", type=int, default=0, metavar="REPS",
                    help="instead of attention, time REPS 8192^3 bf16 GEMMs (torch.mm) after a 1 s ramp "
                         "(the roofline's attainable-GEMM reference alone)")
    return ap.parse_args()


def copy_calibration(mib: int, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4,
                      "copies": reps}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs with no exchange; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    if args.gemm_only:
        import torch
        tflops = attainable_gemm(torch, torch.device("cuda:0"), reps=args.gemm_only)
        print(json.dumps({"gemm": "8192^3 bf16 torch.mm", "tflops": tflops}), flush=True)
        return
    if args.bwd:
        main_bwd(args)
        return

    import torch
    import flashattention_forward_fa2_amd as fa
    import inputs

    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = dict(inputs.WORKLOADS[args.workload])
    if args.headdim:
        w["d"] = args.headdim
        w["name"] = re.sub(r"-d\d+", "-d%d" % args.headdim, w["name"])
    if args.seq_len:
        w["N"] = args.seq_len
        w["name"] = re.sub(r"-N\d+", "-N%d" % args.seq_len, w["name"])
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    modes = list(w["modes"]) if args.workload != 3 else [0, 1]
    if args.only:
        modes = [c for c in modes if c == (args.only == "causal")]
        if not modes:
            print("workload %d has no %s mode" % (args.workload, args.only), file=sys.stderr)
            sys.exit(2)
    scale = inputs.default_scale(d)
    cfg = tuple(int(x) for x in args.cfg.split(",")) if args.cfg else None

    t0 = time.time()
    q_bits, k_bits, v_bits = inputs.make_qkv(args.workload, N=N, d=d, dtype=args.dtype)
    print("[bench] inputs %s generated in %.1fs" % (w["name"], time.time() - t0), file=sys.stderr, flush=True)
    Nk = N
    if args.nq is not None:
        if not 1 <= args.nq <= N:
            print("--nq must be in 1..%d" % N, file=sys.stderr)
            sys.exit(2)
        q_bits = np.ascontiguousarray(q_bits[:, :, :args.nq])
        N = args.nq
    general = args.layout == "bnhd" or N != Nk or args.splitkv is not None or args.dtype != "bf16"
    tdt = {"f16": torch.float16, "f32": torch.float32}.get(args.dtype, torch.bfloat16)
    if args.dtype == "f32":
        to_dev = lambda a: torch.from_numpy(a).to(dev)
    else:
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)
    peak = PEAK_F32_TFLOPS if args.dtype == "f32" else PEAK_BF16_TFLOPS
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    if args.layout == "bnhd":
        # stored [B, N, H, d]; the kernel sees [B, H, N, d] views with row stride H*d
        q, k, v = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (q, k, v))
        outs = {c: torch.empty((B, N, H, d), dtype=tdt, device=dev).transpose(1, 2) for c in modes}
    else:
        outs = {c: torch.empty_like(q) for c in modes}
    lses = {c: torch.empty((B, H, N), dtype=torch.float32, device=dev) for c in modes}
    stream = torch.cuda.current_stream(dev)

    ws = None
    if args.splitkv is not None:
        ws = torch.empty(fa.splitkv_workspace_bytes(B, H, N, Nk, d, args.splitkv), dtype=torch.uint8, device=dev)

    def launch(c):
        if args.splitkv is not None:
            fa.fa_fwd_splitkv(q, k, v, scale=scale, causal=bool(c), out=outs[c], lse=lses[c], stream=stream,
                              num_splits=args.splitkv, workspace=ws)
        elif general:
            fa.fa_fwd_ex(q, k, v, scale=scale, causal=bool(c), out=outs[c], lse=lses[c], stream=stream, cfg=cfg)
        else:
            fa.fa_fwd(q, k, v, scale=scale, causal=bool(c), out=outs[c], lse=lses[c], stream=stream, cfg=cfg)

    # Warm-up: the requested steps, then keep the GPU busy ~1 s so clocks ramp.
    for _ in range(max(1, args.warmup)):
        for c in modes:
            launch(c)
    torch.cuda.synchronize()
    t_end = time.time() + args.ramp_seconds
    while time.time() < t_end:
        for c in modes:
            launch(c)
        torch.cuda.synchronize()

    # Timed region: exactly K steps, HIP events around every kernel on its stream.
    ev = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for c in modes}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        for c in modes:
            ev[c][s][0].record(stream)
            launch(c)
            ev[c][s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    step_flops = sum(flops(B, H, N, d, c, Nk) for c in modes)
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    per_mode = {}
    # Algorithmic HBM bytes of one call: Q, K, V read once, O and LSE written once.
    esz = 4 if args.dtype == "f32" else 2
    algo_bytes = esz * B * H * (2.0 * N * d + 2.0 * Nk * d) + 4.0 * B * H * N
    for c in modes:
        ms = np.array([a.elapsed_time(b) for a, b in ev[c]])
        avg = float(ms.mean())
        tf = flops(B, H, N, d, c, Nk) / (avg * 1e-3) / 1e12
        per_mode["causal" if c else "noncausal"] = dict(
            kernel_ms_avg=round(avg, 5), kernel_ms_median=round(float(np.median(ms)), 5),
            kernel_ms_min=round(float(ms.min()), 5), kernel_ms_max=round(float(ms.max()), 5),
            tflops=round(tf, 2),
            frac_of_peak=round(tf / peak, 4),
            hbm_gbs=round(algo_bytes / (avg * 1e-3) / 1e9, 1),
            cfg=list(cfg if cfg else fa.launch_cfg(B, H, N, d, bool(c), args.dtype)))
    # Outside the timed region: each mode again with the caches flushed before
    # every launch (a 512 MiB write, more than L2 and the 256 MB Infinity Cache).
    if args.flush_reps > 0:
        junk = torch.empty(512 << 18, dtype=torch.float32, device=dev)
        for c in modes:
            fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.flush_reps)]
            for a, b in fev:
                junk.fill_(1.0)
                a.record(stream)
                launch(c)
                b.record(stream)
            torch.cuda.synchronize()
            fms = np.array([a.elapsed_time(b) for a, b in fev])
            pm = per_mode["causal" if c else "noncausal"]
            pm["kernel_ms_flushed_median"] = round(float(np.median(fms)), 5)
            tf_fl = flops(B, H, N, d, c, Nk) / (float(np.median(fms)) * 1e-3) / 1e12
            pm["tflops_flushed"] = round(tf_fl, 2)
            pm["frac_of_peak_flushed"] = round(tf_fl / peak, 4)
        del junk
    dom_c = max(modes, key=lambda c: per_mode["causal" if c else "noncausal"]["kernel_ms_avg"])
    dom = per_mode["causal" if dom_c else "noncausal"]
    kname = ("fa_fwd_splitkv (split + merge kernels, S=%d) d=%d causal=%d" % (args.splitkv, d, dom_c)
             if args.splitkv else "fa_fwd_kernel d=%d causal=%d cfg=%s" % (d, dom_c, dom["cfg"]))
    # The bound is whichever roof the algorithmic work reaches first: the
    # FLOPs at the MFMA peak or the bytes at the HBM peak (one query row per
    # head, as in decoding, is a stream over K and V).
    if algo_bytes / (PEAK_HBM_GBS * 1e9) > flops(B, H, N, d, dom_c, Nk) / (peak * 1e12):
        roofline = dict(bound="hbm", achieved=dom["hbm_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                        frac=round(dom["hbm_gbs"] / PEAK_HBM_GBS, 4), traffic=None,
                        kernel=kname, bytes_per_launch=algo_bytes)
    else:
        roofline = dict(bound="mfma", achieved=dom["tflops"], peak=peak, unit="TFLOP/s",
                        frac=dom["frac_of_peak"],
                        traffic=measured_traffic(B, H, N, d, dom_c) if not general else None,
                        peak_note=("fp32 dense MFMA peak" if args.dtype == "f32"
                                   else "bf16 and fp16 dense MFMA share the 2.5 PFLOP/s peak"),
                        kernel=kname, flops_per_launch=flops(B, H, N, d, dom_c, Nk))
    if not args.no_gemm and roofline["bound"] == "mfma":
        g = attainable_gemm(torch, dev)
        roofline["attainable_gemm_tflops"] = g
        roofline["frac_of_attainable"] = round(dom["tflops"] / g, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, w, modes, q_bits, k_bits, v_bits, scale, outs, lses, args.dtype)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGES_STEP_TFLOPS, 3)
                        if args.workload == 3 and len(modes) == 2 and N == Nk and args.dtype == "bf16" and d == 64
                        else None),
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": "%s%s %s%s%s%s" % (w["name"], {"bf16": "", "f16": " fp16", "f32": " fp32"}[args.dtype],
                                                  "+".join("causal" if c else "non-causal" for c in modes),
                                                "" if args.layout == "bhnd" else " [B,N,H,d] strided",
                                                "" if N == Nk else " Nq=%d" % N,
                                                "" if args.splitkv is None else " split-keys S=%d" % args.splitkv),
                   "Nq": N, "Nk": Nk,
                   "B": B, "H": H, "N": N, "d": d, "scale": scale, "sigma_qk": w["sigma_qk"],
                   "flops_per_step": step_flops, "modes": per_mode},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if rec["vs_baseline"] is not None:
        rec["vs_baseline_basis"] = ("the pages' final Triton kernel on this workload and step (RTX 4070 SUPER, "
                                    "1.954 + 1.077 ms): another machine's figure, context only")
    if cpu is not None:
        rec["vs_cpu_baseline"] = round(value / cpu["value"], 1)
    default_run = (args.workload == 3 and args.layout == "bhnd" and args.nq is None and args.splitkv is None
                   and args.dtype == "bf16" and not args.headdim and not args.seq_len and not args.cfg
                   and not args.only)
    if default_run and not args.no_extra:
        del q, k, v, outs, lses
        torch.cuda.empty_cache()
        ramp = min(0.3, args.ramp_seconds)
        fl = max(0, args.flush_reps)
        rec["targets"] = {"B1-H32-N32768-d128 causal": other_workload(4, [1], args.extra_steps, fl, 8, ramp),
                          "B4-H32-N8192-d128-peaked non-causal": other_workload(5, [0], args.extra_steps, fl, 8, ramp)}
        rec["short_configs"] = {"B1-H1-N256-d64": other_workload(1, [0], 50, 4 * fl, None, ramp),
                                "B1-H8-N1024-d64": other_workload(2, [0, 1], 50, 4 * fl, None, ramp)}
    print(json.dumps(rec), flush=True)


def other_workload(wl, modes, steps, flush_reps, rows_per_head, ramp_seconds=0.3):
    """One more workload through fa_fwd with the default launch: per mode, kernel
    time from HIP events on the launch stream (back to back after a short ramp,
    and again each launch after a 512 MiB cache flush), TFLOP/s and fraction of
    the bf16 dense peak both ways, algorithmic HBM GB/s, and the output's parity
    with the oracle on every row (rows_per_head None) or on a row sample."""
    import torch
    import flashattention_forward_fa2_amd as fa
    import inputs
    import oracle
    from inputs import bits_to_f64, sample_rows, workload_seed

    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[wl]
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    scale = inputs.default_scale(d)
    t0 = time.time()
    q_bits, k_bits, v_bits = inputs.make_qkv(wl)
    print("[bench] inputs %s generated in %.1fs" % (w["name"], time.time() - t0), file=sys.stderr, flush=True)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to_dev(q_bits), to_dev(k_bits), to_dev(v_bits)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    algo_bytes = 2.0 * B * H * 4 * N * d + 4.0 * B * H * N
    res = {"B": B, "H": H, "N": N, "d": d, "sigma_qk": w["sigma_qk"]}
    junk = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    for c in modes:
        launch = lambda: fa.fa_fwd(q, k, v, scale=scale, causal=bool(c), out=out, lse=lse, stream=stream)
        launch()
        torch.cuda.synchronize()
        t_end = time.time() + ramp_seconds
        while time.time() < t_end:
            launch()
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(flush_reps)]
        for a, b in fev:
            junk.fill_(1.0)
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        fms = np.array([a.elapsed_time(b) for a, b in fev]) if fev else ms
        f = flops(B, H, N, d, c)
        avg, fmed = float(ms.mean()), float(np.median(fms))
        entry = dict(kernel_ms_avg=round(avg, 5), kernel_ms_median=round(float(np.median(ms)), 5),
                     kernel_ms_min=round(float(ms.min()), 5), kernel_ms_max=round(float(ms.max()), 5),
                     tflops=round(f / (avg * 1e-3) / 1e12, 2), frac_of_peak=round(f / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     kernel_ms_flushed_median=round(fmed, 5),
                     tflops_flushed=round(f / (fmed * 1e-3) / 1e12, 2),
                     frac_of_peak_flushed=round(f / (fmed * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     hbm_gbs=round(algo_bytes / (avg * 1e-3) / 1e9, 1),
                     hbm_gbs_flushed=round(algo_bytes / (fmed * 1e-3) / 1e9, 1),
                     cfg=list(fa.launch_cfg(B, H, N, d, bool(c))), launches=steps, flushed_launches=flush_reps)
        # parity of this output with the oracle
        rows = (np.arange(B * H * N, dtype=np.int64) if rows_per_head is None
                else sample_rows(workload_seed(wl, 3), B, H, N, per_head=rows_per_head))
        o_ref, l_ref = oracle.attention_rows(q_bits, k_bits, v_bits, scale, bool(c), rows)
        o = bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(-1, d)[rows]
        L = lse.cpu().numpy().reshape(-1)[rows]
        err = np.abs(o - o_ref)
        entry["parity"] = dict(rows=int(rows.size), max_abs=float(err.max()), mean_abs=float(err.mean()),
                               lse_rel=float((np.abs(L - l_ref) / np.maximum(1.0, np.abs(l_ref))).max()))
        res["causal" if c else "noncausal"] = entry
    del junk, q, k, v, out, lse
    torch.cuda.empty_cache()
    return res


BWD_METRIC = "attention bwd TFLOP/s (bf16, dQ dK dV; 2.5x the forward's FLOPs) and % of bf16 MFMA peak"


def main_bwd(args):
    """The backward pass (three kernels per call) over the workload's modes:
    out, LSE and dO are computed / drawn before the timed region; one step is
    one backward call per mode (fa_bwd, or fa_bwd_ex for fp16 or the [B, N, H, d]
    layout).  FLOPs are the 5 matrix products of the chain rule,
    10*B*H*N^2*d (halved for causal); the dQ pass's recomputation of S and dP
    is not counted."""
    import torch
    import flashattention_forward_fa2_amd as fa
    import inputs

    if args.dtype == "f32":
        print("the backward takes bf16 or f16 inputs", file=sys.stderr)
        sys.exit(2)
    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = dict(inputs.WORKLOADS[args.workload])
    if args.headdim:
        w["d"] = args.headdim
        w["name"] = re.sub(r"-d\d+", "-d%d" % args.headdim, w["name"])
    if args.seq_len:
        w["N"] = args.seq_len
        w["name"] = re.sub(r"-N\d+", "-N%d" % args.seq_len, w["name"])
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    modes = list(w["modes"]) if args.workload != 3 else [0, 1]
    if args.only:
        modes = [c for c in modes if c == (args.only == "causal")]
    scale = inputs.default_scale(d)
    q_bits, k_bits, v_bits = inputs.make_qkv(args.workload, N=N, d=d, dtype=args.dtype)
    g_bits = inputs.normal_bits(inputs.workload_seed(args.workload, 4), B * H * N * d,
                                dtype=args.dtype).reshape(B, H, N, d)
    tdt = torch.float16 if args.dtype == "f16" else torch.bfloat16
    general = args.layout == "bnhd" or args.dtype != "bf16"
    if args.layout == "bnhd":
        # stored [B, N, H, d]; the kernels see [B, H, N, d] views with row stride H*d
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)).view(np.int16)).view(
            tdt).to(dev).transpose(1, 2)
        new = lambda: torch.empty((B, N, H, d), dtype=tdt, device=dev).transpose(1, 2)
    else:
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)
        new = lambda: torch.empty((B, H, N, d), dtype=tdt, device=dev)
    q, k, v, dout = (to_dev(a) for a in (q_bits, k_bits, v_bits, g_bits))
    stream = torch.cuda.current_stream(dev)
    fwd = fa.fa_fwd_ex if general else fa.fa_fwd
    fw = {}
    for c in modes:
        o = new()
        fw[c] = fwd(q, k, v, scale=scale, causal=bool(c), out=o, stream=stream)
    grads = {c: tuple(new() for _ in range(3)) for c in modes}
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    bwd = fa.fa_bwd_ex if general else fa.fa_bwd

    def launch(c):
        bwd(q, k, v, fw[c][0], fw[c][1], dout, scale=scale, causal=bool(c), dq=grads[c][0], dk=grads[c][1],
            dv=grads[c][2], workspace=ws, stream=stream)

    for _ in range(max(1, args.warmup)):
        for c in modes:
            launch(c)
    torch.cuda.synchronize()
    t_end = time.time() + args.ramp_seconds
    while time.time() < t_end:
        for c in modes:
            launch(c)
        torch.cuda.synchronize()
    ev = {c: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for c in modes}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        for c in modes:
            ev[c][s][0].record(stream)
            launch(c)
            ev[c][s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    bflops = lambda c: 2.5 * flops(B, H, N, d, c)
    step_flops = sum(bflops(c) for c in modes)
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    per_mode = {}
    for c in modes:
        ms = np.array([a.elapsed_time(b) for a, b in ev[c]])
        avg = float(ms.mean())
        tf = bflops(c) / (avg * 1e-3) / 1e12
        per_mode["causal" if c else "noncausal"] = dict(
            call_ms_avg=round(avg, 5), call_ms_median=round(float(np.median(ms)), 5),
            call_ms_min=round(float(ms.min()), 5), tflops=round(tf, 2), frac_of_peak=round(tf / PEAK_BF16_TFLOPS, 4))
    dom_c = max(modes, key=lambda c: per_mode["causal" if c else "noncausal"]["call_ms_avg"])
    dom = per_mode["causal" if dom_c else "noncausal"]
    traffic = None if general else measured_traffic_bwd(B, H, N, d, dom_c)
    roofline = dict(bound="mfma", achieved=dom["tflops"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=dom["frac_of_peak"], traffic=traffic,
                    kernel="%s (pre + dK/dV + dQ kernels) d=%d causal=%d" % (bwd.__name__, d, dom_c),
                    flops_per_launch=bflops(dom_c))

    cpu = None
    if not args.no_cpu_baseline and 2.5 * flops(1, 1, N, d, max(modes)) <= 300e9:
        import oracle
        from inputs import bits_to_f64
        # one whole head per oracle thread, within ~300 GFLOP of fp64 work
        nh = min(B * H, max(1, oracle.num_threads()), int(300e9 // (2.5 * flops(1, 1, N, d, max(modes)) * len(modes))))
        heads = [(i // H, i % H) for i in range(0, B * H, max(1, (B * H) // nh))][:nh]
        sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
        total_flops, total_s, parity = 0.0, 0.0, {}
        for c in modes:
            t0 = time.perf_counter()
            ref = oracle.attention_bwd(sel(q_bits), sel(k_bits), sel(v_bits), sel(g_bits), scale, bool(c),
                                       dtype=args.dtype)
            total_s += time.perf_counter() - t0
            total_flops += 2.5 * flops(1, len(heads), N, d, c)
            errs = {}
            for name, g, r in zip(("dq", "dk", "dv"), grads[c], ref):
                gb = sel(g.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
                e = np.abs(bits_to_f64(gb, args.dtype) - r)
                errs[name] = dict(max_rel=float(e.max() / np.abs(r).max()),
                                  rms_rel=float(np.sqrt(np.mean(e ** 2)) / np.sqrt(np.mean(r ** 2))))
            parity["causal" if c else "noncausal"] = errs
        cpu = dict(value=round(total_flops / total_s / 1e12, 6), unit="TFLOP/s", cores=oracle.num_threads(),
                   kind="oracle",
                   sample="%d whole heads of %s (b, h = %s), modes %s; fp64 backward, %.1f GFLOP in %.2fs"
                          % (len(heads), w["name"], heads, modes, total_flops / 1e9, total_s),
                   parity_on_sample=parity)

    rec = {
        "metric": BWD_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": "%s%s%s backward %s" % (w["name"], " fp16" if args.dtype == "f16" else "",
                                                       " [B,N,H,d] strided" if args.layout == "bnhd" else "",
                                                       "+".join("causal" if c else "non-causal" for c in modes)),
                   "B": B, "H": H, "N": N, "d": d, "scale": scale, "flops_per_step": step_flops, "modes": per_mode},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def attainable_gemm(torch, dev, n=8192, reps=20, ramp_seconds=1.0):
    """A large dense bf16 GEMM through torch (hipBLASLt) on the same GPU: the MFMA
    rate a library reaches here, reported beside the nominal peak.  Timed after
    ramp_seconds of back-to-back GEMMs (its first dispatches run up to a third
    slower while the clock settles)."""
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    torch.mm(a, b)
    torch.cuda.synchronize()
    t_end = time.time() + ramp_seconds
    while time.time() < t_end:
        for _ in range(4):
            torch.mm(a, b)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)


def measured_traffic(B, H, N, d, causal):
    """HBM bytes per launch from the committed counter summary under profiles/
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's counts), or None when
    there is none for this shape or the kernel sources changed since."""
    from flashattention_forward_fa2_amd.buildlib import source_digest
    path = os.path.join(ROOT, "profiles", "fa_fwd_all_workloads_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    digest = re.search(r"kernel-source-sha256: ([0-9a-f]{64})", text)
    if not digest or digest.group(1) != source_digest():
        return None
    m = re.search(r"traffic-bytes-per-launch d%d %s B%dH%dN%d: (\d+)"
                  % (d, "causal" if causal else "noncausal", B, H, N), text)
    return int(m.group(1)) if m else None


def measured_traffic_bwd(B, H, N, d, causal):
    """HBM bytes of one fa_bwd call (its three kernels) from the committed counter
    summary, or None when there is none for this shape or the sources changed."""
    from flashattention_forward_fa2_amd.buildlib import BWD_SOURCES, source_digest
    path = os.path.join(ROOT, "profiles", "fa_bwd_d%d_B%dH%dN%d_hbm_traffic.md" % (d, B, H, N))
    if not os.path.exists(path):
        return None
    text = open(path).read()
    digest = re.search(r"kernel-source-sha256: ([0-9a-f]{64})", text)
    if not digest or digest.group(1) != source_digest(BWD_SOURCES):
        return None
    m = re.search(r"traffic-bytes-per-call d%d %s B%dH%dN%d: (\d+)"
                  % (d, "causal" if causal else "noncausal", B, H, N), text)
    return int(m.group(1)) if m else None


def cpu_baseline(args, w, modes, q_bits, k_bits, v_bits, scale, outs, lses, dtype="bf16"):
    """The oracle, as it stands, on a bounded row sample of the same workload."""
    import torch
    import oracle
    from inputs import bits_to_f64, sample_rows, workload_seed

    B, H, d = w["B"], w["H"], w["d"]
    N, Nk = q_bits.shape[2], k_bits.shape[2]  # query rows, key rows
    # About 250 GFLOP of fp64 oracle work (~10 s on 16 host cores), at most every row.
    mode_weight = sum(0.5 if c else 1.0 for c in modes)
    per_head = args.cpu_rows_per_head or int(np.clip(250e9 / (B * H * 4.0 * Nk * d * mode_weight), 16, N))
    if per_head >= N:  # the budget covers the whole workload: every row
        rows = np.arange(B * H * N, dtype=np.int64)
    else:
        rows = sample_rows(workload_seed(args.workload, 3), B, H, N, per_head=per_head)
    i = rows % N
    total_flops, total_s = 0.0, 0.0
    parity = {}
    for c in modes:
        t0 = time.perf_counter()
        if dtype == "f32":
            o_ref, l_ref = oracle.attention_rows_f32(q_bits, k_bits, v_bits, scale, bool(c), rows)
        else:
            o_ref, l_ref = oracle.attention_rows(q_bits, k_bits, v_bits, scale, bool(c), rows, dtype=dtype)
        total_s += time.perf_counter() - t0
        nkeys = np.minimum(i + 1, Nk) if c else np.full(rows.shape, Nk)
        total_flops += float(np.sum(4.0 * nkeys * d))
        if dtype == "f32":
            o = outs[c].contiguous().cpu().numpy().astype(np.float64).reshape(-1, d)[rows]
        else:
            o = bits_to_f64(outs[c].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), dtype).reshape(-1, d)[rows]
        L = lses[c].cpu().numpy().reshape(-1)[rows]
        err = np.abs(o - o_ref)
        parity["causal" if c else "noncausal"] = dict(
            max_abs=float(err.max()), mean_abs=float(err.mean()),
            lse_rel=float((np.abs(L - l_ref) / np.maximum(1.0, np.abs(l_ref))).max()))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(value=round(total_flops / total_s / 1e12, 6), unit="TFLOP/s", cores=oracle.num_threads(),
                kind="oracle",
                sample="%d rows (%d per head; all rows, or fixed edge rows + seeded) of %s, modes %s; fp64, %.1f GFLOP in %.2fs"
                       % (rows.size, per_head, w["name"], modes, total_flops / 1e9, total_s),
                cpu_model=cpu_model, parity_on_sample=parity)


if __name__ == "__main__":
    main()
