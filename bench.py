"""Throughput of exact tiled attention (fa_fwd + fa_bwd) on one MI355X.

One step is the whole hot path over one batch: the forward (O, LSE) and the
backward (dQ, dK, dV) of causal bf16 attention at B=4, H=64, N=4096, d=128
with Q, K ~ N(0, 3^2) and V, dO ~ N(0, 1) (synthetic, seeded). Inputs are
resident in HBM before the timed region starts.

FLOPs are counted algorithmically: 4 B H N^2 d for the forward, halved when
causal, and 2.5 times that for the backward. The printed JSON line carries:
  value      whole-step (fwd + bwd) TFLOP/s
  fwd_*      the forward alone, the figure the 50%-of-peak target is set on
  roofline   the dominant launch (the one with the largest time share),
             timed live with HIP events on the stream it runs on; fa_bwd is
             one launch sequence of three kernels and is timed as a unit
  roofline_fwd  the same for fa_fwd
  cpu_baseline  the CPU fp64 oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "exact_tiled_attention_17_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_4x64x4096x128_causal.json")

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0

# Page 4 ("RTX Flash Attention Implementation COMPLETE", Performance
# Specifications) times for the same shapes on another GPU; context only.
PAGE_TIMES_MS = {"2x8x512x64": 0.85, "4x32x1024x128": 2.1, "8x64x2048x128": 8.3,
                 "4x64x4096x128": 15.2}


def _strip_comments(src: str) -> str:
    """C++ source without comments and blank lines (string literals in these
    sources hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """sha256 over the HIP sources' code (comments dropped), to tell whether
    stored counters still apply."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _strip_comments(f.read()).encode())
    return h.hexdigest()


def stored_traffic(launch: str):
    """HBM bytes per launch from the committed counter summary, or None if the
    kernels changed since the counters were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch", {}).get(launch)


def time_stats(ms):
    """Median, min and 90th percentile of per-launch times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def parse_dpm_levels(text):
    """Engine-clock levels (MHz) from a pp_dpm_sclk listing ("0: 500Mhz *")."""
    out = []
    for line in text.splitlines():
        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
        if m:
            out.append(int(m.group(1)))
    return out


def reported_peak(cus):
    """bf16 dense matrix-core peak at the highest engine clock the driver lists:
    CUs x 4096 FLOP per clock (4 SIMDs x one 32x32x16 product, 32768 FLOP, per
    32 cycles each). Returns (peak TFLOP/s, clock MHz, source) or Nones."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                levels = parse_dpm_levels(f.read())
        except OSError:
            continue
        if levels:
            mhz = max(levels)
            return cus * 4096 * mhz * 1e6 / 1e12, mhz, path
    return None, None, None


def flops(w, causal):
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    if causal:
        f *= 0.5
    return f, 2.5 * f


def cpu_baseline(w, causal, budget_s=15.0):
    """The fp64 oracle (as it stands) on whole heads of the same workload."""
    import numpy as np
    import attn_inputs as ai
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((int(i.get("num_threads", 1)) for i in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    f_fwd_head = 4.0 * w.N * w.N * w.d * (0.5 if causal else 1.0)
    f_head = 3.5 * f_fwd_head
    x = ai.make_qkv(1, 1, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v, with_do=True)
    heads, t_total = 0, 0.0
    while t_total < budget_s and heads < 64:
        q, k, v, do = (oracle.bf16_bits_to_f64(x[n][0, 0]) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        oracle.head_forward(q, k, v, causal, w.scale)
        oracle.head_backward(q, k, v, do, causal, w.scale)
        t_total += time.perf_counter() - t0
        heads += 1
    return {"value": heads * f_head / t_total / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads} whole head(s) of {w.label} causal={causal}, fwd+bwd in fp64 "
                      f"({t_total:.1f} s); FLOPs counted like the GPU line (the oracle does "
                      f"the full N^2 work)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", help="attn_inputs workload name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time only fa_fwd (profiling aid)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="K/V heads (grouped-query attention; default: as many as query heads)")
    ap.add_argument("--dtype", choices=("bf16", "f16"), default="bf16",
                    help="element type of Q, K, V, O, dO and the gradients")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warmup, run one device-to-device copy of this many MiB "
                         "(a known-size kernel to calibrate HBM byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every (batch, head) "
              "is independent, so N GPUs would each run this same kernel on B*H/N heads.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import attn_inputs as ai
    import exact_tiled_attention_17_amd as fa

    w = ai.WORKLOADS[args.workload]
    causal = True if True in w.causal_modes else False
    hkv = args.kv_heads or w.H
    if w.H % hkv:
        sys.exit(f"--kv-heads {hkv} must divide the {w.H} query heads")
    # the stored counter figures are for the default launch only
    default_launch = hkv == w.H and args.dtype == "bf16"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v,
                    with_do=True, dtype=args.dtype, Hkv=hkv)
    tdt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    t = {n: torch.from_numpy(x[n].view(np.int16)).view(tdt).to(dev) for n in x}
    del x
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.forward(q, k, v, causal, w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        if not args.fwd_only:
            fa.backward(do, q, k, v, o, lse, causal, w.scale, dq=dq, dk=dk, dv=dv)
            if ev is not None:
                ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the per-key attention mass (a second pass after the forward, not part of
    # the training step): timed on its own, same stream, same inputs
    mass_ms = None
    if not args.fwd_only:
        mass = torch.empty((w.B, w.N), dtype=torch.float32, device=dev)
        fa.key_mass(q, k, lse, causal, w.scale, out=mass)
        mev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in mev:
            e0.record(stream)
            fa.key_mass(q, k, lse, causal, w.scale, out=mass)
            e1.record(stream)
        torch.cuda.synchronize()
        mass_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in mev]))
    # the FP8 forward (Q, K quantised per 16 x 16 block), bf16 inputs only
    fp8_ms = None
    if args.dtype == "bf16":
        o8 = torch.empty_like(q)
        l8 = torch.empty_like(lse)
        fa.forward_fp8(q, k, v, causal, w.scale, out=o8, lse=l8)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in fev:
            e0.record(stream)
            fa.forward_fp8(q, k, v, causal, w.scale, out=o8, lse=l8)
            e1.record(stream)
        torch.cuda.synchronize()
        fp8_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fev]))
        del o8, l8

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs] if not args.fwd_only else [0.0]
    f_fwd, f_bwd = flops(w, causal)
    ms_step = wall * 1e3 / args.steps
    t_fwd = float(np.mean(fwd_ms))
    t_bwd = float(np.mean(bwd_ms))
    fwd_tf = f_fwd / (t_fwd * 1e-3) / 1e12
    bwd_tf = f_bwd / (t_bwd * 1e-3) / 1e12 if t_bwd > 0 else 0.0
    step_flops = f_fwd + (0.0 if args.fwd_only else f_bwd)
    value = step_flops / (ms_step * 1e-3) / 1e12

    def roof(launch, kernels, fl, tms):
        achieved = fl / (tms * 1e-3) / 1e12
        traffic = stored_traffic(launch) if default_launch else None
        r = {"bound": "mfma", "kernel": f"{launch} ({kernels})", "achieved": round(achieved, 2),
             "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
             "traffic": traffic,
             "avg_launch_ms": round(tms, 4)}
        if traffic is not None:  # measured HBM bytes per launch over this launch time
            r["hbm_gbs"] = round(traffic / (tms * 1e-3) / 1e9, 1)
            r["hbm_frac"] = round(traffic / (tms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        return r

    r_fwd = roof("fa_fwd", "fwd_kernel", f_fwd, t_fwd)
    r_bwd = roof("fa_bwd", "bwd_dq_kernel + bwd_dkdv_kernel", f_bwd, t_bwd) \
        if not args.fwd_only else None
    roofline = r_bwd if (r_bwd is not None and t_bwd >= t_fwd) else r_fwd
    # S = Q K^T is the pass's only product: half the forward's FLOPs
    r_mass = roof("fa_key_mass", "key_mass_kernel + key_mass_reduce_kernel", f_fwd / 2, mass_ms) \
        if mass_ms is not None else None
    # its products run on bf16 matrix cores (the dequantised operands are exact in bf16)
    r_fp8 = roof("fa_fwd_fp8", "quant_e4m3_kernel (K) + fwd_kernel (Q quantised on load)", f_fwd, fp8_ms) \
        if fp8_ms is not None else None

    out = {
        "metric": "bf16 attention TFLOP/s fwd & fwd+bwd at 4x64x4096x128 causal, % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"attention fwd+bwd, causal={causal}, B={w.B} H={w.H} N={w.N} "
                               f"d={w.d}, Q,K~N(0,{w.sigma_qk:g}^2), V,dO~N(0,1), seed {w.seed}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                   "fwd_only": args.fwd_only},
        "fwd_ms": round(t_fwd, 4),
        "bwd_ms": round(t_bwd, 4),
        "fwd_ms_stats": time_stats(fwd_ms),
        "bwd_ms_stats": time_stats(bwd_ms),
        "fwd_tflops": round(fwd_tf, 2),
        "bwd_tflops": round(bwd_tf, 2),
        "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
        "fwd_bwd_pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "page_context_ms": PAGE_TIMES_MS.get(w.label),
        "roofline": roofline,
        "roofline_fwd": r_fwd,
        "roofline_key_mass": r_mass,
        "roofline_fwd_fp8": r_fp8,
        "cpu_baseline": None,
    }
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    pk, mhz, src = reported_peak(cus)
    out["peak_at_reported_clock"] = {
        "tflops": round(pk, 1) if pk else None, "sclk_mhz": mhz, "cus": cus, "source": src,
        "fwd_frac": round(fwd_tf / pk, 4) if pk else None,
        "note": "bf16 dense matrix-core peak recomputed as CUs x 4096 FLOP/clock at the highest "
                "engine clock the driver lists; `peak` in the roofline objects is the published "
                "2.5 PFLOP/s"}
    if hkv != w.H:
        out["config"]["workload"] += f", {hkv} K/V heads"
        out["config"]["Hkv"] = hkv
    if args.dtype != "bf16":
        out["config"]["workload"] += f", {args.dtype} inputs"
    if not args.no_cpu_baseline and default_launch:
        out["cpu_baseline"] = cpu_baseline(w, causal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
