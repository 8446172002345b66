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

`--all-workloads` instead times all five workloads of attn_inputs (the shapes
of the "Performance Specifications" table of "RTX Flash Attention
Implementation COMPLETE") in one run, forward and backward each, with the
oracle timed on a bounded sample of distinct heads of each, and prints one
JSON line per workload and causal mode (optionally a markdown table too).
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
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)
# S = Q K^T on FP8, P V on bf16, equal FLOPs
PEAK_MX_MIX_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
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


def alg_bytes(w):
    """The method's minimum HBM bytes per launch: the forward reads Q, K, V and
    writes O (bf16) and the LSE (float32); the backward reads Q, K, V, O, dO
    and writes dQ, dK, dV (bf16), and reads the LSE, writes and reads D."""
    n = w.B * w.H * w.N
    return 8.0 * n * w.d + 4.0 * n, 16.0 * n * w.d + 12.0 * n


def host_cores():
    return len(os.sched_getaffinity(0))


def oracle_rate(w, causal, x, backward=True, budget_s=15.0, max_heads=64):
    """The fp64 oracle, as it stands, on distinct whole heads (b, h) of the
    workload's own inputs `x` (uint16 bits), in order (0, 0), (0, 1), ...,
    until `budget_s` of oracle time; BLAS threads = the cores this process may
    run on. FLOPs are counted like the GPU line (the oracle does the full N^2
    work even when causal)."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores = host_cores()
    f_fwd_head = 4.0 * w.N * w.N * w.d * (0.5 if causal else 1.0)
    f_head = f_fwd_head * (3.5 if backward else 1.0)
    heads, t_total = [], 0.0
    with threadpool_limits(limits=cores):
        while t_total < budget_s and len(heads) < min(max_heads, w.B * w.H):
            b, h = divmod(len(heads), w.H)
            q, k, v = (oracle.bf16_bits_to_f64(x[n][b, h]) for n in ("q", "k", "v"))
            t0 = time.perf_counter()
            oracle.head_forward(q, k, v, causal, w.scale)
            if backward:
                oracle.head_backward(q, k, v, oracle.bf16_bits_to_f64(x["do"][b, h]), causal, w.scale)
            t_total += time.perf_counter() - t0
            heads.append((b, h))
    what = "fwd+bwd" if backward else "fwd"
    return {"value": len(heads) * f_head / t_total / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(heads)} distinct whole heads (b, h) = (0, 0) .. {heads[-1]} of "
                      f"{w.label} causal={causal}, {what} in fp64, {t_total:.1f} s on {cores} "
                      f"BLAS threads; FLOPs counted like the GPU line (the oracle does the full "
                      f"N^2 work)",
            "seconds": round(t_total, 2), "heads": len(heads)}


def cpu_baseline(w, causal, x, budget_s=15.0):
    """The oracle on a bounded sample of the timed workload (fwd + bwd)."""
    r = oracle_rate(w, causal, x, backward=True, budget_s=budget_s)
    r.pop("seconds")
    r.pop("heads")
    return r


def device_inputs(w, dtype="bf16", hkv=None):
    """Seeded inputs of workload w (with dO), as host bits and as device tensors."""
    import numpy as np
    import torch
    import attn_inputs as ai
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v,
                    with_do=True, dtype=dtype, Hkv=hkv or w.H)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = {n: torch.from_numpy(x[n].view(np.int16)).view(tdt).to("cuda:0") for n in x}
    return x, t


def time_launches(fa, w, t, causal, steps, warmup, backward=True):
    """Per-launch HIP-event times (ms) of fa_fwd and fa_bwd over `steps` steps
    (after `warmup` untimed ones), on the stream they are launched on, and the
    wall time per step."""
    import numpy as np
    import torch
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(q.device)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.forward(q, k, v, causal, w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        if backward:
            fa.backward(do, q, k, v, o, lse, causal, w.scale, dq=dq, dk=dk, dv=dv)
            if ev is not None:
                ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs] if backward else [0.0]
    return fwd_ms, bwd_ms, wall * 1e3 / steps, (o, lse)


def all_workloads(args):
    """One JSON line per workload and causal mode: fa_fwd and fa_bwd times,
    TFLOP/s, % of the bf16 peak, algorithmic HBM GB/s, and the oracle's rate on
    a bounded sample of the same inputs."""
    import numpy as np
    import torch
    import attn_inputs as ai
    import exact_tiled_attention_17_amd as fa
    torch.cuda.set_device(0)
    rows = []
    for wname in ("c1", "c2", "c3", "c4", "c5"):
        w = ai.WORKLOADS[wname]
        x, t = device_inputs(w)
        for causal in w.causal_modes:
            fwd_ms, bwd_ms, step_ms, _ = time_launches(fa, w, t, causal, args.steps, args.warmup)
            f_fwd, f_bwd = flops(w, causal)
            b_fwd, b_bwd = alg_bytes(w)
            tf, tb = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
            r = {"workload": wname, "shape": w.label, "causal": causal,
                 "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4), "step_ms": round(tf + tb, 4),
                 "fwd_ms_stats": time_stats(fwd_ms), "bwd_ms_stats": time_stats(bwd_ms),
                 "fwd_tflops": round(f_fwd / tf / 1e9, 1),
                 "bwd_tflops": round(f_bwd / tb / 1e9, 1),
                 "step_tflops": round((f_fwd + f_bwd) / (tf + tb) / 1e9, 1),
                 "fwd_pct_peak": round(100 * f_fwd / tf / 1e9 / PEAK_BF16_TFLOPS, 2),
                 "step_pct_peak": round(100 * (f_fwd + f_bwd) / (tf + tb) / 1e9 / PEAK_BF16_TFLOPS, 2),
                 "fwd_alg_hbm_gbs": round(b_fwd / tf / 1e6, 1),
                 "bwd_alg_hbm_gbs": round(b_bwd / tb / 1e6, 1),
                 "page_context_ms": PAGE_TIMES_MS.get(w.label)}
            if not args.no_cpu_baseline:
                budget = 6.0
                r["oracle_fwd"] = oracle_rate(w, causal, x, backward=False, budget_s=budget)
                r["oracle_fwd_bwd"] = oracle_rate(w, causal, x, backward=True, budget_s=budget)
            rows.append(r)
            print(json.dumps(r), flush=True)
        del x, t
        torch.cuda.empty_cache()
    if args.report_md:
        with open(args.report_md, "w") as f:
            f.write(workload_table(rows, args))
    return rows


def workload_table(rows, args):
    """Markdown table of all_workloads' rows."""
    out = ["| workload | B×H×N×d | causal | fa_fwd ms | fwd TFLOP/s (% peak) | fa_bwd ms | "
           "step TFLOP/s (% peak) | fwd / bwd alg. HBM GB/s | oracle fwd / fwd+bwd GFLOP/s "
           "(heads, cores) | page ms |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        orc = "—"
        if "oracle_fwd" in r:
            a, b = r["oracle_fwd"], r["oracle_fwd_bwd"]
            orc = (f"{a['value'] * 1e3:.1f} ({a['heads']}) / {b['value'] * 1e3:.1f} ({b['heads']}), "
                   f"{a['cores']} cores")
        out.append(f"| {r['workload']} | {r['shape']} | {r['causal']} | {r['fwd_ms']:.4f} | "
                   f"{r['fwd_tflops']:.0f} ({r['fwd_pct_peak']:.1f}%) | {r['bwd_ms']:.4f} | "
                   f"{r['step_tflops']:.0f} ({r['step_pct_peak']:.1f}%) | "
                   f"{r['fwd_alg_hbm_gbs']:.0f} / {r['bwd_alg_hbm_gbs']:.0f} | {orc} | "
                   f"{r['page_context_ms']} |")
    return "\n".join(out) + "\n"


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
    ap.add_argument("--all-workloads", action="store_true",
                    help="time all five workloads (one JSON line each) instead of the step line")
    ap.add_argument("--report-md", default="", help="with --all-workloads: also write a markdown table")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every (batch, head) "
              "is independent, so N GPUs would each run this same kernel on B*H/N heads.",
              file=sys.stderr)
        sys.exit(2)

    if args.all_workloads:
        all_workloads(args)
        return

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
    x, t = device_inputs(w, args.dtype, hkv)
    if not default_launch or args.no_cpu_baseline:
        del x  # the host bits serve only the CPU baseline
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    stream = torch.cuda.current_stream(dev)
    if args.copy_probe_mib > 0:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    fwd_ms, bwd_ms, ms_step, (o, lse) = time_launches(fa, w, t, causal, args.steps, args.warmup,
                                                      backward=not args.fwd_only)

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
    # the FP8 forwards (Q, K quantised per 16 x 16 block, or per 1 x 32 block), bf16 only
    fp8_ms = mx_ms = None
    if args.dtype == "bf16":
        o8 = torch.empty_like(q)
        l8 = torch.empty_like(lse)

        def time_fwd8(fn):
            fn(q, k, v, causal, w.scale, out=o8, lse=l8)
            fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for e0, e1 in fev:
                e0.record(stream)
                fn(q, k, v, causal, w.scale, out=o8, lse=l8)
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([e0.elapsed_time(e1) for e0, e1 in fev]))

        fp8_ms = time_fwd8(fa.forward_fp8)
        mx_ms = time_fwd8(fa.forward_mxfp8)
        del o8, l8

    f_fwd, f_bwd = flops(w, causal)
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
    # half its FLOPs (S = Q K^T) run on the FP8 matrix instruction (5.0 PFLOP/s dense), half
    # (P V) on bf16 (2.5): the peak of that mix is 1 / (0.5 / 5.0 + 0.5 / 2.5) PFLOP/s
    r_mx = None
    if mx_ms is not None:
        r_mx = roof("fa_fwd_mxfp8", "quant_mx_kernel (K) + fwd_kernel (S on the scaled FP8 "
                    "instruction)", f_fwd, mx_ms)
        r_mx["peak"] = PEAK_MX_MIX_TFLOPS
        r_mx["frac"] = round(r_mx["achieved"] / PEAK_MX_MIX_TFLOPS, 4)
        r_mx["peak_note"] = ("S = Q K^T at the dense FP8 peak (5000 TFLOP/s), P V at the bf16 "
                             "peak (2500): equal FLOPs, so 1 / (0.5 / 5000 + 0.5 / 2500)")

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
        "roofline_fwd_mxfp8": r_mx,
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
        out["cpu_baseline"] = cpu_baseline(w, causal, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
