"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--head-dim D] [--dtype bf16|f16] [--pass fwd|bwd]
                    [--no-cpu-baseline] [--copy-calibration MIB]

A step is one attn_fwd call over the whole workload (every query row of every
(batch, head)) with inputs already resident in HBM. The default workload is
the non-causal d=128, N=4096 one (B=16, H=16) that the throughput target is
quoted on. --head-dim and --dtype keep the workload's B, H, N and causality
and change the head dimension (32, 64, 96, 128, 256) or the element type (float16
goes through attn_fwd_ex); the workload name then carries the change. Prints
ONE JSON line on stdout; diagnostics go to stderr.

--pass bwd times attn_bwd instead (dq, dk, dv from o, lse of one forward
call made before timing, and a seeded upstream gradient); its FLOP count is
2.5x the forward's (five products of the same size as the forward's two:
the score recomputation, dP, dV, dQ, dK), halved when causal, and its
roofline covers the whole call (two kernels).

FLOP per step follow the metric: 4*B*H*N^2*d, halved when causal.
roofline.achieved = FLOP per launch / average launch duration, the duration
taken with HIP events on the stream the kernel is launched on. Peak is the
MI355X dense bf16 (and fp16) MFMA figure, 2516.6 TFLOP/s (256 CU x 4096
FLOP/clk x 2.4 GHz). roofline.traffic (HBM bytes per launch) comes from the rocprofv3
FETCH_SIZE / WRITE_SIZE summary committed under profiles/, and is null when
that summary was taken on a different kernel source.

The line also carries the median and minimum of 20 separately timed launches,
and the peak re-derived from rocminfo (CUs x 4096 FLOP/clk x max engine
clock) next to the nominal figure.

--copy-calibration MIB runs only a plain device-to-device copy of that many
MiB (the known-size reference for the FETCH_SIZE / WRITE_SIZE counters) and
prints its size as JSON.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import dataclasses
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "b16h16n4096d128"
PKG = os.path.join(ROOT, "tiled_attention_forward_02_amd")
# The files each timed pass is built from, its compile flags included (hashed
# to tie profiles to code).
KERNEL_SRCS = {"fwd": ("csrc/attn_fwd.hip", "csrc/common.h", "build.py"),
               "bwd": ("csrc/attn_bwd.hip", "csrc/attn_bwd_kernels.h", "csrc/attn_bwd256.hip",
                       "csrc/common.h", "build.py")}
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_text(name, raw):
    """Source text with comments and blank lines dropped (C++ `//` comments in
    the HIP sources, `#` comment lines in build.py), so that editing a comment
    does not mark the profiles taken on that code as stale."""
    text = raw.decode()
    if name.endswith(".py"):
        lines = [l for l in text.splitlines() if not l.lstrip().startswith("#")]
    else:
        lines = [re.sub(r"//.*$", "", l) for l in text.splitlines()]
    return "\n".join(l.rstrip() for l in lines if l.strip()).encode()


def kernel_sha(which="fwd"):
    """Hash of the code each timed pass is built from (comments excluded)."""
    h = hashlib.sha256()
    for name in KERNEL_SRCS[which]:
        with open(os.path.join(PKG, name), "rb") as f:
            h.update(_code_text(name, f.read()))
    return h.hexdigest()[:16]


def stored_traffic(workload, which="fwd"):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing or was taken on another version of the kernel source."""
    path = os.path.join(PROFILES, f"attn_{which}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != kernel_sha(which):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, inp, budget_s=15.0, backward=False):
    """Time the fp64 oracle on whole heads of the same workload until about
    budget_s seconds of CPU work are done; report it in the metric's unit
    (backward: the oracle's gradients, on the backward's FLOP count)."""
    import torch

    from oracle import attend_head, attend_head_grad
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: numpy's BLAS threads unknown
        threads = os.cpu_count() or 1
    q, k, v = inp["q"], inp["k"], inp["v"]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    for b, h in heads:
        if backward:
            attend_head_grad(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(inp["do"][b, h]),
                             inp["scale"], w.causal)
        else:
            attend_head(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), inp["scale"], w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = done * (10.0 if backward else 4.0) * w.N * w.N * w.d / (2 if w.causal else 1)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads (N={w.N}, d={w.d}, "
                  f"causal={w.causal}){' gradients' if backward else ''} in {dt:.1f} s, "
                  f"numpy fp64, metric FLOP of those heads / wall time",
    }


def parity_sample(w, inp, o, lse, rows=16):
    """A quick sampled check against the oracle before timing."""
    import numpy as np
    import torch

    from oracle import attend_head
    rng = np.random.default_rng(7)
    eo = el = 0.0
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        r = np.sort(rng.choice(w.N, rows, replace=False))
        o_ref, l_ref = attend_head(inp["q"][b, h][r].to(torch.float64).numpy(),
                                   inp["k"][b, h].to(torch.float64).numpy(),
                                   inp["v"][b, h].to(torch.float64).numpy(),
                                   inp["scale"], w.causal, q_pos=r)
        eo = max(eo, float(np.abs(o[b, h][r] - o_ref).max()))
        el = max(el, float(np.abs(lse[b, h][r] - l_ref).max()))
    return {"max_abs_dO": eo, "max_abs_dlse": el, "ok": eo <= 2e-2 and el <= 1e-3}


def parity_sample_bwd(w, inp, dq, rows=16):
    """Sampled dq rows against the oracle (a row's dq needs only its own
    weights) before timing the backward."""
    import numpy as np
    import torch

    from oracle import attend_head_grad
    rng = np.random.default_rng(8)
    worst = 0.0
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        r = np.sort(rng.choice(w.N, rows, replace=False))
        ref, _, _ = attend_head_grad(f64(inp["q"][b, h][r]), f64(inp["k"][b, h]),
                                     f64(inp["v"][b, h]), f64(inp["do"][b, h][r]),
                                     inp["scale"], w.causal, q_pos=r)
        worst = max(worst, float(np.abs(dq[b, h][r] - ref).max() / np.abs(ref).max()))
    return {"max_abs_ddq_over_max_ref": worst, "ok": worst <= 2e-2}


def device_peak():
    """CUs and max engine clock of the gfx950 agent from rocminfo, and the dense
    bf16 MFMA peak they give (4096 FLOP per CU per clock). Runs rocminfo as a
    child process, so it must be called before this process touches the GPU.
    None if rocminfo is unavailable."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for block in out.split("Agent ")[1:]:
        if "gfx950" not in block:
            continue
        cus = re.search(r"Compute Unit:\s+(\d+)", block)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
        if cus and mhz:
            c, m = int(cus.group(1)), int(mhz.group(1))
            return {"compute_units": c, "max_sclk_mhz": m,
                    "bf16_tflops": round(c * 4096 * m * 1e6 / 1e12, 1)}
    return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 32, 64, 96, 128, 256])
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"])
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    peak_check = None
    if args.gpus == 1 and world == 1 and not args.copy_calibration:
        peak_check = device_peak()  # before anything touches the GPU
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention forward is built and "
              "measured on a single MI355X (each head is independent; sharding "
              "heads over GPUs needs no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_attention_forward_02_amd as mi
    from tiled_attention_forward_02_amd.workloads import attn_flops, make_inputs, workload

    if not torch.cuda.is_available():
        log("no HIP device visible")
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    w = workload(args.workload)
    if args.head_dim and args.head_dim != w.d:
        w = dataclasses.replace(w, d=args.head_dim,
                                name=re.sub(r"d\d+$", f"d{args.head_dim}", w.name))
    elem = torch.bfloat16
    if args.dtype == "f16":
        w = dataclasses.replace(w, name=w.name + "_f16")
        elem = torch.float16
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} {args.dtype}")
    inp = make_inputs(w, dtype=elem)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    shape = mi.attn_fwd_launch_shape(w.B, w.H, w.N, w.d, w.causal)
    log(f"launch: {shape}")

    fwd = mi.attn_fwd if args.dtype == "bf16" else mi.attn_fwd_ex
    backward = args.which == "bwd"

    def step():
        fwd(q, k, v, scale=inp["scale"], causal=w.causal, out=o, lse=lse)

    step()
    torch.cuda.synchronize()
    if backward:
        # o, lse of the forward above are the backward's inputs from here on.
        g = torch.Generator("cpu").manual_seed(w.seed + 1000)
        inp["do"] = torch.randn(q.shape, generator=g, dtype=torch.float32).to(elem)
        do = inp["do"].to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
        w = dataclasses.replace(w, name=w.name + "_bwd")

        def step():  # noqa: F811
            mi.attn_bwd(q, k, v, o, lse, do, scale=inp["scale"], causal=w.causal, dq=dq, dk=dk,
                        dv=dv, delta=delta)

        step()
        torch.cuda.synchronize()
        parity = parity_sample_bwd(w, inp, dq.float().cpu().numpy())
    else:
        parity = parity_sample(w, inp, o.float().cpu().numpy(), lse.cpu().numpy())
    log(f"parity sample: {parity}")
    if not parity["ok"]:
        log("parity check failed; refusing to report a throughput")
        sys.exit(1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = ev0.elapsed_time(ev1)
    # Per-launch times, each launch between its own pair of events.
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_us = sorted(a.elapsed_time(b) * 1e3 for a, b in per)

    flops = attn_flops(w.B, w.H, w.N, w.d, w.causal) * (2.5 if backward else 1.0)
    launch_s = event_ms / 1e3 / args.steps
    achieved = flops / launch_s / 1e12
    value = flops * args.steps / wall / 1e12
    traffic = stored_traffic(w.name, args.which)
    log(f"wall {wall*1e3:.2f} ms for {args.steps} steps; event avg {launch_s*1e6:.1f} us/launch")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        cpu = cpu_baseline(w, inp, args.cpu_budget, backward=backward)

    metric = "attention fwd TFLOP/s and % of MI355X bf16 MFMA peak at d=64/128"
    if backward:
        metric = "attention bwd TFLOP/s (2.5x the forward's FLOP) and % of MI355X bf16 MFMA peak"
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": w.as_dict(),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernel_avg_us": round(launch_s * 1e6, 2),
        "launch_us_median": round(per_us[len(per_us) // 2], 2),
        "launch_us_min": round(per_us[0], 2),
        "peak_check": peak_check,
        "parity_sample": parity,
        "kernel_source_sha256_16": kernel_sha(args.which),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
