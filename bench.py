"""Throughput of the In-Place TTT gated-MLP prefill layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--schedule prefix|running] [--no-cpu-baseline]

One step is one call of ttt_layer_forward on the whole workload (gate/up,
target, update with per-chunk snapshots, apply), with inputs resident in HBM.
Prints one JSON line: tokens/s for the step, the per-kernel device times
(HIP events recorded by the library around each launch, on the stream it
launches on), the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "test_layer_gate_amd", "csrc", "ttt_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_work(name, cfg, T_pad):
    """(bound, algorithmic amount per launch, unit) of each kernel of one
    step: FLOPs of the contraction (2 per multiply-add) for MFMA kernels,
    bytes moved once for the bandwidth-bound ones."""
    B, T, d, f, K = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.conv_k
    if name == "gate_up":
        return "mfma", 4.0 * B * T * d * f
    if name == "target":
        return "mfma", 2.0 * B * T * d * d
    if name in ("update_prefix", "apply"):
        return "mfma", 2.0 * B * T * d * f
    if name == "conv":
        return "hbm", 2.0 * B * T * d + 2.0 * B * T_pad * d + 2.0 * K * d
    if name == "transpose_w_target":
        return "hbm", 4.0 * d * d
    return None, None


def source_hash():
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the kernel source as it is now."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None
    ent = rec.get("kernels", {}).get(workload, {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, x, budget_s=15.0):
    """The float64 oracle on the first j chunks of the workload (plus the
    conv's K-1 look-ahead rows), j chosen so the sample takes ~budget_s."""
    import oracle.ttt_oracle as ora
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    C, K = cfg.chunk, cfg.conv_k

    def run(j):
        n = j * C
        t0 = time.perf_counter()
        ora.ttt_prefill(x["H"][:1, :n], x["X0"][:1, :n + K - 1], x["Wg"], x["Wu"],
                        x["W_down0"], x["taps"], x["W_target"], cfg.eta, C)
        return time.perf_counter() - t0

    t1 = run(1)
    j = int(max(2, min(cfg.n_chunks, budget_s / max(t1, 1e-3))))
    tj = run(j)
    return {"value": round(j * C / tj, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle on the first {j} of {cfg.n_chunks} chunks "
                      f"({j * C} tokens, batch row 0) of {cfg.name}; {tj:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=synth.BENCH_CONFIG, choices=sorted(synth.CONFIGS))
    ap.add_argument("--schedule", default="prefix", choices=["prefix", "running"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import test_layer_gate_amd as ttt

    cfg = synth.CONFIGS[args.workload]
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    x = synth.make_inputs(cfg)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = {k: torch.from_numpy(v).to(dev).to(tdt) for k, v in x.items()}
    B, T, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    T_pad = -(-T // 256) * 256
    O = torch.empty_like(t["H"])
    Wf = torch.empty((B, d, f), dtype=torch.float32, device=dev)
    desc = ttt.make_desc(B, T, d, f, cfg.conv_k, 0 if cfg.dtype == "bf16" else 1,
                         0 if cfg.dtype == "bf16" else 1, 0,
                         2 if args.schedule == "running" else 4)
    ws = torch.empty(ttt.workspace_size(desc, cfg.chunk), dtype=torch.uint8, device=dev)

    def step():
        ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                          t["W_target"], cfg.eta, cfg.chunk, schedule=args.schedule,
                          out=O, W_down_final=Wf, workspace=ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ttt.profile_enable(True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kstats = ttt.profile_read()
    ttt.profile_enable(False)
    dev_ms = ev0.elapsed_time(ev1)
    ms_per_step = dev_ms / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.3f} s)",
          file=sys.stderr, flush=True)

    tokens = B * T
    flops = synth.algorithmic_flops(cfg)
    value = tokens / (ms_per_step / 1e3)
    tflops = flops / (ms_per_step / 1e3) / 1e12
    kernels = {n: {"launches_per_step": c / args.steps, "avg_ms": ms / c}
               for n, (c, ms) in kstats.items()}
    dom = max(kstats, key=lambda n: kstats[n][1])
    bound, work = kernel_work(dom, cfg, T_pad)
    avg_s = kstats[dom][1] / kstats[dom][0] / 1e3
    if bound == "mfma":
        achieved = work / avg_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = work / avg_s / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(dom, cfg.name)

    line = {
        "metric": "TTT-MLP layer prefill tokens/s + MFMA util (Qwen3-4B shape, 64k ctx)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "seq_len": T, "chunk": cfg.chunk,
                   "d_model": d, "d_ff": f, "conv_k": cfg.conv_k, "eta": cfg.eta,
                   "schedule": args.schedule},
        "layer_tflops": round(tflops, 1),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels": {n: {k: round(v, 4) for k, v in s.items()} for n, s in kernels.items()},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, x)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
