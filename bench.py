"""Throughput of the In-Place TTT gated-MLP prefill layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--schedule prefix|running] [--no-cpu-baseline]
                    [--variant plain|packed|clipped|packed_clipped|continue|decode|
                               backward|train]
    python bench.py --summarize DIR [--fetch DIR2 --write DIR3]
                    --summary-out FILE.md --command "..."
    python bench.py --vendor-gemm

The third form times torch.matmul (hipBLASLt) on the plain GEMM shapes of
the layer's four contractions, as a vendor-library reference point (run
only). The second form turns rocprofv3 output (a --kernel-trace --stats run, and
optionally --pmc FETCH_SIZE / WRITE_SIZE runs) of the first form into the
text summaries kept under profiles/.

One step is one call of ttt_layer_forward on the whole workload (gate/up,
target, update with per-chunk snapshots, apply), with inputs resident in HBM.
--variant times the other entry points on the same workload instead: packed
(ttt_layer_forward_packed, the sequence cut into --docs equal documents),
clipped (ttt_layer_forward_clipped, limit --clip), packed_clipped
(ttt_layer_forward_packed_clipped: both at once), continue
(ttt_layer_forward_continue: an fp32 state updated in place and K - 1
look-ahead rows), decode (ttt_decode_step token by token with chunk-local
padding; one step is one chunk of C tokens, the chunk's update included) or
backward (ttt_layer_backward: every gradient of the prefill for a random
upstream dO and dW_final, the forward's activations recomputed inside) or
train (a training step: ttt_layer_forward_train, whose workspace keeps the
activations, then ttt_layer_backward_saved on it).
Prints one JSON line: tokens/s for the step, the per-kernel device times
(HIP events recorded by the library around each launch, on the stream it
launches on), the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same workload. The K timed steps run twice: the
first pass, with no events around the launches, gives the step time and
tokens/s; the second, the same K steps with the library's events around
every launch, gives the per-kernel times (events between launches lengthen
a step of short kernels, such as a decode step's).
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
KERNEL_SRC_DIR = os.path.join(ROOT, "test_layer_gate_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CALIB_BYTES = 256 << 20      # the known-size copy run before the timed region
# library timing names -> kernel names in rocprofv3 traces
KERNEL_NAMES = {"gate_up": "gate_up_kernel", "target": "target_kernel",
                "gate_up_target": "gate_up_target_kernel",
                "update_prefix": "update_kernel", "update_running": "update_kernel",
                "apply": "apply_kernel", "conv": "conv_kernel",
                "transpose_w_target": "transpose_kernel", "cast_bf16": "cast_kernel",
                "pack_weights": "pack_weight_kernel",
                "calibration_copy": "calibration_copy_kernel",
                "range_clear": "range_clear_kernel", "amax": "amax_kernel",
                "conv_repair": "conv_repair_kernel", "gate_up_repair": "gate_up_repair_kernel",
                "target_repair": "target_repair_kernel",
                "bwd_gate_up": "gate_up_bwd_kernel", "bwd_target": "target_bwd_kernel",
                "bwd_states": "update_kernel", "bwd_state_grads": "update_kernel",
                "bwd_dz": "dz_gemm_kernel", "bwd_dv": "dv_gemm_kernel",
                "bwd_dy": "nt_gemm_kernel", "bwd_dh": "nt_gemm_kernel",
                "bwd_dw_target": "update_kernel", "bwd_dw_gate_up": "update_kernel",
                "bwd_conv": "conv_bwd", "bwd_rows": "rows_bf16_kernel",
                "bwd_to_slab": "to_slab_kernel",
                "bwd_transpose_w": "transpose_bf16_kernel", "bwd_sum": "sum_parts_kernel"}


def backward_flops(cfg):
    """Contraction FLOPs (2 per multiply-add) that one ttt_layer_backward
    call executes: the recomputed gate/up (4 B T d f) and target (2 B T d^2),
    the scans for the states and the state gradients (2 B T d f each), dZ
    (4 B T d f: two products side by side), dV (2 B T d f), dY and dW_target
    (2 B T d^2 each), dWg and dWu (4 B T d f) and dH (4 B T d f)."""
    B, T, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    return 22.0 * B * T * d * f + 6.0 * B * T * d * d


def train_flops(cfg):
    """A training step's contraction FLOPs: the prefill (8 B T d f + 2 B T
    d^2) and the saved backward, which skips the gate/up recompute (4 B T d
    f) and the state scan (2 B T d f)."""
    B, T, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    return synth.algorithmic_flops(cfg) + backward_flops(cfg) - 6.0 * B * T * d * f


def kernel_work(name, cfg, T_pad):
    """(bound, algorithmic amount per step) of each kernel of one step:
    FLOPs of the contraction (2 per multiply-add) for MFMA kernels, bytes
    moved once for the bandwidth-bound ones. A kernel launched several times
    per step (the running schedule's per-chunk apply and update) shares the
    amount over its launches."""
    B, T, d, f, K = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.conv_k
    if name == "gate_up":
        return "mfma", 4.0 * B * T * d * f
    if name == "target":
        return "mfma", 2.0 * B * T * d * d
    if name == "gate_up_target":  # both in one launch, where that saves a round
        return "mfma", 4.0 * B * T * d * f + 2.0 * B * T * d * d
    if name in ("update_prefix", "update_running", "apply"):
        return "mfma", 2.0 * B * T * d * f
    if name in ("bwd_gate_up", "bwd_dz", "bwd_dw_gate_up", "bwd_dh"):
        return "mfma", 4.0 * B * T * d * f
    if name in ("bwd_states", "bwd_state_grads", "bwd_dv"):
        return "mfma", 2.0 * B * T * d * f
    if name in ("bwd_target", "bwd_dy", "bwd_dw_target"):
        return "mfma", 2.0 * B * T * d * d
    if name == "conv":
        return "hbm", 2.0 * B * T * d + 2.0 * B * T_pad * d + 2.0 * K * d
    if name == "transpose_w_target":
        return "hbm", 4.0 * d * d
    if name == "pack_weights":  # one of W_g / W_u per launch: read d*f, write the packed copy
        return "hbm", 2.0 * d * f + 2.0 * d * (-(-f // 128) * 128)
    # decode, one launch per token, C tokens per step: W_g and W_u read once
    # per token; each state's bf16 copy read once per token
    if name == "decode_gate_up":
        return "hbm", cfg.chunk * (2.0 * 2 * f * d + B * (4.0 * d + 4.0 * f))
    if name == "decode_apply":
        return "hbm", cfg.chunk * B * (2.0 * d * f + 2.0 * f + 2.0 * d)
    return None, None


def source_hash():
    """sha256[:16] over the kernel sources (.hip and .h files, by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_key(workload, variant):
    return workload if variant == "plain" else f"{workload}/{variant}"


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the kernel source as it is now and the kernel's
    name in the trace belongs to this one timing name of the step."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None
    ent = rec.get("kernels", {}).get(workload, {}).get(kernel)
    if ent is None or ent.get("shared_name"):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, x, budget_s=15.0, variant="plain", clip=None, doc_len=None):
    """The float64 oracle on the first j chunks of the workload (plus the
    conv's K-1 look-ahead rows), j chosen so the sample takes ~budget_s.
    For the packed variant the sample is the first j chunks' worth of whole
    documents, run through the packed oracle; for the clipped one the oracle
    clips; a continued segment is the plain recurrence from a given state."""
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
        if variant in ("backward", "train"):
            B, T, d = x["H"].shape
            if variant == "train":   # the step's forward, then its backward
                ora.ttt_prefill(x["H"][:1, :n], x["X0"][:1, :n], x["Wg"], x["Wu"],
                                x["W_down0"], x["taps"], x["W_target"], cfg.eta, C)
            dO = np.random.default_rng(1).standard_normal((1, n, d))
            dWf = np.random.default_rng(2).standard_normal((1, d, x["Wg"].shape[0]))
            ora.ttt_prefill_backward(x["H"][:1, :n], x["X0"][:1, :n], x["Wg"], x["Wu"],
                                     x["W_down0"], x["taps"], x["W_target"], cfg.eta, C, dO,
                                     dW_final=dWf)
        elif variant == "decode":
            ora.ttt_decode(x["H"][:1, :n], x["X0"][:1, :n], x["Wg"], x["Wu"], x["W_down0"],
                           x["taps"], x["W_target"], cfg.eta, C)
        elif variant in ("packed", "packed_clipped"):
            n = max(doc_len, n // doc_len * doc_len)
            ora.ttt_prefill_packed(x["H"][0, :n], x["X0"][0, :n], x["Wg"], x["Wu"],
                                   x["W_down0"], x["taps"], x["W_target"], cfg.eta, C,
                                   list(range(0, n, doc_len)),
                                   clip=clip if variant == "packed_clipped" else None)
        else:
            ora.ttt_prefill(x["H"][:1, :n], x["X0"][:1, :n + K - 1], x["Wg"], x["Wu"],
                            x["W_down0"], x["taps"], x["W_target"], cfg.eta, C,
                            clip=clip if variant == "clipped" else None)
        return time.perf_counter() - t0

    t1 = run(1)
    j = int(max(2, min(cfg.n_chunks, budget_s / max(t1, 1e-3))))
    tj = run(j)
    return {"value": round(j * C / tj, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle on the first {j} of {cfg.n_chunks} chunks "
                      f"({j * C} tokens, batch row 0) of {cfg.name}; {tj:.1f} s"}


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[-1]


N_XCD, SIMD_NUM = 8, 1024      # MI355X: GRBM counters sum over the 8 XCDs; 256 CUs x 4 SIMDs


def mfma_section(args):
    """MFMA utilisation per MFMA kernel from the counter run's last dispatch
    of each: SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of the dispatch
    (GRBM_GUI_ACTIVE per XCD x SIMD_NUM), the clock those cycles imply over
    the dispatch's duration, and the MFMA work (MOPS x 512 FLOPs)."""
    last = {}
    for r in _read_csv(_find(args.mfma, "counter_collection.csv")):
        key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
        e = last.setdefault(key, {"dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    per = {}
    for (name, disp), e in sorted(last.items(), key=lambda kv: kv[0][1]):
        if e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) > 0:
            per[name] = e                     # the later dispatch wins
    out = ["", "## MFMA utilisation (rocprofv3 --pmc)", "",
           f"Command: `{args.mfma_command}`", "",
           "Busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); the "
           "clock is GRBM_GUI_ACTIVE / 8 over the dispatch's duration; FLOPs = MFMA MOPS x 512. "
           "Last dispatch of each kernel (a timed step).", "",
           "| kernel | ms | MFMA busy | clock GHz | MFMA TFLOP | TFLOP/s | of 2.5 PF at 2.4 GHz | of peak at that clock |",
           "|---|---|---|---|---|---|---|---|"]
    for name, e in per.items():
        cyc = e["GRBM_GUI_ACTIVE"] / N_XCD
        busy = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMD_NUM)
        clk = cyc / (e["dur"] * 1e-9) / 1e9
        flops = (e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) +
                 e.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)) * 512
        tfs = flops / (e["dur"] * 1e-9) / 1e12
        out.append(f"| {name} | {e['dur'] / 1e6:.3f} | {busy * 100:.1f}% | {clk:.2f} | "
                   f"{flops / 1e12:.3f} | {tfs:.0f} | {tfs / PEAK_BF16_TFLOPS * 100:.1f}% | "
                   f"{tfs / (PEAK_BF16_TFLOPS * clk / 2.4) * 100:.1f}% |")
    return out


def summarize(args):
    """Write a markdown summary of rocprofv3 results (and, with --fetch and
    --write, the per-launch HBM traffic record used by the bench line)."""
    stats = _read_csv(_find(args.summarize, "kernel_stats.csv"))
    # Per-dispatch durations, to average the timed steps alone: the profiled
    # command runs prof_warmup + 2 x prof_steps steps of the same launches.
    durs = {}
    for r in _read_csv(_find(args.summarize, "kernel_trace.csv")):
        durs.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    # bench.py runs warm-up steps, then the timed steps twice (without and
    # with the library's per-launch events)
    n_steps = 2 * args.prof_steps + args.prof_warmup
    lines = [f"# rocprofv3 kernel summary: {args.title}", "",
             f"Command: `{args.command}`", "",
             f"Kernel source sha256[:16]: `{source_hash()}`", "",
             f"\"timed avg\" leaves out the dispatches of the {args.prof_warmup} warm-up "
             f"step(s) (kernels launched once per step of the {n_steps}).", "",
             "| kernel | calls | avg us | timed avg us | min us | max us | total ms | share |",
             "|---|---|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        d = [x[1] for x in sorted(durs.get(r["Name"], []))]
        timed = "-"
        if d and len(d) % n_steps == 0:
            per = len(d) // n_steps
            rest = d[per * args.prof_warmup:]
            timed = f"{sum(rest) / len(rest) / 1e3:.1f}"
        lines.append("| {} | {} | {:.1f} | {} | {:.1f} | {:.1f} | {:.3f} | {:.1f}% |".format(
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, timed,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    if args.fetch and args.write:
        per = {}
        for which, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
            for r in _read_csv(_find(d, "counter_collection.csv")):
                if r["Counter_Name"] != which:
                    continue
                per.setdefault(r["Kernel_Name"], {}).setdefault(which, []).append(
                    float(r["Counter_Value"]) * 1024.0)
        cal = per.get("calibration_copy_kernel")
        if not cal:
            raise SystemExit("no calibration_copy_kernel dispatch in the counter runs")
        f_fac = CALIB_BYTES / (sum(cal["FETCH_SIZE"]) / len(cal["FETCH_SIZE"]))
        w_fac = CALIB_BYTES / (sum(cal["WRITE_SIZE"]) / len(cal["WRITE_SIZE"]))
        lines += ["", "## HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)", "",
                  f"Fetch command: `{args.fetch_command}`", "",
                  f"Write command: `{args.write_command}`", "",
                  f"Calibration: calibration_copy_kernel moves {CALIB_BYTES} bytes each way; "
                  f"counter-to-byte factors: fetch {f_fac:.4f}, write {w_fac:.4f}.", "",
                  "| kernel | dispatches | fetch MB | write MB | HBM MB (scaled) |",
                  "|---|---|---|---|---|"]
        # One record per kernel source; each workload (and variant) keeps its
        # own entry, so profiling one does not drop another's.
        key = traffic_key(args.workload, args.variant)
        rec = {}
        try:
            with open(TRAFFIC_FILE) as fh:
                rec = json.load(fh)
        except (OSError, ValueError):
            pass
        if rec.get("kernel_source_sha256_16") != source_hash():
            rec = {"kernel_source_sha256_16": source_hash(), "kernels": {}}
        rec.pop("workload", None)
        rec.setdefault("factors", {})[key] = {"fetch": f_fac, "write": w_fac}
        rec.pop("fetch_factor", None)
        rec.pop("write_factor", None)
        rec["kernels"][key] = {}
        names_in_step = [n for n in KERNEL_NAMES
                         if args.variant == "train" or
                         n.startswith("bwd_") == (args.variant == "backward")]
        for name, v in sorted(per.items()):
            fe = sum(v.get("FETCH_SIZE", [0])) / max(len(v.get("FETCH_SIZE", [])), 1)
            wr = sum(v.get("WRITE_SIZE", [0])) / max(len(v.get("WRITE_SIZE", [])), 1)
            tot = fe * f_fac + wr * w_fac
            lines.append(f"| {name} | {len(v.get('FETCH_SIZE', []))} | {fe / 1e6:.1f} | "
                         f"{wr / 1e6:.1f} | {tot / 1e6:.1f} |")
            sharing = [n for n in names_in_step if KERNEL_NAMES[n] == name]
            for lib_name in sharing:
                rec["kernels"][key][lib_name] = {
                    "hbm_bytes_per_launch": tot, "fetch_bytes": fe * f_fac,
                    "write_bytes": wr * w_fac, "shared_name": len(sharing) > 1}
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(rec, fh, indent=1)
    if args.mfma:
        lines += mfma_section(args)
    os.makedirs(os.path.dirname(args.summary_out) or ".", exist_ok=True)
    with open(args.summary_out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def vendor_gemm(cfg):
    """torch.matmul (hipBLASLt) on the plain GEMMs with the layer's shapes
    (bf16, fp32 accumulation): gate/up as one [T, d] x [2f, d]^T product, the
    target, the apply with one weight for all chunks, and the update over
    all tokens. Context only: the layer's kernels also fuse SiLU, write Z in
    two layouts, read one state per chunk and store the snapshots."""
    import torch
    T, d, f = cfg.batch * cfg.seq_len, cfg.d_model, cfg.d_ff
    out = {}
    for name, M, N, K in [("gate_up", T, 2 * f, d), ("target", T, d, d), ("apply", T, d, f),
                          ("update", f, d, T)]:
        A = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        B = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        for _ in range(2):
            torch.matmul(A, B.t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(A, B.t())
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4),
                     "tflops": round(2.0 * M * N * K / ms / 1e9, 1)}
        del A, B
    print(json.dumps({"vendor_gemm": "torch.matmul (hipBLASLt), bf16", "workload": cfg.name,
                      "shapes": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=synth.BENCH_CONFIG, choices=sorted(synth.CONFIGS))
    ap.add_argument("--schedule", default="prefix", choices=["prefix", "running"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", default="plain",
                    choices=["plain", "packed", "clipped", "packed_clipped", "continue",
                             "decode", "backward", "train"])
    ap.add_argument("--docs", type=int, default=32, help="packed variant: equal documents")
    ap.add_argument("--clip", type=float, default=1e-3, help="clipped variant: norm limit")
    ap.add_argument("--summarize", help="rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output directory")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output directory")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time torch.matmul on the layer's GEMM shapes instead")
    ap.add_argument("--mfma", help="rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                                   "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 "
                                   "output directory")
    ap.add_argument("--mfma-command", default="")
    ap.add_argument("--summary-out")
    ap.add_argument("--prof-steps", type=int, default=5, help="--steps of the profiled command")
    ap.add_argument("--prof-warmup", type=int, default=1, help="--warmup of the profiled command")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    ap.add_argument("--fetch-command", default="")
    ap.add_argument("--write-command", default="")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    cfg = synth.CONFIGS[args.workload]
    if args.vendor_gemm:
        vendor_gemm(cfg)
        return

    import torch
    import test_layer_gate_amd as ttt

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
    doc_len = None
    if args.variant == "decode":
        if (args.warmup + 2 * args.steps) * cfg.chunk > T:
            raise SystemExit("--variant decode: (warmup + 2 x steps) chunks must fit the workload")
        ddesc = ttt.make_desc(B, 1, d, f, cfg.conv_k, 0 if cfg.dtype == "bf16" else 1,
                              0 if cfg.dtype == "bf16" else 1, 0, 1)
        ws_bytes = ttt.decode_state_size(ddesc, cfg.chunk)
        W_state = t["W_down0"].float().expand(B, d, f).contiguous()
        O_tok = torch.empty((B, d), dtype=t["H"].dtype, device=dev)
        H_tok = t["H"].transpose(0, 1).contiguous()     # [T, B, d]: each token's rows together
        X0_tok = t["X0"].transpose(0, 1).contiguous()
        pos = [0]
    elif args.variant in ("packed", "packed_clipped"):
        if B != 1 or T % args.docs or (T // args.docs) % 64:
            raise SystemExit("--variant packed needs batch 1 and documents of a multiple of 64 tokens")
        doc_len = T // args.docs
        starts = list(range(0, T, doc_len))
        pclip = args.clip if args.variant == "packed_clipped" else None
        ws_bytes = ttt.packed_workspace_size(desc, cfg.chunk, starts, pclip)
    elif args.variant == "clipped":
        ws_bytes = ttt.clipped_workspace_size(desc, cfg.chunk, args.clip)
    elif args.variant == "continue":
        ws_bytes = ttt.continue_workspace_size(desc, cfg.chunk)
        # the segment continues a document: its state is fp32 and K - 1 rows follow it
        W_state = t["W_down0"].float().expand(B, d, f).contiguous()
        X0_next = t["X0"][:, :cfg.conv_k - 1].contiguous()
    elif args.variant in ("backward", "train"):
        ws_bytes = (ttt.backward_workspace_size(desc, cfg.chunk) if args.variant == "backward"
                    else ttt.backward_saved_workspace_size(desc, cfg.chunk))
        saved = (torch.empty(ttt.train_workspace_size(desc, cfg.chunk), dtype=torch.uint8,
                             device=dev) if args.variant == "train" else None)
        gen = torch.Generator(device=dev).manual_seed(5)
        dO = torch.randn(t["H"].shape, generator=gen, device=dev).to(tdt)
        dWf_up = torch.randn((B, d, f), generator=gen, device=dev)
        shapes = {"dH": (B, T, d), "dX0": (B, T, d), "dWg": (f, d), "dWu": (f, d),
                  "dW_down0": (d, f), "dtaps": (cfg.conv_k, d), "dW_target": (d, d)}
        grads = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
    else:
        ws_bytes = ttt.workspace_size(desc, cfg.chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    if args.variant == "decode":
        ttt.decode_begin(W_state, cfg.chunk, ws, act_dtype=t["H"].dtype,
                         weight_dtype=t["Wg"].dtype, conv_k=cfg.conv_k)

    def step():
        if args.variant == "decode":
            for _ in range(cfg.chunk):
                p = pos[0]
                ttt.decode_step(H_tok[p], X0_tok[p], t["Wg"], t["Wu"], t["taps"],
                                t["W_target"], cfg.eta, cfg.chunk, p, W_state, ws, out=O_tok)
                pos[0] = p + 1
        elif args.variant in ("packed", "packed_clipped"):
            ttt.layer_forward_packed(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                                     t["W_target"], cfg.eta, cfg.chunk, starts,
                                     schedule=args.schedule, clip=pclip, out=O, W_down_final=Wf,
                                     workspace=ws)
        elif args.variant in ("backward", "train"):
            if saved is not None:
                ttt.layer_forward_train(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"],
                                        t["taps"], t["W_target"], cfg.eta, cfg.chunk, out=O,
                                        W_down_final=Wf, workspace=saved)
            ttt.layer_backward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                               t["W_target"], cfg.eta, cfg.chunk, dO, dW_final=dWf_up,
                               saved=saved, out=grads, workspace=ws)
        elif args.variant == "continue":
            ttt.layer_forward_continue(t["H"], t["X0"], X0_next, t["Wg"], t["Wu"], W_state,
                                       t["taps"], t["W_target"], cfg.eta, cfg.chunk,
                                       schedule=args.schedule, out=O, workspace=ws)
        else:
            ttt.layer_forward(t["H"], t["X0"], t["Wg"], t["Wu"], t["W_down0"], t["taps"],
                              t["W_target"], cfg.eta, cfg.chunk, schedule=args.schedule,
                              clip=args.clip if args.variant == "clipped" else None,
                              out=O, W_down_final=Wf, workspace=ws)

    # A plain copy of known size, outside the timed region: the reference that
    # converts hardware traffic counters to bytes in profiled runs.
    calib_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    calib_dst = torch.empty_like(calib_src)
    ttt.copy_calibration(calib_dst, calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    dev_ms = ev0.elapsed_time(ev1)
    # the same steps again, with the library's events around every launch
    ttt.profile_enable(True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    prof_ms = ev0.elapsed_time(ev1) / args.steps
    kstats = ttt.profile_read()
    ttt.profile_enable(False)
    ms_per_step = dev_ms / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.3f} s)",
          file=sys.stderr, flush=True)

    tokens = B * (cfg.chunk if args.variant == "decode" else T)
    if args.variant == "backward":
        flops = backward_flops(cfg)
    elif args.variant == "train":
        flops = train_flops(cfg)
    else:
        flops = synth.algorithmic_flops(cfg) * tokens / (B * T)
    value = tokens / (ms_per_step / 1e3)
    tflops = flops / (ms_per_step / 1e3) / 1e12
    kernels = {n: {"launches_per_step": c / args.steps, "avg_ms": ms / c}
               for n, (c, ms) in kstats.items()}
    # the longest-running kernel that has an algorithmic work figure
    dom = max((n for n in kstats if kernel_work(n, cfg, T_pad)[0] is not None),
              key=lambda n: kstats[n][1])
    bound, work = kernel_work(dom, cfg, T_pad)
    launches_per_step = kstats[dom][0] / args.steps
    work = work / launches_per_step          # per launch
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
    roof["traffic"] = measured_traffic(dom, traffic_key(cfg.name, args.variant))

    line = {
        "metric": "TTT-MLP layer prefill tokens/s + MFMA util (Qwen3-4B shape, 64k ctx)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16+fp16", "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "seq_len": T, "chunk": cfg.chunk,
                   "d_model": d, "d_ff": f, "conv_k": cfg.conv_k, "eta": cfg.eta,
                   "schedule": args.schedule, "variant": args.variant},
        "layer_tflops": round(tflops, 1),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels": {n: {k: round(v, 4) for k, v in s.items()} for n, s in kernels.items()},
        "wall_s": round(wall, 3),
        "ms_per_step_with_launch_events": round(prof_ms, 4),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, x, variant=args.variant, clip=args.clip,
                                            doc_len=doc_len)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
