"""CPU checks of bench.py's host logic: the multi-GPU refusal, the
algorithmic work it divides by the measured times, and the rule that a
traffic record is only used for the kernel source it was taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_layer_flops_match_the_method():
    """The MFMA kernels of one step add up to 2*B*T*(4*d*f + d^2): gate/up
    4*B*T*d*f, the target 2*B*T*d^2, the update and the apply 2*B*T*d*f
    each (13.92 TFLOP at the Qwen3-4B 64k shape)."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    B, T, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    total = 0.0
    for k in ("gate_up", "target", "update_prefix", "apply"):
        bound, work = bench.kernel_work(k, cfg, T)
        assert bound == "mfma"
        total += work
    assert total == 2.0 * B * T * (4 * d * f + d * d)
    assert abs(total / 1e12 - 13.92) < 0.01
    # gate/up and the target in one launch count as both
    merged = bench.kernel_work("gate_up_target", cfg, T)
    assert merged == ("mfma", bench.kernel_work("gate_up", cfg, T)[1] +
                      bench.kernel_work("target", cfg, T)[1])


def test_traffic_record_is_tied_to_the_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.source_hash(), "workload": "w",
           "kernels": {"w": {"gate_up": {"hbm_bytes_per_launch": 123.0}}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic("gate_up", "w") == 123.0
    rec["kernel_source_sha256_16"] = "0" * 16
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("gate_up", "w") is None



def test_backward_flops_match_its_kernels():
    """The backward's kernels add up to the contractions it executes:
    22*B*T*d*f + 6*B*T*d^2 (the recomputed gate/up and target, the state
    and state-gradient scans, dZ over K = 2d, dV, dY, dW_target, dWg + dWu
    and dH)."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    total = 0.0
    for k in ("bwd_gate_up", "bwd_target", "bwd_states", "bwd_state_grads", "bwd_dz", "bwd_dv",
              "bwd_dy", "bwd_dw_target", "bwd_dw_gate_up", "bwd_dh"):
        bound, work = bench.kernel_work(k, cfg, cfg.seq_len)
        assert bound == "mfma", k
        total += work
    assert total == bench.backward_flops(cfg)


def test_traffic_of_a_shared_kernel_name_is_not_used(tmp_path, monkeypatch):
    """Timing names whose kernels share one trace name (the backward's
    update-kernel contractions) get no traffic figure: the counters cannot
    tell their launches apart."""
    rec = {"kernel_source_sha256_16": bench.source_hash(),
           "kernels": {"w/backward": {"bwd_states": {"hbm_bytes_per_launch": 5.0,
                                                     "shared_name": True},
                                      "bwd_dz": {"hbm_bytes_per_launch": 7.0,
                                                 "shared_name": False}}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    key = bench.traffic_key("w", "backward")
    assert bench.measured_traffic("bwd_states", key) is None
    assert bench.measured_traffic("bwd_dz", key) == 7.0


def test_train_flops():
    """A training step: the prefill's contractions plus the backward's, less
    the backward's gate/up recompute and state scan."""
    cfg = synth.CONFIGS["qwen3_4b_64k"]
    B, T, d, f = cfg.batch, cfg.seq_len, cfg.d_model, cfg.d_ff
    assert bench.train_flops(cfg) == 24.0 * B * T * d * f + 8.0 * B * T * d * d
