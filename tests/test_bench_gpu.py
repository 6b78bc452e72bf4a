"""bench.py end to end on a small workload (GPU): every variant the
driver and the profiles use prints one JSON line with the contract's
fields, and the plain line's CPU baseline is the oracle's."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline")


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_amp",
                        "--steps", "1", "--warmup", "1", *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("variant", ["plain", "backward", "train", "decode"])
def test_bench_line(variant):
    extra = [] if variant == "plain" else ["--no-cpu-baseline"]
    d = run_bench("--variant", variant, *extra)
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "tiny_amp" and d["config"]["variant"] == variant
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and 0 < roof["frac"] < 1
    assert roof["achieved"] > 0 and roof["peak"] > 0
    if variant == "plain":
        cb = d["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
