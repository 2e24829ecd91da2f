"""The bench's JSON line on the GPU: one line with the contract's keys, the
roofline and CPU-baseline objects, for the default forward and for the other
passes (few steps; numbers not checked, only their presence and sanity)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
        "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
        "cpu_baseline"}


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "2", *args], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


@pytest.mark.parametrize("args", [(), ("--pass", "bwd", "--no-cpu-baseline"),
                                  ("--workload", "fp8_b2h32_n4096_d128_causal",
                                   "--no-cpu-baseline"),
                                  ("--pass", "decode", "--no-cpu-baseline")])
def test_bench_line(args):
    rec = _run(*args)
    assert KEYS <= set(rec), KEYS - set(rec)
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 2
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["data"] == "synthetic"
    roof = rec["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and roof["peak"] > 0 and roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "workload" in rec["config"]
    if not args:
        cb = rec["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
        assert rec["parity_vs_oracle"]["o_max_abs"] <= 1e-2
