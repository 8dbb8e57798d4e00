"""bench.py end to end on a small configuration (16384-token prefill, batch-2 decode
over 16384-token caches, no side legs): it must print exactly one JSON line with
the fields the benchmark contract names, with finite positive figures and the
roofline and timing objects filled in."""
import json
import math
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1", "--warmup", "1",
           "--seq", "16384", "--decode-len", "16384", "--decode-batch", "2", "--no-sweep",
           "--no-serving", "--no-chunked", "--no-xattn", "--no-triangle", "--no-qwen",
           "--no-config2", "--no-cpu-baseline", "--no-clock"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "timing"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 1
    assert d["dtype"] == "bf16" and d["higher_is_better"] is True
    assert "workload" in d["config"]
    assert math.isfinite(d["value"]) and d["value"] > 0
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert d["decode"]["tok_s"] > 0
    c = d["ceilings"]
    assert c["read"]["best_gbs"] > 0 and c["mix"]["prefill_mix_tflops"] > 0
    assert 0 < c["fa_prefill_over_its_mix_stream"] and 0 < c["fa_decode_over_read_stream"]
    assert d["timing"]["prefill_fa_layer_ms"]["n"] >= 1
