"""Host logic of bench.py (CPU only): the work counts behind its roofline and
throughput figures against brute-force enumeration of the visibility rule, the
timing distribution, the amd-smi clock parsing and the refusal of more than one
GPU.  No GPU is touched."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def visible_pairs_brute(T, sink, window, block, tail_blocks=0):
    """Count (t, s), s <= t < T, that the streaming rule (and an optional dense
    tail of the last tail_blocks query blocks) keeps, by enumeration."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    qb, kb = t // block, s // block
    nqb = -(-T // block)
    keep = (kb < sink // block) | (kb >= qb - window // block + 1) | (qb >= nqb - tail_blocks)
    return int(((s <= t) & keep).sum())


@pytest.mark.parametrize("T,sink,window,block", [
    (1, 128, 2048, 64), (63, 128, 2048, 64), (64, 128, 2048, 64), (2175, 128, 2048, 64),
    (2176, 128, 2048, 64), (3000, 128, 2048, 64), (1000, 0, 64, 16), (777, 48, 96, 16),
    (1500, 256, 512, 128)])
def test_pair_counts_match_enumeration(T, sink, window, block):
    assert bench.pairs_fa(T) == T * (T + 1) // 2 == visible_pairs_brute(T, T, T, 1)
    assert bench.pairs_sa(T, sink, window, block) == visible_pairs_brute(T, sink, window, block)
    for last_q in (block, 4 * block, 1 << 20):
        nl = min(last_q // block, -(-T // block))
        assert bench.pairs_ta(T, last_q, sink, window, block) == visible_pairs_brute(
            T, sink, window, block, nl)


def test_pair_counts_at_the_benchmark_sizes():
    # 131072 tokens, sink 128, window 2048, block 64 (the counts the roofline uses)
    assert bench.pairs_fa(131072) == 8590000128
    assert bench.flops_of_pairs(bench.pairs_fa(131072)) == 4.0 * 128 * 32 * 8590000128
    sa = bench.pairs_sa(131072)
    # every row past the first window sees exactly its sink, its full window blocks and
    # the causal part of its own block: 128 + 31 * 64 + (t mod 64) + 1 keys
    first = 2176  # rows before this see everything causal up to the block rule
    tail_rows = 131072 - first
    expect_tail = tail_rows * (128 + 31 * 64) + (tail_rows // 64) * (64 * 65 // 2)
    assert sa == bench.pairs_sa(first) + expect_tail


@pytest.mark.parametrize("n", [1, 2, 64, 65, 128, 129, 2176, 2177, 5000, 131072])
def test_decode_kept_tokens_match_enumeration(n):
    sink, window, block = 128, 2048, 64
    s = np.arange(n)
    kb, qb = s // block, (n - 1) // block
    keep = (kb < sink // block) | (kb >= qb - window // block + 1)
    assert bench.kept_tokens_decode(n, False, sink, window, block) == int(keep.sum())
    assert bench.kept_tokens_decode(n, True, sink, window, block) == n


def test_timing_distribution():
    d = bench.dist([5.0, 1.0, 3.0, 2.0, 4.0])
    assert d == {"median": 3.0, "p10": 1.4, "p90": 4.6, "mean": 3.0, "n": 5}
    assert bench.dist([]) is None


def test_clock_parsing(monkeypatch):
    doc = {"gpu_data": [{"gpu": 0, "clock": {
        "gfx_0": {"clk": {"value": 1500, "unit": "MHz"}},
        "gfx_1": {"clk": {"value": 1600, "unit": "MHz"}},
        "gfx_2": {"clk": {"value": "N/A", "unit": "MHz"}},
        "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]}

    class R:
        stdout = json.dumps(doc)

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())
    c = bench.ClockSampler()
    c.exe = "amd-smi"
    assert c._read() == 1550.0  # graphics domains only, numeric values only
    R.stdout = json.dumps(doc["gpu_data"])  # a bare list of devices
    assert c._read() == 1550.0
    c.exe = None
    c.samples = [1500.0, 1550.0, 1600.0]
    out = c.stop("test window")
    assert out["median"] == 1550.0 and out["n"] == 3 and out["unit"] == "MHz"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
