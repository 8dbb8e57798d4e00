"""Mutation check of the oracle's pins: each planted mistake must make a pin fail.

A plausible mistake in the oracle (a window bound off by one, a dropped term, a
wrong sign, index or head mapping, a transposed operand) is written into a
temporary copy of ``oracle/``, the copy's C library is rebuilt with gcc, and the
pin tests of that part of the oracle run against the copy in a subprocess.  The
test asserts that every mutant is caught (some pin fails) and that the
unmutated copy passes.  Each mutation replaces an exact source snippet, and the
snippet must occur the stated number of times, so a mutation cannot go stale
silently when the oracle is edited.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS_C = "test_oracle_pins.py"
PINS_XA = "test_xattn_pins.py"
PINS_TA = "test_triangle_pins.py"

# (id, file under oracle/, [(old snippet, new snippet, occurrences)], pin file)
MUTATIONS = [
    # ---- fa_oracle.c: routing, the streaming block rule, attention
    ("window_one_wider", "fa_oracle.c",
     [("return (j < ns) || (j > i - nw);", "return (j < ns) || (j >= i - nw);", 1)], PINS_C),
    ("window_one_narrower", "fa_oracle.c",
     [("return (j < ns) || (j > i - nw);", "return (j < ns) || (j > i - nw + 1);", 1)], PINS_C),
    ("sink_one_wider", "fa_oracle.c",
     [("return (j < ns) || (j > i - nw);", "return (j <= ns) || (j > i - nw);", 1)], PINS_C),
    ("causal_edge_excludes_diagonal", "fa_oracle.c",
     [("    if (s > t)\n        return 0;", "    if (s >= t && t > 0)\n        return 0;", 1)],
     PINS_C),
    ("causal_edge_one_late", "fa_oracle.c",
     [("    if (s > t)\n        return 0;", "    if (s > t + 1)\n        return 0;", 1)], PINS_C),
    ("pool_window_shifted", "fa_oracle.c",
     [("for (int t = T - P; t < T; ++t) {", "for (int t = T - P - 1; t < T - 1; ++t) {", 1)],
     PINS_C),
    ("relu_dropped", "fa_oracle.c",
     [("h32[i] = a32 > 0.0f ? a32 : 0.0f;", "h32[i] = a32;", 1),
      ("h64[i] = a64 > 0.0 ? a64 : 0.0;", "h64[i] = a64;", 1)], PINS_C),
    ("threshold_polarity", "fa_oracle.c",
     [("(z32 > 0.0f) ? 1 : 0", "(z32 > 0.0f) ? 0 : 1", 1)], PINS_C),
    ("threshold_not_strict", "fa_oracle.c",
     [("(z32 > 0.0f) ? 1 : 0", "(z32 >= 0.0f) ? 1 : 0", 1)], PINS_C),
    ("softmax_not_normalised", "fa_oracle.c",
     [("double w = exp(scores[s] - m) / l;", "double w = exp(scores[s] - m);", 1)], PINS_C),
    ("lse_without_max", "fa_oracle.c",
     [("*lse_out = m + log(l);", "*lse_out = log(l);", 1)], PINS_C),
    ("output_bias_dropped", "fa_oracle.c",
     [("z32 += b2[l];", "", 1), ("z64 += (double)b2[l];", "", 1)], PINS_C),
    ("plan_window_one_wider", "fa_oracle.c",
     [("win_begin = i - nw + 1;", "win_begin = i - nw;", 1)], PINS_C),
    ("gqa_heads_interleaved", "fa_oracle.c",
     [("        int g = h / G;\n        int is_fa = j->route[(size_t)b * j->n_layers + j->layer] != 0;\n"
       "        for (int c = 0; c < j->d; ++c)\n            qv[c] = orc_load(j->q, j->dtype,\n"
       "                             ((size_t)token",
       "        int g = h % j->hkv;\n        int is_fa = j->route[(size_t)b * j->n_layers + j->layer] != 0;\n"
       "        for (int c = 0; c < j->d; ++c)\n            qv[c] = orc_load(j->q, j->dtype,\n"
       "                             ((size_t)token", 1)], PINS_C),
    ("decode_query_one_position_late", "fa_oracle.c",
     [("                n - 1, n, is_fa, j->sink,", "                n, n, is_fa, j->sink,", 1)],
     PINS_C),
    # ---- xattn.py: antidiagonal scoring and threshold selection
    ("xa_query_not_reversed", "xattn.py",
     [("qr = qp.reshape(Tr, stride, d)[:, ::-1, :].reshape(Tr, stride * d)",
       "qr = qp.reshape(Tr, stride, d).reshape(Tr, stride * d)", 1)], PINS_XA),
    ("xa_scale_without_stride", "xattn.py",
     [("A = (qr @ kr.T) * (sm_scale / stride)", "A = (qr @ kr.T) * sm_scale", 2)], PINS_XA),
    ("xa_causal_edge_one_late", "xattn.py",
     [("A[np.triu_indices(Tr, 1)] = -np.inf", "A[np.triu_indices(Tr, 2)] = -np.inf", 1)],
     PINS_XA),
    ("xa_causal_edge_dropped", "xattn.py",
     [("    A[np.triu_indices(Tr, 1)] = -np.inf\n", "", 1)], PINS_XA),
    ("xa_sink_not_forced", "xattn.py",
     [("    keep[0] = True\n    keep[i] = True\n    kept = np.float32(row[0])",
       "    keep[i] = True\n    kept = np.float32(0.0)", 1)], PINS_XA),
    ("xa_diagonal_not_forced", "xattn.py",
     [("    keep[i] = True\n    kept = np.float32(row[0])\n    if i > 0:\n"
       "        kept = np.float32(kept + row[i])",
       "    kept = np.float32(row[0])", 1)], PINS_XA),
    ("xa_ascending_order", "xattn.py",
     [("key=lambda j: (-float(row[j]), j)", "key=lambda j: (float(row[j]), j)", 1)], PINS_XA),
    ("xa_threshold_not_strict", "xattn.py",
     [("if not kept < goal:", "if not kept <= goal:", 1)], PINS_XA),
    ("xa_gqa_heads_interleaved", "xattn.py",
     [("A = reshaped_scores(q[s0:s1, h], k[s0:s1, h // G], stride, sm_scale)",
       "A = reshaped_scores(q[s0:s1, h], k[s0:s1, h % hkv], stride, sm_scale)", 1)], PINS_XA),
    ("xa_mask_transposed", "xattn.py",
     [("kept = keep[b, :, t // block][:, keys // block]",
       "kept = keep[b, :, :, t // block][:, keys // block]", 1)], PINS_XA),
    ("xa_attention_past_causal_edge", "xattn.py",
     [("        keys = np.arange(t + 1)\n",
       "        keys = np.arange(min(t + 2, int(cu[b + 1]) - s0))\n", 1)], PINS_XA),
    # ---- triangle.py: the dense tail on top of the streaming blocks
    ("ta_tail_one_short", "triangle.py",
     [("dense_row = i >= nb - nl", "dense_row = i > nb - nl", 1)], PINS_TA),
    ("ta_tail_one_long", "triangle.py",
     [("dense_row = i >= nb - nl", "dense_row = i >= nb - nl - 1", 1)], PINS_TA),
    ("ta_window_one_wider", "triangle.py",
     [("keep[i, j] = dense_row or j < ns or j > i - nw",
       "keep[i, j] = dense_row or j < ns or j >= i - nw", 1)], PINS_TA),
    ("ta_sink_one_wider", "triangle.py",
     [("keep[i, j] = dense_row or j < ns or j > i - nw",
       "keep[i, j] = dense_row or j <= ns or j > i - nw", 1)], PINS_TA),
    ("ta_route_inverted", "triangle.py",
     [("        if route_bits[b]:\n", "        if not route_bits[b]:\n", 1)], PINS_TA),
    ("ta_ragged_block_dropped", "triangle.py",
     [("    nb = -(-T // block)\n    ns, nw, nl", "    nb = max(1, T // block)\n    ns, nw, nl", 1)],
     PINS_TA),
    ("ta_tail_size", "triangle.py",
     [("last_q // block\n", "last_q // block + 1\n", 1)], PINS_TA),
]


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.tmp", "__pycache__"))
    tdir = os.path.join(dst, "tests")
    os.makedirs(tdir)
    for f in ("conftest.py", PINS_C, PINS_XA, PINS_TA):
        shutil.copy(os.path.join(ROOT, "tests", f), tdir)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tdir, "golden"))
    pdir = os.path.join(dst, "sparse_attention_layerrouter_amd")
    os.makedirs(pdir)
    for f in ("__init__.py", "_lib.py", "synth.py"):
        shutil.copy(os.path.join(ROOT, "sparse_attention_layerrouter_amd", f), pdir)


def _mutate(dst, fname, edits):
    path = os.path.join(dst, "oracle", fname)
    with open(path) as f:
        src = f.read()
    for old, new, count in edits:
        n = src.count(old)
        if n != count:
            raise AssertionError(f"{fname}: snippet found {n} times, expected {count}: {old!r}")
        src = src.replace(old, new)
    with open(path, "w") as f:
        f.write(src)


def _run_pins(dst, pin_file):
    env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
    env["OMP_NUM_THREADS"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", pin_file)], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_unmutated_copy_passes_every_pin(tmp_path):
    _copy_tree(str(tmp_path))
    for pins in (PINS_C, PINS_XA, PINS_TA):
        rc, out = _run_pins(str(tmp_path), pins)
        assert rc == 0, f"{pins} fails on the unmutated copy:\n{out}"


def test_every_planted_mistake_is_caught(tmp_path):
    def one(m):
        mid, fname, edits, pins = m
        dst = os.path.join(str(tmp_path), mid)
        os.makedirs(dst)
        _copy_tree(dst)
        _mutate(dst, fname, edits)
        rc, out = _run_pins(dst, pins)
        return mid, rc, out

    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(one, MUTATIONS))
    survivors = [(mid, out) for mid, rc, out in results if rc == 0]
    # a mutant is caught by a failing pin (rc 1); a crash or a collection error would
    # not show that a pin sees the mistake
    odd = [(mid, rc, out) for mid, rc, out in results if rc not in (0, 1)]
    assert not survivors, "mutants no pin catches: " + ", ".join(m for m, _ in survivors)
    assert not odd, "mutants that did not end in a pin failure: " + "; ".join(
        f"{m} rc={rc}: {out[-400:]}" for m, rc, out in odd)


@pytest.mark.parametrize("fname", ["fa_oracle.c", "xattn.py", "triangle.py"])
def test_mutations_cover_each_oracle_file(fname):
    assert sum(1 for m in MUTATIONS if m[1] == fname) >= 7
