"""Build libfluxattn.so (the C-ABI library of include/fluxattn.h) for gfx950.

Every attention HIP source under csrc/ and the host ABI (csrc/api.cpp) is
compiled with hipcc for gfx950 only and linked in-tree into
sparse_attention_layerrouter_amd/libfluxattn.so.  The ceiling kernels
(csrc/ceilings.hip, measuring instruments of the benchmark, not part of the
attention path) are linked into a library of their own, libfa_ceilings.so.

    python -m sparse_attention_layerrouter_amd.build
"""
from __future__ import annotations

import concurrent.futures
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfluxattn.so")
CEILINGS_OUT = os.path.join(PKG, "libfa_ceilings.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
SOURCES = ["router.hip", "prefill.hip", "decode.hip", "xattn.hip", "api.cpp"]
CEILINGS_SOURCE = "ceilings.hip"
# The hot MFMA / split-K kernels keep everything in registers: a build whose
# compiler places any of their state in scratch memory (spills or a stack
# array) is refused, since it would run many times slower.
HOT_KERNELS = ("prefill_bf16_kernel", "decode_bf16_kernel", "decode_split_kernel",
               "xa_score_kernel")
_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs Spill|VGPRs|AGPRs"
                     r"|LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]):\s+(\S+)")


def _resources(stderr: str) -> dict:
    """{kernel symbol: {field: value}} from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, csrc: str = CSRC, build_dir: str = BUILD_DIR):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    flags = [f if f != CSRC else csrc for f in FLAGS]
    cmd = [HIPCC, *flags, "-c", os.path.join(csrc, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    else:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def check_resources(res: dict) -> None:
    bad = [f"{k}: scratch {v.get('ScratchSize [bytes/lane]')} B/lane, "
           f"{v.get('VGPRs Spill')} VGPR spills"
           for k, v in res.items()
           if any(h in k for h in HOT_KERNELS)
           and (v.get("ScratchSize [bytes/lane]", 0) != 0 or v.get("VGPRs Spill", 0) != 0)]
    if bad:
        raise RuntimeError("hot kernels would use scratch memory:\n  " + "\n  ".join(bad))


def _link(objs: list, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build_copy(csrc: str, out: str, build_dir: str) -> str:
    """Build the attention library from another source directory (a patched copy of
    csrc/, e.g. an instrumented one for measurement) into `out`; the same flags."""
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(lambda src: _compile(src, csrc, build_dir), SOURCES))
    _link([o for o, _ in done], out)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + [CEILINGS_SOURCE]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = dict(zip(srcs, ex.map(_compile, srcs)))
    res = {k: v for src in SOURCES for k, v in done[src][1].items()}
    with open(os.path.join(BUILD_DIR, "kernel_resources.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    check_resources(res)
    _link([done[src][0] for src in SOURCES], OUT)
    _link([done[CEILINGS_SOURCE][0]], CEILINGS_OUT)
    if verbose:
        print(f"built {OUT}")
        print(f"built {CEILINGS_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
