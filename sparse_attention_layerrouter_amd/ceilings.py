"""ctypes binding and timing of libfa_ceilings.so (csrc/ceilings.hip).

The ceiling kernels are measuring instruments of the benchmark, not part of
the attention path: a plain non-temporal read stream (the rate a read of N
bytes reaches on this board) and a dependence-free stream of 32x32x16 bf16
matrix products with a chosen LDS operand read rate and an optional
online-softmax VALU mix (the rate that mix reaches under the board's power
limit).  The functions below marshal arguments and time launches with HIP
events on the given stream; the kernels do the work.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_ceilings.so")
EXPORTS = ("fa_ceiling_last_error", "fa_ceiling_read", "fa_ceiling_mix", "fa_ceiling_valu")

MIX_THREADS = 512
MIX_WAVES = 8
MIX_PRODUCTS = 8              # products per wave per iteration
MIX_PRODUCT_FLOP = {0: 32 * 32 * 16 * 2, 1: 16 * 16 * 32 * 2}  # by shape
SHAPE_NAME = {0: "32x32x16", 1: "16x16x32"}
READ_THREADS = 256

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_attention_layerrouter_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.fa_ceiling_last_error.restype = ctypes.c_char_p
    L.fa_ceiling_last_error.argtypes = []
    L.fa_ceiling_read.restype = I32
    L.fa_ceiling_read.argtypes = [P, SZ, SZ, P, P]
    L.fa_ceiling_mix.restype = I32
    L.fa_ceiling_mix.argtypes = [I32, I32, I32, I32, I32, P, P, P]
    L.fa_ceiling_valu.restype = I32
    L.fa_ceiling_valu.argtypes = [I32, I32, I32, I32, P, P, P]
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        msg = lib().fa_ceiling_last_error().decode()
        raise RuntimeError(f"ceiling kernel: status {status}: {msg}")


def _stream_ptr(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fa_ceiling_read(buf, chunk: int, sink, stream=None) -> None:
    """Read every byte of buf (a device tensor) once, chunk bytes per workgroup;
    sink (device uint32 / int32, (nbytes / chunk) * 256 entries) receives each
    thread's XOR of the 32-bit words it read."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().fa_ceiling_read(ctypes.c_void_p(buf.data_ptr()), nbytes, chunk,
                                 ctypes.c_void_p(sink.data_ptr()), _stream_ptr(stream)))


def fa_ceiling_mix(reads_per_8: int, softmax: bool, n_workgroups: int, iterations: int,
                   seed, out, stream=None, shape: int = 0) -> None:
    """One launch of the product stream: n_workgroups x 8 waves x iterations x 8
    products (shape 0: 32x32x16, 1: 16x16x32); seed is an 8 KiB device buffer,
    out n_workgroups * 512 floats."""
    _check(lib().fa_ceiling_mix(reads_per_8, 1 if softmax else 0, shape, n_workgroups, iterations,
                                ctypes.c_void_p(seed.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                _stream_ptr(stream)))


def fa_ceiling_valu(kind: int, n_workgroups: int, threads: int, iterations: int, out, cycles,
                    stream=None) -> None:
    """One launch of the VALU issue stream (kind 0 FMA, 1 exponential, 2 both);
    out: n_workgroups * threads floats, cycles: n_workgroups * threads / 32 int64
    (per wave: loop shader-clock ticks, loop realtime ticks)."""
    _check(lib().fa_ceiling_valu(kind, n_workgroups, threads, iterations,
                                 ctypes.c_void_p(out.data_ptr()),
                                 ctypes.c_void_p(cycles.data_ptr()), _stream_ptr(stream)))


def mix_flop(n_workgroups: int, iterations: int, shape: int = 0) -> float:
    return float(n_workgroups) * MIX_WAVES * iterations * MIX_PRODUCTS * MIX_PRODUCT_FLOP[shape]


def _time_ms(fn, stream, reps: int) -> list:
    import torch

    fn()  # warm-up
    out = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def measure_read(stream, nbytes: int = 1 << 32, chunks=(128 << 10, 1 << 20, 4 << 20),
                 reps: int = 5) -> dict:
    """Read rate of an nbytes buffer at each chunk size (best of reps, GB/s)."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.stream(stream):
        buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_()
        sink = torch.empty(nbytes // min(chunks) * READ_THREADS, dtype=torch.int32, device=dev)
    res = {}
    for c in chunks:
        ts = _time_ms(lambda: fa_ceiling_read(buf, c, sink, stream), stream, reps)
        best = min(ts)
        res[f"{c >> 10}KiB"] = {"ms_best": round(best, 4), "gbs": round(nbytes / best / 1e6, 1)}
    del buf, sink
    torch.cuda.synchronize()
    return {"bytes": nbytes, "workgroup_threads": READ_THREADS, "by_chunk": res,
            "best_gbs": max(v["gbs"] for v in res.values())}


def measure_mix(stream, configs=((0, False, 0), (8, False, 0), (6, False, 0), (4, False, 0),
                                 (0, True, 0), (8, True, 0), (6, True, 0), (4, True, 0),
                                 (0, False, 1), (8, False, 1), (4, False, 1), (4, True, 1),
                                 (8, True, 1)),
                n_workgroups: int = 1024, iterations: int = 40000, reps: int = 3) -> dict:
    """TFLOP/s of the product stream for each (LDS reads per 8 products,
    softmax mix, shape) triple (median of reps launches of about 25-60 ms each)."""
    import numpy as np
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    # bf16 operand values of magnitude 2^-4 .. 2^-3 with random signs and mantissas
    rng = np.random.default_rng(1)
    expo = 123 + rng.integers(0, 2, 4096)  # biased exponents of 2^-4 and 2^-3
    bits = ((rng.integers(0, 2, 4096) << 15) | (expo << 7) | rng.integers(0, 128, 4096)).astype(
        np.uint16)
    with torch.cuda.stream(stream):
        seed = torch.from_numpy(bits.view(np.int16)).to(dev)
        out = torch.empty(n_workgroups * MIX_THREADS, dtype=torch.float32, device=dev)
    res = []
    for rd, sm, shape in configs:
        flop = mix_flop(n_workgroups, iterations, shape)
        ts = sorted(_time_ms(lambda: fa_ceiling_mix(rd, sm, n_workgroups, iterations, seed, out,
                                                    stream, shape), stream, reps))
        med = ts[len(ts) // 2]
        res.append({"shape": SHAPE_NAME[shape], "lds_reads_per_product": rd / 8,
                    "softmax_mix": bool(sm), "ms": round(med, 3),
                    "tflops": round(flop / med / 1e9, 1)})
    torch.cuda.synchronize()
    return {"workgroups": n_workgroups, "iterations": iterations, "streams": res}


VALU_KINDS = {0: "fma", 1: "exp", 2: "exp_and_fma"}
# waves per SIMD -> (workgroups, threads) on a 256-CU board with 4 SIMDs per CU
VALU_LAYOUTS = {1: (256, 256), 2: (512, 256), 8: (512, 1024)}


def measure_valu(stream, iterations: int = 4000) -> dict:
    """VALU issue rates for three launch layouts (nominally 1, 2 and 8 waves per
    SIMD on a 256-CU board).  Per kind: wave_cycles_per_instruction, the median
    wave's loop shader-clock ticks / its instructions (the interval between one
    wave's instructions under whatever shares its SIMD); simd_cycles_per_instruction,
    the launch's wall time x the loop clock x 1024 SIMDs / all waves' instructions
    (the SIMD's throughput, with no assumption about which waves were resident
    together); and the clock (ticks / realtime)."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    res = {}
    for wps, (nwg, threads) in VALU_LAYOUTS.items():
        with torch.cuda.stream(stream):
            out = torch.empty(nwg * threads, dtype=torch.float32, device=dev)
            cyc = torch.empty(nwg * threads // 32, dtype=torch.int64, device=dev)
        row = {}
        for kind, name in VALU_KINDS.items():
            fa_ceiling_valu(kind, nwg, threads, iterations, out, cyc, stream)  # warm-up
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fa_ceiling_valu(kind, nwg, threads, iterations, out, cyc, stream)
            b.record(stream)
            b.synchronize()
            wall_s = a.elapsed_time(b) * 1e-3
            c = cyc.cpu().view(-1, 2)
            order = sorted(range(c.shape[0]), key=lambda i: int(c[i, 0]))
            mid = order[len(order) // 2]
            ticks, real = int(c[mid, 0]), int(c[mid, 1])
            clock = ticks / (real * 10.0) if real else None  # GHz (realtime: 100 MHz)
            instr = iterations * 64 * (2 if kind == 2 else 1)
            waves = nwg * threads // 64
            row[name] = {
                "wave_cycles_per_instruction": round(ticks / instr, 3),
                "simd_cycles_per_instruction": (round(wall_s * clock * 1e9 * 1024 / (waves * instr), 3)
                                                if clock else None),
                "clock_ghz": round(clock, 3) if clock else None}
        res[f"{wps}_waves_per_simd_nominal"] = row
    return {"iterations": iterations, "chains_per_lane": 8, "steps_per_iteration": 8,
            "layouts": res}
