"""CPU oracle for Flux Attention's layer-routed hybrid attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` (the oracle's timing and the parity checks that
reuse it, all behind ``bench.load_oracle``) may import this package; the product
library never does.  The arithmetic lives in ``fa_oracle.c`` (plain C, fp64
accumulation, exact two-pass softmax); this module only marshals numpy arrays
into it with ctypes.

Sources: the pages about "Flux Attention: Context-Aware Hybrid Attention for
Efficient LLMs Inference" -- the HF model card's summary paragraph, the
thelatestinai paper page (Figure 2, Figure 8, Table 3, Table 6) and the
codewithpapers function list (``repeat_kv``,
``generate_streaming_info_blocksparse_flash_attn``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1


def build(force: bool = False) -> str:
    """Compile fa_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall",
             "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_pool.argtypes = [P, I, P, I, I, I, P, P]
        lib.orc_router.argtypes = [P, I, P, I, I, I, P, P, I, P, P, I, P, P, P]
        lib.orc_block_plan.argtypes = [P, I, I, P, I, I, I, I, I, P]
        lib.orc_visible_predicate.argtypes = [I, I, I, I, I, I]
        lib.orc_visible_pairs.argtypes = [I, I, I, I, I]
        lib.orc_visible_pairs.restype = ctypes.c_int64
        lib.orc_attn_prefill.argtypes = [P, P, P, I, P, I, I, I, I, P, I, I,
                                         I, I, I, D, P, I, P, P, I]
        lib.orc_attn_decode.argtypes = [P, P, P, I, P, I, I, I, I, I, P, I, I,
                                        I, I, I, D, P, I, P, P, I]
        for f in (lib.orc_pool, lib.orc_router, lib.orc_block_plan,
                  lib.orc_attn_prefill, lib.orc_attn_decode,
                  lib.orc_visible_predicate):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    """fp32 arrays are F32; uint16 arrays hold raw bf16 bit patterns."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.asarray(a)
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def pool(x, cu_seqlens, pool_tokens):
    """Mean of the last min(pool_tokens, T_b) rows of every sequence.

    Returns (p32, p64): the fp32 (ascending-t sum) and fp64 pools."""
    lib = _load()
    x = _c(x)
    cu = _c(cu_seqlens, np.int32)
    B = cu.size - 1
    hidden = x.shape[-1]
    p32 = np.zeros((B, hidden), np.float32)
    p64 = np.zeros((B, hidden), np.float64)
    _check(lib.orc_pool(_ptr(x), _dtype_code(x), _ptr(cu), B, hidden, pool_tokens,
                        _ptr(p32), _ptr(p64)), "pool")
    return p32, p64


def router(x, cu_seqlens, pool_tokens, w1, b1, w2, b2):
    """Layer Router: pool -> ReLU(W1 p + b1) -> W2 h + b2 -> bit (logit > 0).

    Returns (route uint8 [B, L], logits32 [B, L], logits64 [B, L])."""
    lib = _load()
    x = _c(x)
    cu = _c(cu_seqlens, np.int32)
    w1, b1, w2, b2 = (_c(a, np.float32) for a in (w1, b1, w2, b2))
    B = cu.size - 1
    hidden = x.shape[-1]
    Hr, L = w1.shape[0], w2.shape[0]
    assert w1.shape == (Hr, hidden) and b1.shape == (Hr,)
    assert w2.shape == (L, Hr) and b2.shape == (L,)
    route = np.zeros((B, L), np.uint8)
    l32 = np.zeros((B, L), np.float32)
    l64 = np.zeros((B, L), np.float64)
    _check(lib.orc_router(_ptr(x), _dtype_code(x), _ptr(cu), B, hidden, pool_tokens,
                          _ptr(w1), _ptr(b1), Hr, _ptr(w2), _ptr(b2), L,
                          _ptr(route), _ptr(l32), _ptr(l64)), "router")
    return route, l32, l64


def block_plan(seqlens, max_qblocks, route, layer, sink, window, block):
    """Kept key-block ranges per (sequence, query block): int32 [B, max_qblocks, 4]."""
    lib = _load()
    sl = _c(seqlens, np.int32)
    route = _c(route, np.uint8)
    B, L = route.shape
    plan = np.zeros((B, max_qblocks, 4), np.int32)
    _check(lib.orc_block_plan(_ptr(sl), B, max_qblocks, _ptr(route), L, layer,
                              sink, window, block, _ptr(plan)), "block_plan")
    return plan


def visible(t, s, is_fa, sink, window, block) -> bool:
    return bool(_load().orc_visible_predicate(t, s, int(is_fa), sink, window, block))


def visible_pairs(T, is_fa, sink, window, block) -> int:
    return int(_load().orc_visible_pairs(T, int(is_fa), sink, window, block))


def attn_prefill(q, k, v, cu_seqlens, route, layer, sink, window, block,
                 sm_scale, rows=None, n_threads=None):
    """Prefill attention of one layer (packed varlen layout).

    q [total, Hq, d], k/v [total, Hkv, d] as float32 or bf16 bits (uint16).
    Returns (o float64 [n_rows, Hq, d], lse float64 [n_rows, Hq])."""
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    cu = _c(cu_seqlens, np.int32)
    route = _c(route, np.uint8)
    B = cu.size - 1
    _, Hq, d = q.shape
    Hkv = k.shape[1]
    L = route.shape[1]
    rows_a = None if rows is None else _c(rows, np.int32)
    n_rows = int(cu[-1]) if rows_a is None else rows_a.size
    o = np.zeros((n_rows, Hq, d), np.float64)
    lse = np.zeros((n_rows, Hq), np.float64)
    nt = n_threads or os.cpu_count() or 1
    _check(lib.orc_attn_prefill(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(cu), B, Hq,
                                Hkv, d, _ptr(route), L, layer, sink, window, block,
                                float(sm_scale), _ptr(rows_a), n_rows, _ptr(o),
                                _ptr(lse), nt), "attn_prefill")
    return o, lse


def attn_decode(q, k_cache, v_cache, cache_len, route, layer, sink, window,
                block, sm_scale, heads=None, n_threads=None):
    """Decode attention of one layer; the new token is already in the cache.

    q [B, Hq, d]; k_cache/v_cache [B, Hkv, max_cache, d].
    Returns (o float64 [B, Hq, d], lse float64 [B, Hq])."""
    lib = _load()
    q, kc, vc = _c(q), _c(k_cache), _c(v_cache)
    dt = _dtype_code(q)
    assert _dtype_code(kc) == dt and _dtype_code(vc) == dt
    cl = _c(cache_len, np.int32)
    route = _c(route, np.uint8)
    B, Hq, d = q.shape
    Hkv, max_cache = kc.shape[1], kc.shape[2]
    L = route.shape[1]
    heads_a = None if heads is None else _c(heads, np.int32)
    n_heads = 0 if heads_a is None else heads_a.size
    o = np.zeros((B, Hq, d), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    nt = n_threads or os.cpu_count() or 1
    _check(lib.orc_attn_decode(_ptr(q), _ptr(kc), _ptr(vc), max_cache, _ptr(cl), dt,
                               B, Hq, Hkv, d, _ptr(route), L, layer, sink, window,
                               block, float(sm_scale), _ptr(heads_a), n_heads,
                               _ptr(o), _ptr(lse), nt), "attn_decode")
    return o, lse
