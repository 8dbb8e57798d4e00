"""ctypes binding of libfluxattn.so (the C ABI in include/fluxattn.h).

Argument marshalling only: every function below has the name of its C entry
point, takes torch tensors (device memory owned by the caller), reads shapes
off them, passes raw pointers and the current HIP stream, and raises
FluxAttnError when the C call returns a non-OK status.  All arithmetic happens
in the library's gfx950 kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfluxattn.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)
FA_F32, FA_BF16 = 0, 1

EXPORTS = (
    "fa_last_error", "fa_abi_version", "fa_router_workspace_size", "fa_router_decide",
    "fa_block_plan", "fa_attn_prefill", "fa_decode_workspace_size", "fa_attn_decode",
    "fa_kv_compact", "fa_attn_decode_ring", "fa_attn_prefill_kv", "fa_xattn_scores",
    "fa_xattn_select", "fa_attn_prefill_xattn", "fa_attn_prefill_triangle",
    "fa_xattn_workspace_size", "fa_attn_decode_noalloc",
)


class FluxAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfluxattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_attention_layerrouter_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_abi_version.restype = I32
    L.fa_abi_version.argtypes = []
    L.fa_router_workspace_size.restype = SZ
    L.fa_router_workspace_size.argtypes = [I32, I32, I32]
    L.fa_router_decide.restype = I32
    L.fa_router_decide.argtypes = [P, I32, P, I32, I32, I32, P, P, I32, P, P, I32, P, P, P, SZ, P]
    L.fa_block_plan.restype = I32
    L.fa_block_plan.argtypes = [P, I32, I32, P, I32, I32, I32, I32, I32, P, P]
    L.fa_attn_prefill.restype = I32
    L.fa_attn_prefill.argtypes = [P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, P, P, I32,
                                  I32, I32, I32, I32, F, P]
    L.fa_attn_prefill_kv.restype = I32
    L.fa_attn_prefill_kv.argtypes = [P, P, P, P, P, I32, P, P, I32, I32, I32, I32, I32, P, P,
                                     I32, I32, I32, I32, I32, F, P]
    L.fa_attn_prefill_triangle.restype = I32
    L.fa_attn_prefill_triangle.argtypes = [P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, P, P,
                                           I32, I32, I32, I32, I32, I32, F, P]
    L.fa_xattn_scores.restype = I32
    L.fa_xattn_scores.argtypes = [P, P, I32, P, I32, I32, I32, I32, I32, I32, I32, F, P, I32, P,
                                  SZ, P]
    L.fa_xattn_workspace_size.restype = SZ
    L.fa_xattn_workspace_size.argtypes = [I32, I32, I32]
    L.fa_xattn_select.restype = I32
    L.fa_xattn_select.argtypes = [P, P, I32, I32, I32, I32, F, P, P]
    L.fa_attn_prefill_xattn.restype = I32
    L.fa_attn_prefill_xattn.argtypes = [P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32, P,
                                        I32, F, P]
    L.fa_decode_workspace_size.restype = SZ
    L.fa_decode_workspace_size.argtypes = [I32, I32, I32, I32]
    L.fa_attn_decode.restype = I32
    L.fa_attn_decode.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, P, P, I32,
                                 I32, I32, I32, I32, F, P, SZ, P]
    L.fa_attn_decode_noalloc.restype = I32
    L.fa_attn_decode_noalloc.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32,
                                         P, P, I32, I32, I32, I32, I32, F, P]
    L.fa_kv_compact.restype = I32
    L.fa_kv_compact.argtypes = [P, P, I32, P, I32, I32, I32, I32, I32, I32, P, P, I32, P]
    L.fa_attn_decode_ring.restype = I32
    L.fa_attn_decode_ring.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                      I32, I32, F, P, SZ, P]
    _lib = L
    return _lib


def last_error() -> str:
    return lib().fa_last_error().decode()


def _check(status: int):
    if status != FA_OK:
        raise FluxAttnError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libfluxattn works on device tensors only")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def fa_abi_version() -> int:
    return int(lib().fa_abi_version())


def fa_router_workspace_size(batch: int, hidden: int, router_hidden: int) -> int:
    return int(lib().fa_router_workspace_size(batch, hidden, router_hidden))


def fa_decode_workspace_size(batch: int, n_q_heads: int, head_dim: int, max_cache: int) -> int:
    return int(lib().fa_decode_workspace_size(batch, n_q_heads, head_dim, max_cache))


def fa_router_decide(x_q, cu_seqlens, pool_tokens, w1, b1, w2, b2, route, logits=None,
                     workspace=None, stream=None):
    """Layer Router: x_q [total, hidden] -> route [B, L] uint8 (1 = FA)."""
    import torch
    _require_cuda(x_q, cu_seqlens, w1, b1, w2, b2, route, logits)
    batch = cu_seqlens.numel() - 1
    hidden = x_q.shape[-1]
    router_hidden, n_layers = w1.shape[0], w2.shape[0]
    if workspace is None:
        n = fa_router_workspace_size(batch, hidden, router_hidden)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=x_q.device)
    _check(lib().fa_router_decide(
        _ptr(x_q), _dtype_code(x_q), _ptr(cu_seqlens), batch, hidden, pool_tokens, _ptr(w1),
        _ptr(b1), router_hidden, _ptr(w2), _ptr(b2), n_layers, _ptr(route), _ptr(logits),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def fa_block_plan(cu_seqlens, max_qblocks, route, layer, sink_tokens, window_tokens,
                  block_tokens, plan, stream=None):
    """Kept key-block ranges: plan [B, max_qblocks, 4] int32."""
    _require_cuda(cu_seqlens, route, plan)
    batch = cu_seqlens.numel() - 1
    _check(lib().fa_block_plan(
        _ptr(cu_seqlens), batch, max_qblocks, _ptr(route), route.shape[1], layer, sink_tokens,
        window_tokens, block_tokens, _ptr(plan), _stream(stream)))


def _host_u8(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.uint8))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def fa_attn_prefill(q, k, v, o, cu_seqlens, max_seqlen, route, layer, sink_tokens,
                    window_tokens, block_tokens, sm_scale, lse=None, route_host=None,
                    stream=None):
    """Prefill attention of one layer: q [total, Hq, d], k/v [total, Hkv, d] -> o."""
    _require_cuda(q, k, v, o, cu_seqlens, route, lse)
    batch = cu_seqlens.numel() - 1
    _, hq, d = q.shape
    hkv = k.shape[1]
    keep, rh = _host_u8(route_host)
    _check(lib().fa_attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), _ptr(cu_seqlens), batch,
        int(max_seqlen), hq, hkv, d, _ptr(route), rh, route.shape[1], layer, sink_tokens,
        window_tokens, block_tokens, float(sm_scale), _stream(stream)))
    del keep


def fa_attn_prefill_kv(q, k, v, o, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, route, layer,
                       sink_tokens, window_tokens, block_tokens, sm_scale, lse=None,
                       route_host=None, stream=None):
    """Prefill of the last Tq tokens of each sequence against all Tk of its keys:
    q [total_q, Hq, d], k/v [total_k, Hkv, d] -> o [total_q, Hq, d]."""
    _require_cuda(q, k, v, o, cu_seqlens_q, cu_seqlens_k, route, lse)
    batch = cu_seqlens_q.numel() - 1
    _, hq, d = q.shape
    hkv = k.shape[1]
    keep, rh = _host_u8(route_host)
    _check(lib().fa_attn_prefill_kv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), batch, int(max_seqlen_q), hq, hkv, d, _ptr(route), rh,
        route.shape[1], layer, sink_tokens, window_tokens, block_tokens, float(sm_scale),
        _stream(stream)))
    del keep


def fa_attn_prefill_triangle(q, k, v, o, cu_seqlens, max_seqlen, route, layer, sink_tokens,
                             window_tokens, block_tokens, last_q_tokens, sm_scale, lse=None,
                             route_host=None, stream=None):
    """Prefill with Triangle Attention as the sparse branch (SA rows plus a dense
    tail of last_q_tokens rows per sequence): q [total, Hq, d], k/v [total, Hkv, d] -> o."""
    _require_cuda(q, k, v, o, cu_seqlens, route, lse)
    batch = cu_seqlens.numel() - 1
    _, hq, d = q.shape
    hkv = k.shape[1]
    keep, rh = _host_u8(route_host)
    _check(lib().fa_attn_prefill_triangle(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), _ptr(cu_seqlens), batch,
        int(max_seqlen), hq, hkv, d, _ptr(route), rh, route.shape[1], layer, sink_tokens,
        window_tokens, block_tokens, last_q_tokens, float(sm_scale), _stream(stream)))
    del keep


def fa_xattn_workspace_size(batch, n_q_heads, n_qblocks) -> int:
    return int(lib().fa_xattn_workspace_size(batch, n_q_heads, n_qblocks))


def fa_xattn_scores(q, k, cu_seqlens, max_seqlen, block_tokens, stride, sm_scale, scores,
                    workspace=None, stream=None):
    """XAttention antidiagonal block scores: scores [B, Hq, NQB, NQB] float32 out."""
    import torch
    _require_cuda(q, k, cu_seqlens, scores, workspace)
    batch = cu_seqlens.numel() - 1
    _, hq, d = q.shape
    nqb = scores.shape[2]
    if workspace is None:
        n = fa_xattn_workspace_size(batch, hq, nqb)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_xattn_scores(
        _ptr(q), _ptr(k), _dtype_code(q), _ptr(cu_seqlens), batch, int(max_seqlen), hq,
        k.shape[1], d, block_tokens, stride, float(sm_scale), _ptr(scores), nqb,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def fa_xattn_select(scores, cu_seqlens, block_tokens, threshold, mask, stream=None):
    """XAttention block selection: mask [B, Hq, NQB, ceil(NQB/32)] int32 (uint32 bits) out."""
    _require_cuda(scores, cu_seqlens, mask)
    batch, hq, nqb = scores.shape[0], scores.shape[1], scores.shape[2]
    _check(lib().fa_xattn_select(
        _ptr(scores), _ptr(cu_seqlens), batch, hq, nqb, block_tokens, float(threshold),
        _ptr(mask), _stream(stream)))


def fa_attn_prefill_xattn(q, k, v, o, cu_seqlens, max_seqlen, block_tokens, mask, sm_scale,
                          lse=None, stream=None):
    """Prefill over kept blocks: mask [B, Hq, NQB, ceil(NQB/32)] (uint32 bits as int32)."""
    _require_cuda(q, k, v, o, cu_seqlens, mask, lse)
    batch = cu_seqlens.numel() - 1
    _, hq, d = q.shape
    _check(lib().fa_attn_prefill_xattn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _dtype_code(q), _ptr(cu_seqlens), batch,
        int(max_seqlen), hq, k.shape[1], d, block_tokens, _ptr(mask), mask.shape[2],
        float(sm_scale), _stream(stream)))


def fa_attn_decode(q, o, k_cache, v_cache, cache_len, route, layer, sink_tokens, window_tokens,
                   block_tokens, sm_scale, workspace=None, k_new=None, v_new=None, lse=None,
                   route_host=None, stream=None):
    """Decode step of one layer: q [B, Hq, d] over k/v_cache [B, Hkv, max_cache, d] -> o."""
    import torch
    _require_cuda(q, o, k_cache, v_cache, cache_len, route, k_new, v_new, lse)
    batch, hq, d = q.shape
    hkv, max_cache = k_cache.shape[1], k_cache.shape[2]
    if workspace is None:
        n = fa_decode_workspace_size(batch, hq, d, max_cache)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    keep, rh = _host_u8(route_host)
    _check(lib().fa_attn_decode(
        _ptr(q), _ptr(o), _ptr(lse), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        max_cache, _ptr(cache_len), _dtype_code(q), batch, hq, hkv, d, _ptr(route), rh,
        route.shape[1], layer, sink_tokens, window_tokens, block_tokens, float(sm_scale),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    del keep


def fa_attn_decode_noalloc(q, o, k_cache, v_cache, cache_len, route, layer, sink_tokens,
                           window_tokens, block_tokens, sm_scale, k_new=None, v_new=None,
                           lse=None, route_host=None, stream=None):
    """fa_attn_decode with the split partials in the library's static device scratch
    (no workspace, nothing allocated)."""
    _require_cuda(q, o, k_cache, v_cache, cache_len, route, k_new, v_new, lse)
    batch, hq, d = q.shape
    hkv, max_cache = k_cache.shape[1], k_cache.shape[2]
    keep, rh = _host_u8(route_host)
    _check(lib().fa_attn_decode_noalloc(
        _ptr(q), _ptr(o), _ptr(lse), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        max_cache, _ptr(cache_len), _dtype_code(q), batch, hq, hkv, d, _ptr(route), rh,
        route.shape[1], layer, sink_tokens, window_tokens, block_tokens, float(sm_scale),
        _stream(stream)))
    del keep


def fa_kv_compact(k, v, cu_seqlens, sink_tokens, window_tokens, block_tokens, k_ring, v_ring,
                  stream=None):
    """Build the SA ring caches [B, Hkv, sink + window, d] from prefill K/V [total, Hkv, d]."""
    _require_cuda(k, v, cu_seqlens, k_ring, v_ring)
    batch = cu_seqlens.numel() - 1
    _, hkv, d = k.shape
    _check(lib().fa_kv_compact(
        _ptr(k), _ptr(v), _dtype_code(k), _ptr(cu_seqlens), batch, hkv, d, sink_tokens,
        window_tokens, block_tokens, _ptr(k_ring), _ptr(v_ring), k_ring.shape[2],
        _stream(stream)))


def fa_attn_decode_ring(q, o, k_ring, v_ring, cache_len, sink_tokens, window_tokens,
                        block_tokens, sm_scale, workspace=None, k_new=None, v_new=None, lse=None,
                        stream=None):
    """Decode step of an SA layer over ring caches [B, Hkv, sink + window, d]."""
    import torch
    _require_cuda(q, o, k_ring, v_ring, cache_len, k_new, v_new, lse)
    batch, hq, d = q.shape
    hkv, ring = k_ring.shape[1], k_ring.shape[2]
    if workspace is None:
        n = fa_decode_workspace_size(batch, hq, d, ring)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _check(lib().fa_attn_decode_ring(
        _ptr(q), _ptr(o), _ptr(lse), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring), ring,
        _ptr(cache_len), _dtype_code(q), batch, hq, hkv, d, sink_tokens, window_tokens,
        block_tokens, float(sm_scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
