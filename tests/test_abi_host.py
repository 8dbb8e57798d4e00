"""Host-only checks of the C ABI (no GPU needed).

The library must load and export every entry point include/fluxattn.h
declares; every validation error must be returned before anything touches the
GPU, so each one is forced here with placeholder pointers that are never
dereferenced.
"""
import os
import re

import pytest

from sparse_attention_layerrouter_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fluxattn.h")

P = 0x1000  # placeholder non-NULL pointer, never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert len(names) == 17, names
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_abi_version_and_clean_error_state():
    assert _lib.fa_abi_version() == 8


def test_workspace_sizes():
    assert _lib.fa_router_workspace_size(1, 4096, 256) == 4096 * 4 + 256 * 4
    assert _lib.fa_router_workspace_size(0, 4096, 256) == 0
    # 64 splits minimum, (d + 1) floats per split row, 256-byte aligned parts
    n = _lib.fa_decode_workspace_size(8, 32, 128, 131072)
    assert n == 8 * 32 * 64 * 128 * 4 + 8 * 32 * 64 * 4
    assert _lib.fa_decode_workspace_size(8, 32, 128, 0) == 0
    # longer caches need more splits once the 4096-token split cap binds
    assert _lib.fa_decode_workspace_size(1, 1, 128, 1 << 20) > _lib.fa_decode_workspace_size(
        1, 1, 128, 1 << 17)
    assert _lib.fa_decode_workspace_size(8, 32, 128, 1 << 20) == (
        8 * 32 * 256 * 128 * 4 + 8 * 32 * 256 * 4)


def prefill_args(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, dtype=1, cu=P, batch=1, max_seqlen=256, hq=32,
             hkv=8, d=128, route=P, route_host=None, n_layers=2, layer=0, sink=128,
             window=2048, block=64, scale=0.088, stream=None)
    a.update(kw)
    return [a[k] for k in ("q", "k", "v", "o", "lse", "dtype", "cu", "batch", "max_seqlen",
                           "hq", "hkv", "d", "route", "route_host", "n_layers", "layer", "sink",
                           "window", "block", "scale", "stream")]


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(route=None), _lib.FA_ERR_INVALID_ARG),
    (dict(batch=0), _lib.FA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), _lib.FA_ERR_INVALID_ARG),
    (dict(hq=30, hkv=8), _lib.FA_ERR_INVALID_ARG),
    (dict(hkv=0), _lib.FA_ERR_INVALID_ARG),
    (dict(layer=2), _lib.FA_ERR_INVALID_ARG),
    (dict(layer=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(sink=100), _lib.FA_ERR_INVALID_ARG),   # not a multiple of the block
    (dict(window=32), _lib.FA_ERR_INVALID_ARG),  # smaller than one block
    (dict(block=48), _lib.FA_ERR_INVALID_ARG),   # not a power of two
    (dict(block=256, window=256, sink=0), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.FA_ERR_UNSUPPORTED),
])
def test_prefill_validation(kw, status):
    assert _lib.lib().fa_attn_prefill(*prefill_args(**kw)) == status
    assert _lib.last_error().startswith("fa_attn_prefill")


def prefill_kv_args(cu_k=P, **kw):
    a = prefill_args(**kw)
    return a[:7] + [cu_k] + a[7:]


@pytest.mark.parametrize("kw,status", [
    (dict(cu_k=None), _lib.FA_ERR_INVALID_ARG),
    (dict(cu=None), _lib.FA_ERR_INVALID_ARG),
    (dict(max_seqlen=0), _lib.FA_ERR_INVALID_ARG),
    (dict(hq=30, hkv=8), _lib.FA_ERR_INVALID_ARG),
    (dict(layer=2), _lib.FA_ERR_INVALID_ARG),
    (dict(sink=100), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
])
def test_prefill_kv_validation(kw, status):
    assert _lib.lib().fa_attn_prefill_kv(*prefill_kv_args(**kw)) == status
    assert _lib.last_error().startswith("fa_attn_prefill_kv")


def prefill_triangle_args(last_q=128, **kw):
    a = prefill_args(**kw)
    return a[:19] + [last_q] + a[19:]


@pytest.mark.parametrize("kw,status", [
    (dict(last_q=-64), _lib.FA_ERR_INVALID_ARG),
    (dict(last_q=100), _lib.FA_ERR_INVALID_ARG),    # not a multiple of the block
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(window=100), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.FA_ERR_INVALID_ARG),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.FA_ERR_UNSUPPORTED),
])
def test_prefill_triangle_validation(kw, status):
    assert _lib.lib().fa_attn_prefill_triangle(*prefill_triangle_args(**kw)) == status
    assert _lib.last_error().startswith("fa_attn_prefill_triangle")


def decode_args(**kw):
    a = dict(q=P, o=P, lse=None, k_new=None, v_new=None, kc=P, vc=P, max_cache=4096, cl=P,
             dtype=1, batch=2, hq=32, hkv=8, d=128, route=P, route_host=None, n_layers=32,
             layer=3, sink=128, window=2048, block=64, scale=0.088, ws=P, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return [a[k] for k in ("q", "o", "lse", "k_new", "v_new", "kc", "vc", "max_cache", "cl",
                           "dtype", "batch", "hq", "hkv", "d", "route", "route_host",
                           "n_layers", "layer", "sink", "window", "block", "scale", "ws",
                           "ws_bytes", "stream")]


@pytest.mark.parametrize("kw,status", [
    (dict(kc=None), _lib.FA_ERR_INVALID_ARG),
    (dict(cl=None), _lib.FA_ERR_INVALID_ARG),
    (dict(k_new=P), _lib.FA_ERR_INVALID_ARG),   # v_new missing
    (dict(max_cache=0), _lib.FA_ERR_INVALID_ARG),
    (dict(hq=12, hkv=8), _lib.FA_ERR_INVALID_ARG),
    (dict(layer=32), _lib.FA_ERR_INVALID_ARG),
    (dict(window=0), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), _lib.FA_ERR_INVALID_ARG),
    (dict(d=80), _lib.FA_ERR_UNSUPPORTED),
    (dict(hq=24, hkv=8), _lib.FA_ERR_UNSUPPORTED),  # G = 3
    (dict(hq=64, hkv=2), _lib.FA_ERR_UNSUPPORTED),  # G = 32
    (dict(ws=None), _lib.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.FA_ERR_WORKSPACE),
])
def test_decode_validation(kw, status):
    assert _lib.lib().fa_attn_decode(*decode_args(**kw)) == status
    assert _lib.last_error().startswith("fa_attn_decode")


@pytest.mark.parametrize("kw,status", [
    (dict(kc=None), _lib.FA_ERR_INVALID_ARG),
    (dict(k_new=P), _lib.FA_ERR_INVALID_ARG),   # v_new missing
    (dict(layer=32), _lib.FA_ERR_INVALID_ARG),
    (dict(d=80), _lib.FA_ERR_UNSUPPORTED),
    # partials above the 64 MiB static scratch: 512 x 32 heads x 256 splits of 4096
    # tokens x 129 x 4 B
    (dict(batch=512, max_cache=1 << 20), _lib.FA_ERR_WORKSPACE),
])
def test_decode_noalloc_validation(kw, status):
    """The no-allocation variant validates like fa_attn_decode and refuses split
    partials larger than its static scratch, before touching the GPU."""
    a = decode_args(**kw)
    del a[22:24]  # no workspace, no ws_bytes
    assert _lib.lib().fa_attn_decode_noalloc(*a) == status
    assert _lib.last_error().startswith("fa_attn_decode_noalloc")


def test_decode_workspace_matches_sizing_function():
    need = _lib.fa_decode_workspace_size(2, 32, 128, 4096)
    # one byte short of the advertised size must still be enough for the all-FA grid
    # (the advertised size has headroom); zero must fail
    assert _lib.lib().fa_attn_decode(*decode_args(ws_bytes=0)) == _lib.FA_ERR_WORKSPACE
    assert need >= 2 * 32 * 64 * 129 * 4


def router_args(**kw):
    a = dict(x=P, dt=1, cu=P, batch=1, hidden=4096, pool=64, w1=P, b1=P, hr=256, w2=P, b2=P,
             L=32, route=P, logits=None, ws=P, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return [a[k] for k in ("x", "dt", "cu", "batch", "hidden", "pool", "w1", "b1", "hr", "w2",
                           "b2", "L", "route", "logits", "ws", "ws_bytes", "stream")]


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.FA_ERR_INVALID_ARG),
    (dict(w2=None), _lib.FA_ERR_INVALID_ARG),
    (dict(route=None), _lib.FA_ERR_INVALID_ARG),
    (dict(batch=0), _lib.FA_ERR_INVALID_ARG),
    (dict(pool=0), _lib.FA_ERR_INVALID_ARG),
    (dict(L=0), _lib.FA_ERR_INVALID_ARG),
    (dict(dt=3), _lib.FA_ERR_UNSUPPORTED),
    (dict(ws=None), _lib.FA_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.FA_ERR_WORKSPACE),
])
def test_router_validation(kw, status):
    assert _lib.lib().fa_router_decide(*router_args(**kw)) == status
    assert _lib.last_error().startswith("fa_router_decide")


@pytest.mark.parametrize("kw", [
    dict(cu=None), dict(batch=0), dict(mq=0), dict(layer=5), dict(sink=8), dict(block=8),
])
def test_block_plan_validation(kw):
    a = dict(cu=P, batch=1, mq=16, route=P, L=2, layer=0, sink=16, window=64, block=16,
             plan=P, stream=None)
    a.update(kw)
    args = [a[k] for k in ("cu", "batch", "mq", "route", "L", "layer", "sink", "window",
                           "block", "plan", "stream")]
    assert _lib.lib().fa_block_plan(*args) == _lib.FA_ERR_INVALID_ARG
    assert _lib.last_error().startswith("fa_block_plan")


@pytest.mark.parametrize("kw,status", [
    (dict(kr=None), _lib.FA_ERR_INVALID_ARG),
    (dict(ring=2000), _lib.FA_ERR_INVALID_ARG),      # not sink + window
    (dict(block=24), _lib.FA_ERR_INVALID_ARG),
    (dict(batch=0), _lib.FA_ERR_INVALID_ARG),
    (dict(d=32), _lib.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), _lib.FA_ERR_UNSUPPORTED),
])
def test_kv_compact_validation(kw, status):
    a = dict(k=P, v=P, dtype=1, cu=P, batch=2, hkv=8, d=128, sink=128, window=2048, block=64,
             kr=P, vr=P, ring=2176, stream=None)
    a.update(kw)
    args = [a[k] for k in ("k", "v", "dtype", "cu", "batch", "hkv", "d", "sink", "window",
                           "block", "kr", "vr", "ring", "stream")]
    assert _lib.lib().fa_kv_compact(*args) == status
    assert _lib.last_error().startswith("fa_kv_compact")


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(ring=4096), _lib.FA_ERR_INVALID_ARG),      # not sink + window
    (dict(k_new=P), _lib.FA_ERR_INVALID_ARG),
    (dict(hq=30), _lib.FA_ERR_INVALID_ARG),
    (dict(d=48), _lib.FA_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), _lib.FA_ERR_WORKSPACE),
])
def test_decode_ring_validation(kw, status):
    a = dict(q=P, o=P, lse=None, k_new=None, v_new=None, kr=P, vr=P, ring=2176, cl=P, dtype=1,
             batch=2, hq=32, hkv=8, d=128, sink=128, window=2048, block=64, scale=0.088, ws=P,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    args = [a[k] for k in ("q", "o", "lse", "k_new", "v_new", "kr", "vr", "ring", "cl", "dtype",
                           "batch", "hq", "hkv", "d", "sink", "window", "block", "scale", "ws",
                           "ws_bytes", "stream")]
    assert _lib.lib().fa_attn_decode_ring(*args) == status
    assert _lib.last_error().startswith("fa_attn_decode_ring")


def test_xattn_workspace_size():
    # 16 (max, sum) float2 pairs per (head, cell j <= i) plus 16 per (head, query block)
    nqb = 1024
    raw = (8 * 32 * (nqb * (nqb + 1) // 2) * 16 + 8 * 32 * nqb * 16) * 8
    assert _lib.fa_xattn_workspace_size(8, 32, nqb) == (raw + 255) // 256 * 256
    assert _lib.fa_xattn_workspace_size(1, 1, 1) == 256
    assert _lib.fa_xattn_workspace_size(0, 32, 16) == 0
    assert _lib.fa_xattn_workspace_size(1, 32, 4097) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(scores=None), _lib.FA_ERR_INVALID_ARG),
    (dict(batch=0), _lib.FA_ERR_INVALID_ARG),
    (dict(hq=30), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(block=64), _lib.FA_ERR_INVALID_ARG),       # not 16 * stride
    (dict(nqb=7), _lib.FA_ERR_INVALID_ARG),          # fewer than ceil(1000 / 128)
    (dict(nqb=4097), _lib.FA_ERR_INVALID_ARG),
    (dict(stride=2, block=32), _lib.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), _lib.FA_ERR_UNSUPPORTED),
    (dict(d=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(hq=24, hkv=8), _lib.FA_ERR_UNSUPPORTED),   # G = 3
    (dict(ws=None), _lib.FA_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.FA_ERR_WORKSPACE),
])
def test_xattn_scores_validation(kw, status):
    a = dict(q=P, k=P, dtype=1, cu=P, batch=1, max_seqlen=1000, hq=32, hkv=8, d=128, block=128,
             stride=8, scale=0.088, scores=P, nqb=8, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    args = [a[k] for k in ("q", "k", "dtype", "cu", "batch", "max_seqlen", "hq", "hkv", "d",
                           "block", "stride", "scale", "scores", "nqb", "ws", "ws_bytes",
                           "stream")]
    assert _lib.lib().fa_xattn_scores(*args) == status
    assert _lib.last_error().startswith("fa_xattn_scores")


@pytest.mark.parametrize("kw", [dict(scores=None), dict(batch=0), dict(nqb=0), dict(nqb=4097),
                                dict(threshold=0.0), dict(threshold=float("nan"))])
def test_xattn_select_validation(kw):
    a = dict(scores=P, cu=P, batch=1, hq=32, nqb=8, block=128, threshold=0.9, mask=P,
             stream=None)
    a.update(kw)
    args = [a[k] for k in ("scores", "cu", "batch", "hq", "nqb", "block", "threshold", "mask",
                           "stream")]
    assert _lib.lib().fa_xattn_select(*args) == _lib.FA_ERR_INVALID_ARG
    assert _lib.last_error().startswith("fa_xattn_select")
