"""MI355X-native (gfx950) layer-routed hybrid attention: the hot path of Flux Attention.

The library is libfluxattn.so (C ABI: include/fluxattn.h), built from csrc/ by
``python -m sparse_attention_layerrouter_amd.build``.  ``_lib`` is its thin
ctypes binding; ``synth`` draws the seeded synthetic inputs.
"""
from ._lib import (  # noqa: F401
    FA_BF16, FA_ERR_HIP, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_F32,
    FA_OK, FluxAttnError, fa_abi_version, fa_attn_decode, fa_attn_prefill, fa_block_plan,
    fa_attn_decode_ring, fa_attn_decode_noalloc, fa_attn_prefill_kv, fa_decode_workspace_size, fa_kv_compact,
    fa_router_decide, fa_xattn_scores, fa_xattn_select, fa_attn_prefill_xattn,
    fa_attn_prefill_triangle, fa_xattn_workspace_size,
    fa_router_workspace_size, last_error, lib,
)
