// api.cpp -- the C ABI of libfluxattn (include/fluxattn.h): host-side argument
// validation, workspace sizing and dispatch to the gfx950 launchers.
//
// Nothing here touches the GPU before validation has passed, so every error
// path can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "fa_launch.h"
#include "fluxattn.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

fa_status ok()
{
    g_last_error.clear();
    return FA_OK;
}

fa_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(FA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

int ilog2_exact(int v)
{
    int l = 0;
    while ((1 << l) < v) ++l;
    return (1 << l) == v ? l : -1;
}

// Sparse configuration in tokens -> (ns, nw, log2 block); false if invalid.
bool sparse_cfg(int sink, int window, int block, int &ns, int &nw, int &bk_log2)
{
    bk_log2 = ilog2_exact(block);
    if (bk_log2 < 4 || bk_log2 > 7) return false;  // block in {16, 32, 64, 128}
    if (sink < 0 || sink % block != 0) return false;
    if (window < block || window % block != 0) return false;
    ns = sink / block;
    nw = window / block;
    return true;
}

// Route mode of one layer from the optional host copy of the mask.
int route_mode(const uint8_t *route_host, int batch, int n_layers, int layer)
{
    if (!route_host) return fa::kModeMixed;
    int n_fa = 0;
    for (int b = 0; b < batch; ++b)
        if (route_host[(size_t)b * n_layers + layer]) ++n_fa;
    if (n_fa == batch) return fa::kModeFA;
    if (n_fa == 0) return fa::kModeSA;
    return fa::kModeMixed;
}


// Shared by fa_attn_prefill (queries = keys), fa_attn_prefill_kv and
// fa_attn_prefill_triangle (tail_tokens > 0: the last tail_tokens rows of each
// SA sequence keep every key).
fa_status prefill_impl(const char *fn, const void *q, const void *k, const void *v, void *o,
                       float *lse, int32_t dtype, const int32_t *cu_q, const int32_t *cu_k,
                       int32_t batch, int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t head_dim, const uint8_t *route, const uint8_t *route_host,
                       int32_t n_layers, int32_t layer, int32_t sink_tokens,
                       int32_t window_tokens, int32_t block_tokens, int32_t tail_tokens,
                       float sm_scale, void *stream)
{
    if (!q || !k || !v || !o || !cu_q || !route)
        return fail(FA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (batch <= 0 || max_seqlen <= 0)
        return fail(FA_ERR_INVALID_ARG, "%s: batch=%d max_seqlen=%d must be positive", fn, batch,
                    max_seqlen);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_INVALID_ARG,
                    "%s: n_q_heads=%d must be a positive multiple of n_kv_heads=%d", fn,
                    n_q_heads, n_kv_heads);
    if (n_layers <= 0 || layer < 0 || layer >= n_layers)
        return fail(FA_ERR_INVALID_ARG, "%s: layer %d outside [0, %d)", fn, layer, n_layers);
    if (!std::isfinite(sm_scale) || sm_scale <= 0.0f)
        return fail(FA_ERR_INVALID_ARG, "%s: sm_scale must be finite and > 0", fn);
    fa::PrefillArgs a{};
    if (!sparse_cfg(sink_tokens, window_tokens, block_tokens, a.ns, a.nw, a.bk_log2))
        return fail(FA_ERR_INVALID_ARG, "%s: bad sparse config sink=%d window=%d block=%d", fn,
                    sink_tokens, window_tokens, block_tokens);
    if (tail_tokens < 0 || tail_tokens % block_tokens != 0)
        return fail(FA_ERR_INVALID_ARG,
                    "%s: last_q_tokens=%d must be a non-negative multiple of block=%d", fn,
                    tail_tokens, block_tokens);
    a.nl = tail_tokens / block_tokens;
    if (dtype != FA_F32 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F32/FA_BF16", fn, dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.bf16 = dtype == FA_BF16;
    a.cu_seqlens = cu_q;
    a.cu_seqlens_k = cu_k;
    a.batch = batch;
    a.max_seqlen = max_seqlen;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.route = route;
    a.n_layers = n_layers;
    a.layer = layer;
    a.sm_scale = sm_scale;
    a.mode = route_mode(route_host, batch, n_layers, layer);
    return hip_status(fa::launch_prefill(a, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

const char *fa_last_error(void) { return g_last_error.c_str(); }

int32_t fa_abi_version(void) { return 8; }

size_t fa_router_workspace_size(int32_t batch, int32_t hidden, int32_t router_hidden)
{
    if (batch <= 0 || hidden <= 0 || router_hidden <= 0) return 0;
    return round256((size_t)batch * hidden * sizeof(float)) +
           round256((size_t)batch * router_hidden * sizeof(float));
}

fa_status fa_router_decide(const void *x_q, int32_t x_dtype, const int32_t *cu_seqlens,
                           int32_t batch, int32_t hidden, int32_t pool_tokens, const float *w1,
                           const float *b1, int32_t router_hidden, const float *w2,
                           const float *b2, int32_t n_layers, uint8_t *route, float *logits,
                           void *workspace, size_t ws_bytes, void *stream)
{
    if (!x_q || !cu_seqlens || !w1 || !b1 || !w2 || !b2 || !route)
        return fail(FA_ERR_INVALID_ARG, "fa_router_decide: a required pointer is NULL");
    if (batch <= 0 || hidden <= 0 || router_hidden <= 0 || n_layers <= 0 || pool_tokens <= 0)
        return fail(FA_ERR_INVALID_ARG,
                    "fa_router_decide: batch=%d hidden=%d router_hidden=%d n_layers=%d "
                    "pool_tokens=%d must all be positive",
                    batch, hidden, router_hidden, n_layers, pool_tokens);
    if (x_dtype != FA_F32 && x_dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "fa_router_decide: x_dtype %d is not FA_F32/FA_BF16",
                    x_dtype);
    const size_t need = fa_router_workspace_size(batch, hidden, router_hidden);
    if (!workspace || ws_bytes < need)
        return fail(FA_ERR_WORKSPACE, "fa_router_decide: workspace %zu bytes, need %zu",
                    workspace ? ws_bytes : (size_t)0, need);
    fa::RouterArgs a{};
    a.x_q = x_q;
    a.x_bf16 = x_dtype == FA_BF16;
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.hidden = hidden;
    a.pool_tokens = pool_tokens;
    a.w1 = w1;
    a.b1 = b1;
    a.router_hidden = router_hidden;
    a.w2 = w2;
    a.b2 = b2;
    a.n_layers = n_layers;
    a.route = route;
    a.logits = logits;
    a.ws_pool = (float *)workspace;
    a.ws_hidden = (float *)((char *)workspace + round256((size_t)batch * hidden * sizeof(float)));
    return hip_status(fa::launch_router(a, (hipStream_t)stream), "fa_router_decide");
}

fa_status fa_block_plan(const int32_t *cu_seqlens, int32_t batch, int32_t max_qblocks,
                        const uint8_t *route, int32_t n_layers, int32_t layer,
                        int32_t sink_tokens, int32_t window_tokens, int32_t block_tokens,
                        int32_t *plan, void *stream)
{
    if (!cu_seqlens || !route || !plan)
        return fail(FA_ERR_INVALID_ARG, "fa_block_plan: a required pointer is NULL");
    if (batch <= 0 || max_qblocks <= 0)
        return fail(FA_ERR_INVALID_ARG, "fa_block_plan: batch=%d max_qblocks=%d must be positive",
                    batch, max_qblocks);
    if (n_layers <= 0 || layer < 0 || layer >= n_layers)
        return fail(FA_ERR_INVALID_ARG, "fa_block_plan: layer %d outside [0, %d)", layer, n_layers);
    fa::PlanArgs a{};
    if (!sparse_cfg(sink_tokens, window_tokens, block_tokens, a.ns, a.nw, a.bk_log2))
        return fail(FA_ERR_INVALID_ARG,
                    "fa_block_plan: bad sparse config sink=%d window=%d block=%d", sink_tokens,
                    window_tokens, block_tokens);
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.max_qblocks = max_qblocks;
    a.route = route;
    a.n_layers = n_layers;
    a.layer = layer;
    a.plan = plan;
    return hip_status(fa::launch_block_plan(a, (hipStream_t)stream), "fa_block_plan");
}

fa_status fa_attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse,
                          int32_t dtype, const int32_t *cu_seqlens, int32_t batch,
                          int32_t max_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, const uint8_t *route, const uint8_t *route_host,
                          int32_t n_layers, int32_t layer, int32_t sink_tokens,
                          int32_t window_tokens, int32_t block_tokens, float sm_scale,
                          void *stream)
{
    return prefill_impl("fa_attn_prefill", q, k, v, o, lse, dtype, cu_seqlens, cu_seqlens, batch,
                        max_seqlen, n_q_heads, n_kv_heads, head_dim, route, route_host, n_layers,
                        layer, sink_tokens, window_tokens, block_tokens, 0, sm_scale, stream);
}

fa_status fa_attn_prefill_triangle(const void *q, const void *k, const void *v, void *o,
                                   float *lse, int32_t dtype, const int32_t *cu_seqlens,
                                   int32_t batch, int32_t max_seqlen, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, const uint8_t *route,
                                   const uint8_t *route_host, int32_t n_layers, int32_t layer,
                                   int32_t sink_tokens, int32_t window_tokens,
                                   int32_t block_tokens, int32_t last_q_tokens, float sm_scale,
                                   void *stream)
{
    return prefill_impl("fa_attn_prefill_triangle", q, k, v, o, lse, dtype, cu_seqlens,
                        cu_seqlens, batch, max_seqlen, n_q_heads, n_kv_heads, head_dim, route,
                        route_host, n_layers, layer, sink_tokens, window_tokens, block_tokens,
                        last_q_tokens, sm_scale, stream);
}

fa_status fa_attn_prefill_kv(const void *q, const void *k, const void *v, void *o, float *lse,
                             int32_t dtype, const int32_t *cu_seqlens_q,
                             const int32_t *cu_seqlens_k, int32_t batch, int32_t max_seqlen_q,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                             const uint8_t *route, const uint8_t *route_host, int32_t n_layers,
                             int32_t layer, int32_t sink_tokens, int32_t window_tokens,
                             int32_t block_tokens, float sm_scale, void *stream)
{
    if (!cu_seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "fa_attn_prefill_kv: a required pointer is NULL");
    return prefill_impl("fa_attn_prefill_kv", q, k, v, o, lse, dtype, cu_seqlens_q, cu_seqlens_k,
                        batch, max_seqlen_q, n_q_heads, n_kv_heads, head_dim, route, route_host,
                        n_layers, layer, sink_tokens, window_tokens, block_tokens, 0, sm_scale,
                        stream);
}

size_t fa_xattn_workspace_size(int32_t batch, int32_t n_q_heads, int32_t n_qblocks)
{
    if (batch <= 0 || n_q_heads <= 0 || n_qblocks <= 0 || n_qblocks > 4096) return 0;
    return round256(fa::xa_scores_workspace_bytes(batch, n_q_heads, n_qblocks));
}

fa_status fa_xattn_scores(const void *q, const void *k, int32_t dtype,
                          const int32_t *cu_seqlens, int32_t batch, int32_t max_seqlen,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_tokens, int32_t stride, float sm_scale, float *scores,
                          int32_t n_qblocks, void *workspace, size_t ws_bytes, void *stream)
{
    const char *fn = "fa_xattn_scores";
    if (!q || !k || !cu_seqlens || !scores)
        return fail(FA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (batch <= 0 || max_seqlen <= 0)
        return fail(FA_ERR_INVALID_ARG, "%s: batch=%d max_seqlen=%d must be positive", fn, batch,
                    max_seqlen);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_INVALID_ARG,
                    "%s: n_q_heads=%d must be a positive multiple of n_kv_heads=%d", fn,
                    n_q_heads, n_kv_heads);
    if (!std::isfinite(sm_scale) || sm_scale <= 0.0f)
        return fail(FA_ERR_INVALID_ARG, "%s: sm_scale must be finite and > 0", fn);
    if (stride != 4 && stride != 8)
        return fail(FA_ERR_UNSUPPORTED, "%s: stride %d not in {4, 8}", fn, stride);
    if (block_tokens != 16 * stride)
        return fail(FA_ERR_INVALID_ARG, "%s: block %d must be 16 * stride = %d", fn, block_tokens,
                    16 * stride);
    const int64_t need = ((int64_t)max_seqlen + block_tokens - 1) / block_tokens;
    if (n_qblocks < need || n_qblocks > 4096)
        return fail(FA_ERR_INVALID_ARG, "%s: n_qblocks %d must be in [%lld, 4096]", fn, n_qblocks,
                    (long long)need);
    if (dtype != FA_BF16 && dtype != FA_F32)
        return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F32/FA_BF16", fn, dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
    const int G = n_q_heads / n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(FA_ERR_UNSUPPORTED, "%s: GQA ratio %d not in {1,2,4,8,16}", fn, G);
    const size_t ws_need = fa_xattn_workspace_size(batch, n_q_heads, n_qblocks);
    if (!workspace || ws_bytes < ws_need)
        return fail(FA_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                    workspace ? ws_bytes : (size_t)0, ws_need);
    fa::XaScoreArgs a{};
    a.workspace = workspace;
    a.bf16 = dtype == FA_BF16;
    a.q = q;
    a.k = k;
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.stride = stride;
    a.nqb = n_qblocks;
    a.sm_scale = sm_scale;
    a.scores = scores;
    return hip_status(fa::launch_xa_scores(a, (hipStream_t)stream), fn);
}

fa_status fa_xattn_select(const float *scores, const int32_t *cu_seqlens, int32_t batch,
                          int32_t n_q_heads, int32_t n_qblocks, int32_t block_tokens,
                          float threshold, uint32_t *mask, void *stream)
{
    const char *fn = "fa_xattn_select";
    if (!scores || !cu_seqlens || !mask)
        return fail(FA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (batch <= 0 || n_q_heads <= 0 || block_tokens <= 0)
        return fail(FA_ERR_INVALID_ARG, "%s: batch=%d heads=%d block=%d must be positive", fn,
                    batch, n_q_heads, block_tokens);
    if (n_qblocks <= 0 || n_qblocks > 4096)
        return fail(FA_ERR_INVALID_ARG, "%s: n_qblocks %d not in [1, 4096]", fn, n_qblocks);
    if (!std::isfinite(threshold) || threshold <= 0.0f)
        return fail(FA_ERR_INVALID_ARG, "%s: threshold must be finite and > 0", fn);
    fa::XaSelectArgs a{};
    a.scores = scores;
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.hq = n_q_heads;
    a.nqb = n_qblocks;
    a.nw = (n_qblocks + 31) / 32;
    a.block = block_tokens;
    a.threshold = threshold;
    a.mask = mask;
    return hip_status(fa::launch_xa_select(a, (hipStream_t)stream), fn);
}

fa_status fa_attn_prefill_xattn(const void *q, const void *k, const void *v, void *o,
                                float *lse, int32_t dtype, const int32_t *cu_seqlens,
                                int32_t batch, int32_t max_seqlen, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim, int32_t block_tokens,
                                const uint32_t *mask, int32_t n_qblocks, float sm_scale,
                                void *stream)
{
    const char *fn = "fa_attn_prefill_xattn";
    if (!q || !k || !v || !o || !cu_seqlens || !mask)
        return fail(FA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (batch <= 0 || max_seqlen <= 0)
        return fail(FA_ERR_INVALID_ARG, "%s: batch=%d max_seqlen=%d must be positive", fn, batch,
                    max_seqlen);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_INVALID_ARG,
                    "%s: n_q_heads=%d must be a positive multiple of n_kv_heads=%d", fn,
                    n_q_heads, n_kv_heads);
    if (!std::isfinite(sm_scale) || sm_scale <= 0.0f)
        return fail(FA_ERR_INVALID_ARG, "%s: sm_scale must be finite and > 0", fn);
    if (block_tokens != 64 && block_tokens != 128)
        return fail(FA_ERR_INVALID_ARG, "%s: block %d not in {64, 128}", fn, block_tokens);
    const int64_t need = ((int64_t)max_seqlen + block_tokens - 1) / block_tokens;
    if (n_qblocks < need || n_qblocks > 4096)
        return fail(FA_ERR_INVALID_ARG, "%s: n_qblocks %d must be in [%lld, 4096]", fn, n_qblocks,
                    (long long)need);
    if (dtype != FA_F32 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F32/FA_BF16", fn, dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
    fa::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.bf16 = dtype == FA_BF16;
    a.cu_seqlens = cu_seqlens;
    a.cu_seqlens_k = cu_seqlens;
    a.batch = batch;
    a.max_seqlen = max_seqlen;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.route = nullptr;
    a.n_layers = 1;
    a.layer = 0;
    a.ns = 0;
    a.nw = 1;
    a.bk_log2 = block_tokens == 64 ? 6 : 7;
    a.sm_scale = sm_scale;
    a.mode = fa::kModeXA;
    a.xa_mask = mask;
    a.xa_nqb = n_qblocks;
    a.xa_nw = (n_qblocks + 31) / 32;
    return hip_status(fa::launch_prefill(a, (hipStream_t)stream), fn);
}

size_t fa_decode_workspace_size(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                int32_t max_cache)
{
    if (batch <= 0 || n_q_heads <= 0 || head_dim <= 0 || max_cache <= 0) return 0;
    const size_t rows = (size_t)batch * n_q_heads * fa::decode_max_splits(max_cache);
    return round256(rows * head_dim * sizeof(float)) + round256(rows * sizeof(float));
}

}  // extern "C"

namespace {

fa_status decode_impl(const char *fn, bool ring, bool noalloc, const void *q, void *o, float *lse,
                      const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                      int32_t max_cache, const int32_t *cache_len, int32_t dtype, int32_t batch,
                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      const uint8_t *route, const uint8_t *route_host, int32_t n_layers,
                      int32_t layer, int32_t sink_tokens, int32_t window_tokens,
                      int32_t block_tokens, float sm_scale, void *workspace, size_t ws_bytes,
                      void *stream)
{
    if (!q || !o || !k_cache || !v_cache || !cache_len || (!ring && !route))
        return fail(FA_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(FA_ERR_INVALID_ARG, "%s: give both k_new and v_new, or neither", fn);
    if (batch <= 0 || max_cache <= 0)
        return fail(FA_ERR_INVALID_ARG, "%s: batch=%d cache rows=%d must be positive", fn, batch,
                    max_cache);
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_INVALID_ARG,
                    "%s: n_q_heads=%d must be a positive multiple of n_kv_heads=%d", fn,
                    n_q_heads, n_kv_heads);
    if (!ring && (n_layers <= 0 || layer < 0 || layer >= n_layers))
        return fail(FA_ERR_INVALID_ARG, "%s: layer %d outside [0, %d)", fn, layer, n_layers);
    if (!std::isfinite(sm_scale) || sm_scale <= 0.0f)
        return fail(FA_ERR_INVALID_ARG, "%s: sm_scale must be finite and > 0", fn);
    fa::DecodeArgs a{};
    if (!sparse_cfg(sink_tokens, window_tokens, block_tokens, a.ns, a.nw, a.bk_log2))
        return fail(FA_ERR_INVALID_ARG, "%s: bad sparse config sink=%d window=%d block=%d", fn,
                    sink_tokens, window_tokens, block_tokens);
    if (ring && max_cache != sink_tokens + window_tokens)
        return fail(FA_ERR_INVALID_ARG, "%s: ring_tokens=%d must equal sink + window = %d", fn,
                    max_cache, sink_tokens + window_tokens);
    if (dtype != FA_F32 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "%s: dtype %d is not FA_F32/FA_BF16", fn, dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
    const int G = n_q_heads / n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(FA_ERR_UNSUPPORTED, "%s: GQA ratio %d not in {1,2,4,8,16}", fn, G);

    // Grid sizing: kept tokens per sequence are at most max_cache, or at most
    // sink + window for an SA layer.
    a.ring = ring ? 1 : 0;
    a.mode = ring ? fa::kModeSA : route_mode(route_host, batch, n_layers, layer);
    int max_kept = max_cache;
    if (a.mode == fa::kModeSA && sink_tokens + window_tokens < max_kept)
        max_kept = sink_tokens + window_tokens;
    a.split_tokens = fa::decode_split_tokens(max_kept, batch * n_q_heads);
    a.n_splits = fa::decode_n_splits(max_kept, batch * n_q_heads);
    const size_t rows = (size_t)batch * n_q_heads * a.n_splits;
    const size_t o_bytes = round256(rows * head_dim * sizeof(float));
    const size_t need = o_bytes + round256(rows * sizeof(float));
    if (noalloc && need > fa::kDecodeScratchBytes)
        return fail(FA_ERR_WORKSPACE,
                    "%s: the split partials need %zu bytes, above the %zu bytes of static "
                    "scratch (batch x query heads x splits too large)",
                    fn, need, fa::kDecodeScratchBytes);
    if (!noalloc && (!workspace || ws_bytes < need))
        return fail(FA_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                    workspace ? ws_bytes : (size_t)0, need);
    a.q = q;
    a.o = o;
    a.lse = lse;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.max_cache = max_cache;
    a.cache_len = cache_len;
    a.bf16 = dtype == FA_BF16;
    a.batch = batch;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.route = route;
    a.n_layers = ring ? 1 : n_layers;
    a.layer = ring ? 0 : layer;
    a.sm_scale = sm_scale;
    if (noalloc)
        return hip_status(fa::launch_decode_noalloc(a, o_bytes, (hipStream_t)stream), fn);
    a.o_part = (float *)workspace;
    a.lse_part = (float *)((char *)workspace + o_bytes);
    return hip_status(fa::launch_decode(a, (hipStream_t)stream), fn);
}

}  // namespace

extern "C" {

fa_status fa_attn_decode(const void *q, void *o, float *lse, const void *k_new, const void *v_new,
                         void *k_cache, void *v_cache, int32_t max_cache,
                         const int32_t *cache_len, int32_t dtype, int32_t batch,
                         int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                         const uint8_t *route, const uint8_t *route_host, int32_t n_layers,
                         int32_t layer, int32_t sink_tokens, int32_t window_tokens,
                         int32_t block_tokens, float sm_scale, void *workspace, size_t ws_bytes,
                         void *stream)
{
    return decode_impl("fa_attn_decode", false, false, q, o, lse, k_new, v_new, k_cache,
                       v_cache, max_cache, cache_len, dtype, batch, n_q_heads, n_kv_heads,
                       head_dim, route, route_host, n_layers, layer, sink_tokens, window_tokens,
                       block_tokens, sm_scale, workspace, ws_bytes, stream);
}

fa_status fa_attn_decode_noalloc(const void *q, void *o, float *lse, const void *k_new,
                                 const void *v_new, void *k_cache, void *v_cache,
                                 int32_t max_cache, const int32_t *cache_len, int32_t dtype,
                                 int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const uint8_t *route,
                                 const uint8_t *route_host, int32_t n_layers, int32_t layer,
                                 int32_t sink_tokens, int32_t window_tokens,
                                 int32_t block_tokens, float sm_scale, void *stream)
{
    return decode_impl("fa_attn_decode_noalloc", false, true, q, o, lse, k_new, v_new, k_cache,
                       v_cache, max_cache, cache_len, dtype, batch, n_q_heads, n_kv_heads,
                       head_dim, route, route_host, n_layers, layer, sink_tokens, window_tokens,
                       block_tokens, sm_scale, nullptr, 0, stream);
}

fa_status fa_attn_decode_ring(const void *q, void *o, float *lse, const void *k_new,
                              const void *v_new, void *k_ring, void *v_ring, int32_t ring_tokens,
                              const int32_t *cache_len, int32_t dtype, int32_t batch,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              int32_t sink_tokens, int32_t window_tokens, int32_t block_tokens,
                              float sm_scale, void *workspace, size_t ws_bytes, void *stream)
{
    return decode_impl("fa_attn_decode_ring", true, false, q, o, lse, k_new, v_new, k_ring, v_ring,
                       ring_tokens, cache_len, dtype, batch, n_q_heads, n_kv_heads, head_dim,
                       nullptr, nullptr, 1, 0, sink_tokens, window_tokens, block_tokens, sm_scale,
                       workspace, ws_bytes, stream);
}

fa_status fa_kv_compact(const void *k, const void *v, int32_t dtype, const int32_t *cu_seqlens,
                        int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t sink_tokens,
                        int32_t window_tokens, int32_t block_tokens, void *k_ring, void *v_ring,
                        int32_t ring_tokens, void *stream)
{
    if (!k || !v || !cu_seqlens || !k_ring || !v_ring)
        return fail(FA_ERR_INVALID_ARG, "fa_kv_compact: a required pointer is NULL");
    if (batch <= 0 || n_kv_heads <= 0)
        return fail(FA_ERR_INVALID_ARG, "fa_kv_compact: batch=%d n_kv_heads=%d must be positive",
                    batch, n_kv_heads);
    fa::CompactArgs a{};
    if (!sparse_cfg(sink_tokens, window_tokens, block_tokens, a.ns, a.nw, a.bk_log2))
        return fail(FA_ERR_INVALID_ARG, "fa_kv_compact: bad sparse config sink=%d window=%d block=%d",
                    sink_tokens, window_tokens, block_tokens);
    if (ring_tokens != sink_tokens + window_tokens)
        return fail(FA_ERR_INVALID_ARG, "fa_kv_compact: ring_tokens=%d must equal sink + window = %d",
                    ring_tokens, sink_tokens + window_tokens);
    if (dtype != FA_F32 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "fa_kv_compact: dtype %d is not FA_F32/FA_BF16", dtype);
    if (head_dim != 64 && head_dim != 128)
        return fail(FA_ERR_UNSUPPORTED, "fa_kv_compact: head_dim %d not in {64, 128}", head_dim);
    a.k = k;
    a.v = v;
    a.bf16 = dtype == FA_BF16;
    a.cu_seqlens = cu_seqlens;
    a.batch = batch;
    a.hkv = n_kv_heads;
    a.d = head_dim;
    a.k_ring = k_ring;
    a.v_ring = v_ring;
    a.ring = ring_tokens;
    return hip_status(fa::launch_kv_compact(a, (hipStream_t)stream), "fa_kv_compact");
}

}  // extern "C"
