// fa_launch.h -- host-side launchers of the gfx950 kernels (internal to
// libfluxattn; the public surface is include/fluxattn.h).  Every launcher only
// enqueues on `stream` and returns hipGetLastError() of the launch.  Arguments
// are already validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Route knowledge the host has for one layer: a host copy of the mask lets the
// launcher pick a kernel compiled for all-FA or all-SA batches.
constexpr int kModeMixed = 0;  // read each sequence's bit from the device mask
constexpr int kModeFA = 1;     // every sequence is FA for this layer
constexpr int kModeSA = 2;     // every sequence is SA for this layer
constexpr int kModeXA = 3;     // prefill over kept-block masks (XAttention branch)

struct RouterArgs {
    const void *x_q;
    int x_bf16;
    const int32_t *cu_seqlens;
    int batch, hidden, pool_tokens;
    const float *w1, *b1;
    int router_hidden;
    const float *w2, *b2;
    int n_layers;
    uint8_t *route;
    float *logits;
    float *ws_pool;    // [batch][hidden]
    float *ws_hidden;  // [batch][router_hidden]
};
hipError_t launch_router(const RouterArgs &a, hipStream_t stream);

struct PlanArgs {
    const int32_t *cu_seqlens;
    int batch, max_qblocks;
    const uint8_t *route;
    int n_layers, layer;
    int ns, nw, bk_log2;
    int32_t *plan;
};
hipError_t launch_block_plan(const PlanArgs &a, hipStream_t stream);

struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int bf16;
    const int32_t *cu_seqlens;    // query rows of each sequence
    const int32_t *cu_seqlens_k;  // key rows (the queries are the last rows of the keys)
    int batch, max_seqlen, hq, hkv, d;  // max_seqlen bounds the query rows
    const uint8_t *route;
    int n_layers, layer;
    int ns, nw, bk_log2;
    int nl;  // Triangle attention: dense tail blocks per sequence (0: streaming SA)
    float sm_scale;
    int mode;  // kModeMixed / kModeFA / kModeSA / kModeXA
    // kModeXA: kept-block bits [batch][hq][xa_nqb][xa_nw]; the block size is 1 << bk_log2
    const uint32_t *xa_mask;
    int xa_nqb, xa_nw;
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

struct DecodeArgs {
    const void *q;
    void *o;
    float *lse;
    const void *k_new, *v_new;
    void *k_cache, *v_cache;
    int max_cache;
    const int32_t *cache_len;
    int bf16;
    int batch, hq, hkv, d;
    const uint8_t *route;
    int n_layers, layer;
    int ns, nw, bk_log2;
    float sm_scale;
    int mode;          // kModeMixed / kModeFA / kModeSA
    int ring;          // caches are compact SA rings of max_cache = sink + window rows
    int split_tokens;  // KV tokens per split (multiple of 64)
    int n_splits;      // splits launched per (sequence, kv head)
    float *o_part;     // [batch][hq][n_splits][d]
    float *lse_part;   // [batch][hq][n_splits]
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// The same launch with o_part / lse_part taken from the library's per-device
// static scratch (kDecodeScratchBytes, held until the process ends) instead of
// a caller workspace; the caller has checked that the partials fit.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t launch_decode_noalloc(DecodeArgs a, size_t o_bytes, hipStream_t stream);

struct CompactArgs {
    const void *k, *v;
    int bf16;
    const int32_t *cu_seqlens;
    int batch, hkv, d;
    int ns, nw, bk_log2;
    void *k_ring, *v_ring;
    int ring;  // rows per (sequence, kv head) = sink + window
};
hipError_t launch_kv_compact(const CompactArgs &a, hipStream_t stream);

// XAttention branch: antidiagonal block scores and threshold selection
struct XaScoreArgs {
    const void *q, *k;              // [total][hq][d], [total][hkv][d]
    bool bf16;                      // bf16 (MFMA kernel) or fp32 (VALU kernel)
    const int32_t *cu_seqlens;
    int batch, hq, hkv, d;
    int stride;                     // S; block = 16 S
    int nqb;                        // query blocks per sequence in the score layout
    float sm_scale;
    float *scores;                  // [batch][hq][nqb][nqb]
    void *workspace;                // xa_scores_workspace_bytes(batch, hq, nqb)
};
// Score workspace: one (sum, max) float pair per reshaped row of every cell
// j <= i of every (sequence, head), the cells of query block i starting at cell
// i (i + 1) / 2; then one (max, sum) pair per reshaped row of every (sequence,
// head, query block).  kXaRows reshaped rows (and columns) per block: B = 16 S.
constexpr int kXaRows = 16;
inline size_t xa_part_entries(int batch, int hq, int nqb)
{
    return (size_t)batch * hq * ((size_t)nqb * (nqb + 1) / 2) * kXaRows;
}
inline size_t xa_scores_workspace_bytes(int batch, int hq, int nqb)
{
    return (xa_part_entries(batch, hq, nqb) + (size_t)batch * hq * nqb * kXaRows) *
           (2 * sizeof(float));
}
hipError_t launch_xa_scores(const XaScoreArgs &a, hipStream_t stream);

struct XaSelectArgs {
    const float *scores;
    const int32_t *cu_seqlens;
    int batch, hq, nqb, nw, block;
    float threshold;
    uint32_t *mask;                 // [batch][hq][nqb][nw] kept-block bits
};
hipError_t launch_xa_select(const XaSelectArgs &a, hipStream_t stream);

// Split policy shared by fa_decode_workspace_size and fa_attn_decode; rows =
// batch x query heads.  About 64 splits per (sequence, kv head), or fewer when
// rows is large: min(64, kDecodeSplitRows / rows) above kDecodeShortKept kept
// tokens, so a long-cache layer launches about 2048 workgroups at G = 4 (a few
// rounds at two per CU) rather than up to 16384 short ones, whose partials and
// merge cost more than the finer split balances.  Ranges up to kDecodeShortKept
// tokens (every SA layer) keep about 64.  128..4096 tokens per split, a
// multiple of 64.
constexpr int kDecodeShortKept = 8192;
constexpr int kDecodeSplitRows = 8192;
inline int decode_split_target(int max_kept_tokens, int rows)
{
    if (max_kept_tokens <= kDecodeShortKept) return 64;
    const int t = kDecodeSplitRows / (rows > 0 ? rows : 1);
    return t < 1 ? 1 : (t > 64 ? 64 : t);
}
inline int decode_split_tokens(int max_kept_tokens, int rows)
{
    const int target = decode_split_target(max_kept_tokens, rows);
    int st = (max_kept_tokens + target - 1) / target;
    st = (st + 63) / 64 * 64;
    if (st < 128) st = 128;
    if (st > 4096) st = 4096;
    return st;
}
inline int decode_n_splits(int max_kept_tokens, int rows)
{
    int st = decode_split_tokens(max_kept_tokens, rows);
    return (max_kept_tokens + st - 1) / st;
}
// The most splits a call with at most max_cache kept tokens can use: 64 (the
// target never exceeds it), or max_cache / 4096 where the split size is capped.
inline int decode_max_splits(int max_cache)
{
    const int c = (max_cache + 4095) / 4096;
    return c > 64 ? c : 64;
}

}  // namespace fa
