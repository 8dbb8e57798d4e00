/*
 * fluxattn.h -- C ABI of the MI355X (gfx950) layer-routed hybrid attention
 * library (libfluxattn.so).
 *
 * Method: Flux Attention ("Flux Attention: Context-Aware Hybrid Attention for
 * Efficient LLMs Inference").  A lightweight Layer Router reads the query
 * hidden states x_Q and sends every layer to Full Attention (FA) or Sparse
 * Attention (SA) [HF model card, summary paragraph; thelatestinai paper page,
 * Figure 2].  The decision is made once at prefill and reused by decode
 * [thelatestinai paper page, Table 3].  FA is dense causal GQA attention
 * (FlashAttention-2 is the dense path of [thelatestinai paper page, Table 6]);
 * SA is streaming block-sparse attention that keeps the attention-sink blocks
 * plus a local window of blocks (block size / sink size of the same Table 6,
 * and the streaming block-sparse helper named in the codewithpapers function
 * list).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library keeps no pointer after a call returns and allocates no
 *     device memory; scratch space comes in through `workspace`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and returns without
 *     synchronising; results are ready when the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation failure nothing is launched and the call returns
 *     FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED / FA_ERR_WORKSPACE; a launch
 *     failure returns FA_ERR_HIP.  fa_last_error() gives a message for the
 *     calling thread's most recent failure.  Host-side checks cannot see
 *     device-resident values (sequence lengths, cache lengths); their device
 *     behaviour is stated per entry point.
 *   - dtype: FA_F32 (float) or FA_BF16 (bfloat16 bits).  Attention math
 *     accumulates in fp32 in both cases.  Router weights are always fp32.
 *   - Route mask: uint8 route[batch][n_layers], 1 = FA, 0 = SA (any nonzero
 *     value counts as FA).
 *   - Sparse configuration (tokens): block_tokens in {16, 32, 64, 128};
 *     sink_tokens >= 0 and window_tokens >= block_tokens, both multiples of
 *     block_tokens.  With ns = sink/block and nw = window/block, a query at
 *     position t (query block i = t / block) of an SA layer sees key s iff
 *     s <= t and (s / block < ns or s / block >= i - nw + 1): the window counts
 *     whole blocks including the query's own block.  FA layers see every
 *     s <= t.  Positions restart at 0 in every sequence.
 */
#ifndef FLUXATTN_H
#define FLUXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* bad shape, pointer, index or sparse config */
    FA_ERR_UNSUPPORTED = 2, /* valid but not compiled: head_dim, dtype, GQA ratio */
    FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    FA_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/* Message for the calling thread's most recent failure ("" if none).  The
 * pointer stays valid until the next call on the same thread. */
const char *fa_last_error(void);

/* ABI version of this header (increments on any signature change). */
int32_t fa_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Layer Router                                                             */
/* ------------------------------------------------------------------------ */

/*
 * Bytes of workspace fa_router_decide needs: (batch*hidden + batch*router_hidden)
 * floats, rounded up to 256 B.
 */
size_t fa_router_workspace_size(int32_t batch, int32_t hidden,
                                int32_t router_hidden);

/*
 * fa_router_decide -- Layer Router of [thelatestinai paper page, Figure 2]:
 * one FA/SA bit per (sequence, layer) from the query hidden states.
 *
 *   p[b]  = mean of the last P = min(pool_tokens, T_b) rows of x_q[b]
 *           (the suffix pooling budget of [thelatestinai paper page, Figure 8])
 *   h     = ReLU(W1 p + b1)
 *   logit = W2 h + b2
 *   route[b][l] = logit > 0 ? 1 (FA) : 0 (SA)      (NaN -> SA)
 *
 * x_q      [total_tokens][hidden], fp32 or bf16 (x_dtype), packed varlen.
 * cu_seqlens [batch+1] int32, device, prefix sums of the sequence lengths.
 * w1 [router_hidden][hidden], b1 [router_hidden], w2 [n_layers][router_hidden],
 *    b2 [n_layers]: fp32, device.
 * route  [batch][n_layers] uint8 out; logits [batch][n_layers] fp32 out
 *        (nullable).
 * workspace: >= fa_router_workspace_size(batch, hidden, router_hidden) bytes.
 * All sums are fp32 in a fixed order, so repeated calls are bitwise identical.
 * Device behaviour: a sequence with T_b <= 0 gets route 0 and logits NaN.
 * Errors: NULL required pointer, batch/hidden/router_hidden/n_layers <= 0,
 * pool_tokens <= 0 -> FA_ERR_INVALID_ARG; bad x_dtype -> FA_ERR_UNSUPPORTED;
 * small workspace -> FA_ERR_WORKSPACE.
 */
fa_status fa_router_decide(const void *x_q, int32_t x_dtype,
                           const int32_t *cu_seqlens, int32_t batch,
                           int32_t hidden, int32_t pool_tokens,
                           const float *w1, const float *b1,
                           int32_t router_hidden, const float *w2,
                           const float *b2, int32_t n_layers, uint8_t *route,
                           float *logits, void *workspace, size_t ws_bytes,
                           void *stream);

/* ------------------------------------------------------------------------ */
/* Streaming block plan                                                     */
/* ------------------------------------------------------------------------ */

/*
 * fa_block_plan -- kept key blocks of every (sequence, query block) of one
 * layer, the streaming block-sparse layout of [thelatestinai paper page,
 * Table 6] (sink blocks + local window), exported for bit-exact checking.
 * The attention kernels evaluate the same rule internally.
 *
 * plan [batch][max_qblocks][4] int32 out, ascending half-open block ranges
 *   (0, sink_end, win_begin, i + 1):
 *   FA: sink_end = win_begin = i + 1 (one range [0, i+1));
 *   SA: sink_end = min(ns, i + 1), win_begin = max(sink_end, i - nw + 1).
 *   Query blocks at or past ceil(T_b / block) get (0, 0, 0, 0).
 * cu_seqlens [batch+1] int32 device; route [batch][n_layers] uint8 device.
 * Errors: NULL pointer, batch/max_qblocks <= 0, layer outside [0, n_layers),
 * bad sparse config -> FA_ERR_INVALID_ARG.
 */
fa_status fa_block_plan(const int32_t *cu_seqlens, int32_t batch,
                        int32_t max_qblocks, const uint8_t *route,
                        int32_t n_layers, int32_t layer, int32_t sink_tokens,
                        int32_t window_tokens, int32_t block_tokens,
                        int32_t *plan, void *stream);

/* ------------------------------------------------------------------------ */
/* Prefill attention                                                        */
/* ------------------------------------------------------------------------ */

/*
 * fa_attn_prefill -- causal attention of one layer over a packed varlen batch;
 * each sequence runs FA or SA as its route bit for `layer` says.
 *
 *   O[t][h] = sum_s softmax_s(sm_scale * <Q[t][h], K[s][h/G]>) V[s][h/G]
 *   over the visible keys s of the layer's kind; G = n_q_heads / n_kv_heads
 *   (query heads h*G .. h*G+G-1 share KV head h, as `repeat_kv` does).
 *   lse[t][h] = ln sum_s exp(sm_scale * <Q[t][h], K[s][h/G]>).
 *
 * q [total][n_q_heads][head_dim], k, v [total][n_kv_heads][head_dim] (dtype);
 * o [total][n_q_heads][head_dim] out (dtype); lse [total][n_q_heads] fp32 out
 * (nullable).  total = cu_seqlens[batch].
 * max_seqlen: host upper bound of every T_b (sizes the grid; rows of a longer
 * sequence past max_seqlen are not computed).
 * route [batch][n_layers] uint8 device; route_host (nullable) is a host copy of
 *   the same mask: when every sequence has the same bit for `layer`, a kernel
 *   compiled for that kind runs (identical results, no per-sequence branch).
 * Supported: head_dim 64 or 128, any G.  bf16 with G in {1, 2, 4, 8, 16}
 * runs on the MFMA kernel; other bf16 G and all fp32 inputs run on a plain
 * one-thread-per-row kernel (the fp32 correctness path).
 * SA tiles outside the sink and window ranges are never loaded.
 * Errors: NULL pointer, batch/max_seqlen <= 0, heads <= 0, n_q_heads %
 * n_kv_heads != 0, layer outside [0, n_layers), sm_scale not finite or <= 0,
 * bad sparse config -> FA_ERR_INVALID_ARG; other head_dim/dtype/G ->
 * FA_ERR_UNSUPPORTED.
 */
fa_status fa_attn_prefill(const void *q, const void *k, const void *v, void *o,
                          float *lse, int32_t dtype, const int32_t *cu_seqlens,
                          int32_t batch, int32_t max_seqlen, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim,
                          const uint8_t *route, const uint8_t *route_host,
                          int32_t n_layers, int32_t layer, int32_t sink_tokens,
                          int32_t window_tokens, int32_t block_tokens,
                          float sm_scale, void *stream);

/*
 * fa_attn_prefill_kv -- prefill of the last Tq_b tokens of each sequence whose
 * keys and values hold all Tk_b >= Tq_b of its tokens: chunked prefill (the
 * pages run prefill in chunks of 16384 tokens, [thelatestinai paper page,
 * Table 6]) and prefill appended to a cached prefix.  Query row i of sequence
 * b sits at absolute position Tk_b - Tq_b + i; the masks, the route and every
 * output are those of fa_attn_prefill on the whole sequence, restricted to
 * these rows.  fa_attn_prefill is the case cu_seqlens_q = cu_seqlens_k.
 *
 * q [total_q][n_q_heads][head_dim], o [total_q][n_q_heads][head_dim] out,
 * lse [total_q][n_q_heads] fp32 out (nullable), total_q = cu_seqlens_q[batch];
 * k, v [total_k][n_kv_heads][head_dim], total_k = cu_seqlens_k[batch].
 * cu_seqlens_q, cu_seqlens_k [batch + 1] int32 device.
 * max_seqlen_q: host upper bound of every Tq_b (sizes the grid).
 * Other arguments, kernels and support as fa_attn_prefill.
 * Device behaviour: a sequence with Tq_b > Tk_b reads nothing and gets NaN
 * outputs.
 * Errors: as fa_attn_prefill (cu_seqlens_k NULL -> FA_ERR_INVALID_ARG).
 */
fa_status fa_attn_prefill_kv(const void *q, const void *k, const void *v, void *o,
                             float *lse, int32_t dtype,
                             const int32_t *cu_seqlens_q,
                             const int32_t *cu_seqlens_k, int32_t batch,
                             int32_t max_seqlen_q, int32_t n_q_heads,
                             int32_t n_kv_heads, int32_t head_dim,
                             const uint8_t *route, const uint8_t *route_host,
                             int32_t n_layers, int32_t layer, int32_t sink_tokens,
                             int32_t window_tokens, int32_t block_tokens,
                             float sm_scale, void *stream);

/*
 * fa_attn_prefill_triangle -- fa_attn_prefill with Triangle Attention as the
 * sparse branch: the pages use TriangleMix's Triangle Attention (TA), a fixed,
 * training-free triangle-shaped block topology for prefill, as a sparse
 * backend of the router [thelatestinai paper page, Table 3, Table 5 and its
 * caption, Table 12].  They give no steps; the published topology is read as:
 * a query block of an SA sequence keeps its sink and window blocks exactly as
 * in fa_attn_prefill, and every query block among the last last_q_tokens /
 * block_tokens blocks of the sequence keeps every key block (the dense rows at
 * the bottom of the causal triangle).  FA-routed sequences are plain causal
 * attention.  last_q_tokens = 0 is fa_attn_prefill; a value covering the
 * sequence makes it FA.  Decode of such a layer is the FA decode: the decoded
 * token lies in the dense tail.
 *
 * Arguments, layouts, kernels and support as fa_attn_prefill; last_q_tokens
 * is a host int, a non-negative multiple of block_tokens.
 * Errors: as fa_attn_prefill; a negative last_q_tokens or one not a multiple
 * of block_tokens -> FA_ERR_INVALID_ARG.
 */
fa_status fa_attn_prefill_triangle(const void *q, const void *k, const void *v,
                                   void *o, float *lse, int32_t dtype,
                                   const int32_t *cu_seqlens, int32_t batch,
                                   int32_t max_seqlen, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim,
                                   const uint8_t *route,
                                   const uint8_t *route_host, int32_t n_layers,
                                   int32_t layer, int32_t sink_tokens,
                                   int32_t window_tokens, int32_t block_tokens,
                                   int32_t last_q_tokens, float sm_scale,
                                   void *stream);

/* ------------------------------------------------------------------------ */
/* XAttention sparse branch                                                 */
/* ------------------------------------------------------------------------ */

/*
 * The pages name XAttention ("Block Sparse Attention with Antidiagonal
 * Scoring", mlsanity page reference list) as a block-level sparse operator for
 * prefill whose blocks are chosen by a selection score [thelatestinai paper
 * page, Table 3 and Table 12]; the branch runs in three calls:
 * fa_xattn_scores -> fa_xattn_select -> fa_attn_prefill_xattn.
 *
 * fa_xattn_scores -- antidiagonal block scores.  With stride S and block B =
 * 16 S, reshaped query row a of a sequence stands for positions a*S + S-1-s and
 * reshaped key row b for positions b*S + s (s = 0..S-1; positions past the
 * sequence are zero vectors);
 *   A[a][b] = (sm_scale / S) * sum_s <q[a*S+S-1-s][h], k[b*S+s][h/G]>  (b <= a),
 *   P = softmax over b of A[a][.],
 *   scores[b][h][i][j] = sum of P over the 16 reshaped rows of query block i
 *                        and the 16 reshaped columns of key block j (j <= i).
 * q [total][n_q_heads][head_dim], k [total][n_kv_heads][head_dim], bf16 (matrix
 * cores) or fp32 (a plain VALU kernel, fp32 dot products), per dtype.
 * scores [batch][n_q_heads][n_qblocks][n_qblocks] fp32 out; entries with
 *   j > i or past a sequence's blocks are not written.
 * n_qblocks >= ceil(max_seqlen / block_tokens), <= 4096 (layout of scores).
 *   Device behaviour: the query blocks of a sequence at or past n_qblocks (a
 *   sequence longer than max_seqlen promised) are not computed; nothing is
 *   written outside the (sequence, head) rows of the layout.
 * workspace: device scratch of at least fa_xattn_workspace_size(batch,
 *   n_q_heads, n_qblocks) bytes (each reshaped row's partial sums of every
 *   key block, rescaled by a second kernel); caller-owned, contents undefined
 *   on return.
 * Supported: bf16 or fp32, head_dim 64 or 128, stride 4 or 8 with block = 16 * stride,
 * G in {1, 2, 4, 8, 16}.  Fixed reduction orders: repeated calls are bitwise
 * identical.
 * Errors: NULL pointer, batch/max_seqlen <= 0, bad heads, sm_scale not finite
 * or <= 0, block != 16 * stride, n_qblocks out of range -> FA_ERR_INVALID_ARG;
 * workspace NULL or too small -> FA_ERR_WORKSPACE; other dtype / head_dim /
 * stride / G -> FA_ERR_UNSUPPORTED.
 */
fa_status fa_xattn_scores(const void *q, const void *k, int32_t dtype,
                          const int32_t *cu_seqlens, int32_t batch,
                          int32_t max_seqlen, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_tokens, int32_t stride, float sm_scale,
                          float *scores, int32_t n_qblocks, void *workspace,
                          size_t ws_bytes, void *stream);

/* Bytes of workspace fa_xattn_scores needs: 128 bytes per (sequence, head, cell
 * j <= i) plus 128 per (sequence, head, query block), rounded up to 256; 0 for
 * non-positive sizes or n_qblocks > 4096.  About 2.2 GB for 32 heads of one
 * 131072-token sequence at block 128. */
size_t fa_xattn_workspace_size(int32_t batch, int32_t n_q_heads,
                               int32_t n_qblocks);

/*
 * fa_xattn_select -- kept blocks per (sequence, head, query block i): block 0
 * and block i always; then the blocks j < i in order of decreasing score
 * (ties: smaller j first) join while the kept sum is below
 * threshold * sum_{j<=i} scores[i][j].  The sums are fp32, the total in
 * ascending j, the kept sum in the order blocks join, so the decision is a
 * fixed function of the fp32 scores.
 * mask [batch][n_q_heads][n_qblocks][ceil(n_qblocks / 32)] uint32 out: bit j
 *   of row i set iff key block j is kept; rows past a sequence are zero (a
 *   sequence with more than n_qblocks blocks keeps only its first n_qblocks).
 * Errors: NULL pointer, batch/heads/block <= 0, n_qblocks outside [1, 4096],
 * threshold not finite or <= 0 -> FA_ERR_INVALID_ARG.
 */
fa_status fa_xattn_select(const float *scores, const int32_t *cu_seqlens,
                          int32_t batch, int32_t n_q_heads, int32_t n_qblocks,
                          int32_t block_tokens, float threshold, uint32_t *mask,
                          void *stream);

/*
 * fa_attn_prefill_xattn -- prefill attention of one layer over kept blocks:
 * query t of head h sees key s iff s <= t and key block s / block is kept for
 * query block t / block of head h in mask (the output of fa_xattn_select, or
 * any mask of that layout).  Within a kept block the rule is token-causal;
 * a block is never loaded unless some head of the workgroup keeps it.
 * q, k, v, o, lse, cu_seqlens, batch, max_seqlen, heads, head_dim as
 * fa_attn_prefill; mask [batch][n_q_heads][n_qblocks][ceil(n_qblocks / 32)]
 * uint32 device, bit j of row i = key block j kept for query block i.
 * Supported: bf16 (MFMA kernel when 256 / min(G, 4) <= block, else the plain
 * kernel) and fp32, head_dim 64 or 128, block 64 or 128.
 * Errors: NULL pointer, batch/max_seqlen <= 0, bad heads, sm_scale not finite
 * or <= 0, block not in {64, 128}, n_qblocks outside
 * [ceil(max_seqlen / block), 4096] -> FA_ERR_INVALID_ARG; other dtype /
 * head_dim -> FA_ERR_UNSUPPORTED.
 */
fa_status fa_attn_prefill_xattn(const void *q, const void *k, const void *v, void *o,
                                float *lse, int32_t dtype,
                                const int32_t *cu_seqlens, int32_t batch,
                                int32_t max_seqlen, int32_t n_q_heads,
                                int32_t n_kv_heads, int32_t head_dim,
                                int32_t block_tokens, const uint32_t *mask,
                                int32_t n_qblocks, float sm_scale, void *stream);

/* ------------------------------------------------------------------------ */
/* Decode attention                                                         */
/* ------------------------------------------------------------------------ */

/*
 * Bytes of workspace fa_attn_decode needs for a cache of max_cache tokens
 * (split-K partial outputs and log-sum-exps), rounded up to 256 B.
 */
size_t fa_decode_workspace_size(int32_t batch, int32_t n_q_heads,
                                int32_t head_dim, int32_t max_cache);

/*
 * fa_attn_decode -- one decode step of one layer: a single new query token per
 * sequence attends to its KV cache, reusing the prefill route bit
 * [thelatestinai paper page, Table 3: prefill routing, decode reuse].  The
 * query sits at absolute position n - 1, n = cache_len[b] (the cache length
 * INCLUDING the new token); SA layers read only the sink and window blocks of
 * query block (n - 1) / block.
 *
 * q [batch][n_q_heads][head_dim] (dtype); o [batch][n_q_heads][head_dim] out
 * (dtype); lse [batch][n_q_heads] fp32 out (nullable).
 * k_cache, v_cache [batch][n_kv_heads][max_cache][head_dim] (dtype).
 * k_new, v_new [batch][n_kv_heads][head_dim] (nullable, both or neither): when
 *   given, the new token's K/V are read from them and also written into the
 *   cache at position n - 1; when NULL they must already be in the cache.
 * cache_len [batch] int32 device.
 * route [batch][n_layers] uint8 device; route_host (nullable) is a host copy
 *   of the same mask: when every sequence has the same bit for `layer`, a
 *   kernel compiled for that kind runs, and for an all-SA layer the grid is
 *   sized to the sink + window span instead of max_cache.
 * workspace >= fa_decode_workspace_size(batch, n_q_heads, head_dim, max_cache).
 * The work is split over KV-token ranges; partial results are merged in a
 * fixed order, so repeated calls are bitwise identical.
 * Supported: head_dim 64 or 128, G = n_q_heads / n_kv_heads in [1, 16].
 * Device behaviour: a sequence with cache_len outside [1, max_cache] touches
 * no cache memory and gets NaN outputs.
 * Errors: as fa_attn_prefill, plus max_cache <= 0, only one of k_new/v_new
 * given -> FA_ERR_INVALID_ARG; small workspace -> FA_ERR_WORKSPACE.
 */
fa_status fa_attn_decode(const void *q, void *o, float *lse, const void *k_new,
                         const void *v_new, void *k_cache, void *v_cache,
                         int32_t max_cache, const int32_t *cache_len,
                         int32_t dtype, int32_t batch, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim,
                         const uint8_t *route, const uint8_t *route_host,
                         int32_t n_layers, int32_t layer, int32_t sink_tokens,
                         int32_t window_tokens, int32_t block_tokens,
                         float sm_scale, void *workspace, size_t ws_bytes,
                         void *stream);

/*
 * fa_attn_decode_noalloc -- fa_attn_decode for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels, results
 * (bit for bit) and device behaviour as fa_attn_decode, without workspace and
 * ws_bytes: the split partials go to a static device array of the library,
 * 64 MiB per GPU it runs on, held until the process ends.  The call allocates
 * nothing.  Its first call on a device looks up that device's copy of the array
 * (with the device current); the stream must belong to the current device.
 * Calls that overlap on one GPU share the array and race: serialise them (one
 * stream, or events).
 * Errors: as fa_attn_decode; partials larger than the array (batch x n_q_heads
 * x splits x (head_dim + 1) x 4 bytes above 64 MiB, e.g. batch 64 with 32 heads,
 * head_dim 128 and an 8192-token cache, 64 splits) -> FA_ERR_WORKSPACE; a stream of
 * another device -> FA_ERR_HIP.
 */
fa_status fa_attn_decode_noalloc(const void *q, void *o, float *lse,
                                 const void *k_new, const void *v_new,
                                 void *k_cache, void *v_cache, int32_t max_cache,
                                 const int32_t *cache_len, int32_t dtype,
                                 int32_t batch, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 const uint8_t *route, const uint8_t *route_host,
                                 int32_t n_layers, int32_t layer,
                                 int32_t sink_tokens, int32_t window_tokens,
                                 int32_t block_tokens, float sm_scale,
                                 void *stream);

/* ------------------------------------------------------------------------ */
/* Compact KV cache for SA layers                                           */
/* ------------------------------------------------------------------------ */

/*
 * An SA layer's decode only ever reads the sink tokens and the local window of
 * blocks, so its persistent KV can shrink to sink + window tokens per (sequence,
 * KV head): the "persistent KV saving" of SA layers reported by
 * [thelatestinai paper page, Tables 15 and 16].  The ring layout of
 * [batch][n_kv_heads][ring_tokens][head_dim], ring_tokens = sink + window:
 *   position p < sink                -> row p;
 *   position p in window block j     -> row sink + ((j - ns) mod nw) * block
 *                                       + p mod block  (j = p / block >= ns),
 * so a token that starts a new block takes the rows of the block that has just
 * left the window.  The attention result is identical to the full cache.
 */

/*
 * fa_kv_compact -- build the ring caches of one SA layer from its prefill K/V.
 * For every sequence b (length T_b) it copies the tokens the next decode query
 * (position T_b) keeps: positions [0, min(sink, T_b)) and the window blocks
 * max(ns, T_b/block - nw + 1) .. T_b/block below T_b.  Other ring rows are left
 * untouched (they are never read before being written).
 * k, v [total][n_kv_heads][head_dim] (dtype), cu_seqlens [batch+1] int32 device;
 * k_ring, v_ring [batch][n_kv_heads][ring_tokens][head_dim] (dtype) out.
 * Errors: NULL pointer, batch/heads <= 0, bad sparse config, ring_tokens !=
 * sink + window -> FA_ERR_INVALID_ARG; head_dim/dtype -> FA_ERR_UNSUPPORTED.
 */
fa_status fa_kv_compact(const void *k, const void *v, int32_t dtype,
                        const int32_t *cu_seqlens, int32_t batch,
                        int32_t n_kv_heads, int32_t head_dim,
                        int32_t sink_tokens, int32_t window_tokens,
                        int32_t block_tokens, void *k_ring, void *v_ring,
                        int32_t ring_tokens, void *stream);

/*
 * fa_attn_decode_ring -- fa_attn_decode for an SA layer whose caches are ring
 * caches (every sequence is SA; no route argument).  cache_len[b] is the
 * sequence length n including the new token (it may exceed ring_tokens); the
 * query sits at position n - 1 and reads the sink and window tokens of query
 * block (n - 1) / block from their ring rows.  k_new / v_new (nullable, both or
 * neither) are appended at the ring row of position n - 1.  The workspace is
 * fa_decode_workspace_size(batch, n_q_heads, head_dim, ring_tokens) bytes.
 * Device behaviour: cache_len < 1 gives NaN outputs and touches no cache row.
 * Errors: as fa_attn_decode, plus ring_tokens != sink + window ->
 * FA_ERR_INVALID_ARG.
 */
fa_status fa_attn_decode_ring(const void *q, void *o, float *lse,
                              const void *k_new, const void *v_new,
                              void *k_ring, void *v_ring, int32_t ring_tokens,
                              const int32_t *cache_len, int32_t dtype,
                              int32_t batch, int32_t n_q_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              int32_t sink_tokens, int32_t window_tokens,
                              int32_t block_tokens, float sm_scale,
                              void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUXATTN_H */
