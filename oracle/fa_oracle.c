/*
 * fa_oracle.c -- CPU oracle for Flux Attention's layer-routed hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source, header, table or helper with the
 * HIP library; the two meet only through the caller's input buffers.
 *
 * What it computes (sources are the pages about "Flux Attention:
 * Context-Aware Hybrid Attention for Efficient LLMs Inference"):
 *   - the Layer Router: the query hidden states x_Q are pooled and mapped to
 *     one FA/SA decision per layer [HF model card, summary paragraph;
 *     thelatestinai paper page, Figure 2]; the decision is taken once at
 *     prefill and reused in decode [thelatestinai paper page, Table 3].
 *     The pooling window is "the last pool_tokens rows" (the sequence-suffix
 *     budget of [thelatestinai paper page, Figure 8]).
 *   - FA layers: GQA causal softmax attention (FlashAttention-2 is the dense
 *     path in [thelatestinai paper page, Table 6]; query heads share KV heads
 *     as named by `repeat_kv` in the codewithpapers function list).
 *   - SA layers: streaming block-sparse attention that keeps the attention
 *     sink blocks plus a local window of blocks (block size / sink size of
 *     [thelatestinai paper page, Table 6]; "streaming info" block-sparse
 *     kernel named by `generate_streaming_info_blocksparse_flash_attn` in the
 *     codewithpapers function list).  SA is *defined* by its token mask, so
 *     the oracle evaluates the mask predicate token by token.
 *
 * Precision: inputs are read as fp32 or bf16 (bf16 widened exactly), every
 * attention sum is accumulated in double and the softmax is the exact
 * two-pass form (max, then sum).  The router keeps two paths: the route bit is
 * decided in fp32 (the precision the GPU kernel decides it in), and an fp64
 * copy of the logits is returned so callers can report the decision margin.
 *
 * Readings where the pages are silent:
 *   router activation ReLU, strict threshold logit > 0 -> FA (NaN -> SA),
 *   bit 1 = FA; sink and window are counted in tokens and must be multiples of
 *   the block; the window counts whole blocks including the query's own block;
 *   inside kept blocks the token-level causal rule s <= t applies; decode puts
 *   the query at absolute position n-1 of an n-token cache.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_EINVAL 1

/* Read element i of a fp32 or bf16 array, widened exactly to double. */
static double orc_load(const void *base, int dtype, size_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static float orc_load_f32(const void *base, int dtype, size_t i)
{
    return (float)orc_load(base, dtype, i);
}

/* ------------------------------------------------------------------------ */
/* Router                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Pool: p[b][j] = (1/P) * sum_{t = T_b - P}^{T_b - 1} x_Q[t][j], P = min(pool, T_b).
 * The fp32 copy sums in ascending t and divides once at the end; the fp64 copy
 * does the same in double.
 */
int orc_pool(const void *x, int dtype, const int32_t *cu_seqlens, int batch,
             int hidden, int pool_tokens, float *p32, double *p64)
{
    if (!x || !cu_seqlens || batch <= 0 || hidden <= 0 || pool_tokens <= 0)
        return ORC_EINVAL;
    for (int b = 0; b < batch; ++b) {
        int start = cu_seqlens[b], T = cu_seqlens[b + 1] - cu_seqlens[b];
        if (T <= 0)
            return ORC_EINVAL;
        int P = pool_tokens < T ? pool_tokens : T;
        for (int j = 0; j < hidden; ++j) {
            float s32 = 0.0f;
            double s64 = 0.0;
            for (int t = T - P; t < T; ++t) {
                size_t idx = (size_t)(start + t) * hidden + j;
                s32 += orc_load_f32(x, dtype, idx);
                s64 += orc_load(x, dtype, idx);
            }
            if (p32)
                p32[(size_t)b * hidden + j] = s32 / (float)P;
            if (p64)
                p64[(size_t)b * hidden + j] = s64 / (double)P;
        }
    }
    return ORC_OK;
}

/*
 * Router MLP and threshold:
 *   h = ReLU(W1 p + b1)           W1 [router_hidden][hidden]
 *   logit = W2 h + b2             W2 [n_layers][router_hidden]
 *   route[b][l] = (logit > 0) ? 1 (FA) : 0 (SA)
 * Every dot product is summed in ascending index.  route and logits32 come
 * from the fp32 path; logits64 (optional) from the fp64 path.
 */
int orc_router(const void *x, int dtype, const int32_t *cu_seqlens, int batch,
               int hidden, int pool_tokens, const float *w1, const float *b1,
               int router_hidden, const float *w2, const float *b2,
               int n_layers, uint8_t *route, float *logits32,
               double *logits64)
{
    if (!w1 || !b1 || !w2 || !b2 || !route || router_hidden <= 0 ||
        n_layers <= 0)
        return ORC_EINVAL;
    float *p32 = malloc(sizeof(float) * (size_t)batch * hidden);
    double *p64 = malloc(sizeof(double) * (size_t)batch * hidden);
    float *h32 = malloc(sizeof(float) * (size_t)router_hidden);
    double *h64 = malloc(sizeof(double) * (size_t)router_hidden);
    int rc = ORC_EINVAL;
    if (!p32 || !p64 || !h32 || !h64)
        goto out;
    rc = orc_pool(x, dtype, cu_seqlens, batch, hidden, pool_tokens, p32, p64);
    if (rc != ORC_OK)
        goto out;
    for (int b = 0; b < batch; ++b) {
        const float *pb32 = p32 + (size_t)b * hidden;
        const double *pb64 = p64 + (size_t)b * hidden;
        for (int i = 0; i < router_hidden; ++i) {
            float a32 = 0.0f;
            double a64 = 0.0;
            for (int j = 0; j < hidden; ++j) {
                a32 += w1[(size_t)i * hidden + j] * pb32[j];
                a64 += (double)w1[(size_t)i * hidden + j] * pb64[j];
            }
            a32 += b1[i];
            a64 += (double)b1[i];
            h32[i] = a32 > 0.0f ? a32 : 0.0f;
            h64[i] = a64 > 0.0 ? a64 : 0.0;
        }
        for (int l = 0; l < n_layers; ++l) {
            float z32 = 0.0f;
            double z64 = 0.0;
            for (int i = 0; i < router_hidden; ++i) {
                z32 += w2[(size_t)l * router_hidden + i] * h32[i];
                z64 += (double)w2[(size_t)l * router_hidden + i] * h64[i];
            }
            z32 += b2[l];
            z64 += (double)b2[l];
            route[(size_t)b * n_layers + l] = (z32 > 0.0f) ? 1 : 0;
            if (logits32)
                logits32[(size_t)b * n_layers + l] = z32;
            if (logits64)
                logits64[(size_t)b * n_layers + l] = z64;
        }
    }
    rc = ORC_OK;
out:
    free(p32);
    free(p64);
    free(h32);
    free(h64);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Sparsity rule                                                            */
/* ------------------------------------------------------------------------ */

static int orc_cfg_ok(int sink, int window, int block)
{
    return block > 0 && sink >= 0 && window >= block && sink % block == 0 &&
           window % block == 0;
}

/*
 * Token mask of one layer.  Query at absolute position t may attend to key
 * position s iff s <= t and
 *   FA: always;
 *   SA: the key block j = s / Bk is a sink block (j < sink / Bk) or lies in
 *       the local window of the query block i = t / Bk, i.e. j > i - window/Bk.
 */
static int orc_visible(int t, int s, int is_fa, int sink, int window,
                       int block)
{
    if (s > t)
        return 0;
    if (is_fa)
        return 1;
    int i = t / block, j = s / block;
    int ns = sink / block, nw = window / block;
    return (j < ns) || (j > i - nw);
}

int orc_visible_predicate(int t, int s, int is_fa, int sink, int window,
                          int block)
{
    return orc_visible(t, s, is_fa, sink, window, block);
}

/* Number of visible (query, key) pairs of one sequence of length T. */
int64_t orc_visible_pairs(int T, int is_fa, int sink, int window, int block)
{
    int64_t n = 0;
    for (int t = 0; t < T; ++t)
        for (int s = 0; s <= t; ++s)
            n += orc_visible(t, s, is_fa, sink, window, block);
    return n;
}

/*
 * Block plan.  For query block i of sequence b, the kept key blocks are
 *   FA: {0, ..., i}
 *   SA: {j <= i : j < ns  or  j >= i - nw + 1}
 * written ascending as two half-open ranges
 *   plan[b][i] = (0, sink_end, win_begin, i + 1)
 *   FA: sink_end = win_begin = i + 1 (one range [0, i+1), second empty)
 *   SA: sink_end = min(ns, i + 1), win_begin = max(sink_end, i - nw + 1).
 * Query blocks past the sequence end get (0, 0, 0, 0).
 */
int orc_block_plan(const int32_t *seqlens, int batch, int max_qblocks,
                   const uint8_t *route, int n_layers, int layer, int sink,
                   int window, int block, int32_t *plan)
{
    if (!seqlens || !route || !plan || batch <= 0 || max_qblocks <= 0 ||
        layer < 0 || layer >= n_layers || !orc_cfg_ok(sink, window, block))
        return ORC_EINVAL;
    int ns = sink / block, nw = window / block;
    for (int b = 0; b < batch; ++b) {
        int T = seqlens[b];
        int nqb = (T + block - 1) / block;
        int is_fa = route[(size_t)b * n_layers + layer] != 0;
        for (int i = 0; i < max_qblocks; ++i) {
            int32_t *e = plan + ((size_t)b * max_qblocks + i) * 4;
            if (i >= nqb) {
                e[0] = e[1] = e[2] = e[3] = 0;
                continue;
            }
            int sink_end, win_begin;
            if (is_fa) {
                sink_end = i + 1;
                win_begin = i + 1;
            } else {
                sink_end = ns < i + 1 ? ns : i + 1;
                win_begin = i - nw + 1;
                if (win_begin < sink_end)
                    win_begin = sink_end;
            }
            e[0] = 0;
            e[1] = sink_end;
            e[2] = win_begin;
            e[3] = i + 1;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                */
/* ------------------------------------------------------------------------ */

/*
 * One output row: query vector qv (d values, already widened), keys and
 * values of one KV head given by (base pointer, element offset of position 0,
 * stride between positions).  Visible keys come from orc_visible.  Exact
 * two-pass softmax in double:
 *   S_s = sm_scale * <q, k_s>,  m = max S,  l = sum exp(S - m),
 *   o = sum exp(S - m) v_s / l,  lse = m + ln l.
 * A row with no visible key cannot occur (s = t is always visible).
 */
static void orc_row(const double *qv, const void *k, const void *v,
                    int dtype, size_t kv_off, size_t kv_stride, int t,
                    int n_keys, int is_fa, int sink, int window, int block,
                    int d, double sm_scale, double *scores, double *o_out,
                    double *lse_out)
{
    double m = -INFINITY;
    for (int s = 0; s < n_keys; ++s) {
        if (!orc_visible(t, s, is_fa, sink, window, block)) {
            scores[s] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        size_t base = kv_off + (size_t)s * kv_stride;
        for (int c = 0; c < d; ++c)
            dot += qv[c] * orc_load(k, dtype, base + c);
        scores[s] = sm_scale * dot;
        if (scores[s] > m)
            m = scores[s];
    }
    double l = 0.0;
    for (int s = 0; s < n_keys; ++s)
        if (scores[s] != -INFINITY)
            l += exp(scores[s] - m);
    for (int c = 0; c < d; ++c)
        o_out[c] = 0.0;
    for (int s = 0; s < n_keys; ++s) {
        if (scores[s] == -INFINITY)
            continue;
        double w = exp(scores[s] - m) / l;
        size_t base = kv_off + (size_t)s * kv_stride;
        for (int c = 0; c < d; ++c)
            o_out[c] += w * orc_load(v, dtype, base + c);
    }
    if (lse_out)
        *lse_out = m + log(l);
}

typedef struct {
    /* shared, read-only */
    const void *q, *k, *v;
    int dtype;
    const int32_t *cu_seqlens;
    int batch, hq, hkv, d, n_layers, layer, sink, window, block;
    const uint8_t *route;
    double sm_scale;
    const int32_t *rows;
    int n_rows;
    double *o, *lse;
    int max_len;
    /* per thread */
    int tid, n_threads;
} orc_prefill_job;

static int orc_seq_of(const int32_t *cu, int batch, int token)
{
    for (int b = 0; b < batch; ++b)
        if (token >= cu[b] && token < cu[b + 1])
            return b;
    return -1;
}

static void *orc_prefill_worker(void *arg)
{
    orc_prefill_job *j = arg;
    int G = j->hq / j->hkv;
    double *qv = malloc(sizeof(double) * (size_t)j->d);
    double *scores = malloc(sizeof(double) * (size_t)(j->max_len > 0 ? j->max_len : 1));
    if (!qv || !scores) {
        free(qv);
        free(scores);
        return (void *)1;
    }
    size_t n_units = (size_t)j->n_rows * j->hq;
    for (size_t u = (size_t)j->tid; u < n_units; u += (size_t)j->n_threads) {
        int r = (int)(u / j->hq), h = (int)(u % j->hq);
        int token = j->rows ? j->rows[r] : r;
        int b = orc_seq_of(j->cu_seqlens, j->batch, token);
        int start = j->cu_seqlens[b];
        int T = j->cu_seqlens[b + 1] - start;
        int t = token - start;
        int g = h / G;
        int is_fa = j->route[(size_t)b * j->n_layers + j->layer] != 0;
        for (int c = 0; c < j->d; ++c)
            qv[c] = orc_load(j->q, j->dtype,
                             ((size_t)token * j->hq + h) * j->d + c);
        orc_row(qv, j->k, j->v, j->dtype,
                ((size_t)start * j->hkv + g) * j->d, (size_t)j->hkv * j->d,
                t, T, is_fa, j->sink, j->window, j->block, j->d, j->sm_scale,
                scores, j->o + ((size_t)r * j->hq + h) * j->d,
                j->lse ? j->lse + (size_t)r * j->hq + h : NULL);
    }
    free(qv);
    free(scores);
    return NULL;
}

static int orc_run_threads(void *(*fn)(void *), void *jobs, size_t job_size,
                           int n_threads)
{
    pthread_t *th = malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!th)
        return ORC_EINVAL;
    int rc = ORC_OK;
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, fn, (char *)jobs + job_size * i) != 0) {
            rc = ORC_EINVAL;
            break;
        }
        started++;
    }
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(th[i], &ret);
        if (ret)
            rc = ORC_EINVAL;
    }
    free(th);
    return rc;
}

/*
 * Prefill attention of one layer over a packed varlen batch.
 *   q [total][hq][d], k, v [total][hkv][d] (fp32 or bf16), positions restart
 *   at 0 in every sequence (cu_seqlens[b] .. cu_seqlens[b+1]).
 *   rows: packed token indices to compute (NULL = all tokens, n_rows = total).
 *   o [n_rows][hq][d] and lse [n_rows][hq] (nullable) in double.
 * Query head h reads KV head h / (hq / hkv).
 */
int orc_attn_prefill(const void *q, const void *k, const void *v, int dtype,
                     const int32_t *cu_seqlens, int batch, int hq, int hkv,
                     int d, const uint8_t *route, int n_layers, int layer,
                     int sink, int window, int block, double sm_scale,
                     const int32_t *rows, int n_rows, double *o, double *lse,
                     int n_threads)
{
    if (!q || !k || !v || !cu_seqlens || !route || !o || batch <= 0 ||
        hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || layer < 0 ||
        layer >= n_layers || !orc_cfg_ok(sink, window, block) ||
        (dtype != ORC_F32 && dtype != ORC_BF16))
        return ORC_EINVAL;
    int total = cu_seqlens[batch];
    int max_len = 0;
    for (int b = 0; b < batch; ++b) {
        int T = cu_seqlens[b + 1] - cu_seqlens[b];
        if (T <= 0)
            return ORC_EINVAL;
        if (T > max_len)
            max_len = T;
    }
    if (!rows)
        n_rows = total;
    for (int r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total)
            return ORC_EINVAL;
    if (n_threads < 1)
        n_threads = 1;
    orc_prefill_job *jobs = calloc((size_t)n_threads, sizeof *jobs);
    if (!jobs)
        return ORC_EINVAL;
    for (int i = 0; i < n_threads; ++i) {
        orc_prefill_job *j = &jobs[i];
        j->q = q; j->k = k; j->v = v; j->dtype = dtype;
        j->cu_seqlens = cu_seqlens; j->batch = batch;
        j->hq = hq; j->hkv = hkv; j->d = d;
        j->n_layers = n_layers; j->layer = layer;
        j->sink = sink; j->window = window; j->block = block;
        j->route = route; j->sm_scale = sm_scale;
        j->rows = rows; j->n_rows = n_rows; j->o = o; j->lse = lse;
        j->max_len = max_len; j->tid = i; j->n_threads = n_threads;
    }
    int rc = orc_run_threads(orc_prefill_worker, jobs, sizeof *jobs, n_threads);
    free(jobs);
    return rc;
}

typedef struct {
    const void *q, *kc, *vc;
    int dtype, max_cache;
    const int32_t *cache_len;
    int batch, hq, hkv, d, n_layers, layer, sink, window, block;
    const uint8_t *route;
    double sm_scale;
    const int32_t *heads;
    int n_heads;
    double *o, *lse;
    int tid, n_threads;
} orc_decode_job;

static void *orc_decode_worker(void *arg)
{
    orc_decode_job *j = arg;
    int G = j->hq / j->hkv;
    double *qv = malloc(sizeof(double) * (size_t)j->d);
    double *scores = malloc(sizeof(double) * (size_t)j->max_cache);
    if (!qv || !scores) {
        free(qv);
        free(scores);
        return (void *)1;
    }
    int nh = j->heads ? j->n_heads : j->hq;
    size_t n_units = (size_t)j->batch * nh;
    for (size_t u = (size_t)j->tid; u < n_units; u += (size_t)j->n_threads) {
        int b = (int)(u / nh);
        int hi = (int)(u % nh);
        int h = j->heads ? j->heads[hi] : hi;
        int g = h / G;
        int n = j->cache_len[b];
        int is_fa = j->route[(size_t)b * j->n_layers + j->layer] != 0;
        for (int c = 0; c < j->d; ++c)
            qv[c] = orc_load(j->q, j->dtype, ((size_t)b * j->hq + h) * j->d + c);
        /* cache layout [b][g][pos][d]; the query sits at position n - 1 */
        orc_row(qv, j->kc, j->vc, j->dtype,
                (((size_t)b * j->hkv + g) * j->max_cache) * j->d, (size_t)j->d,
                n - 1, n, is_fa, j->sink, j->window, j->block, j->d,
                j->sm_scale, scores,
                j->o + ((size_t)b * j->hq + h) * j->d,
                j->lse ? j->lse + (size_t)b * j->hq + h : NULL);
    }
    free(qv);
    free(scores);
    return NULL;
}

/*
 * Decode attention of one layer, one new token per sequence, which is already
 * stored in the cache at position cache_len[b] - 1.
 *   q [batch][hq][d], k_cache, v_cache [batch][hkv][max_cache][d].
 *   heads: optional list of query heads to compute (NULL = all); outputs are
 *   o [batch][hq][d], lse [batch][hq] in double (rows of skipped heads are
 *   left untouched).
 */
int orc_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                    int max_cache, const int32_t *cache_len, int dtype,
                    int batch, int hq, int hkv, int d, const uint8_t *route,
                    int n_layers, int layer, int sink, int window, int block,
                    double sm_scale, const int32_t *heads, int n_heads,
                    double *o, double *lse, int n_threads)
{
    if (!q || !k_cache || !v_cache || !cache_len || !route || !o ||
        batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 ||
        max_cache <= 0 || layer < 0 || layer >= n_layers ||
        !orc_cfg_ok(sink, window, block) ||
        (dtype != ORC_F32 && dtype != ORC_BF16))
        return ORC_EINVAL;
    for (int b = 0; b < batch; ++b)
        if (cache_len[b] <= 0 || cache_len[b] > max_cache)
            return ORC_EINVAL;
    for (int i = 0; heads && i < n_heads; ++i)
        if (heads[i] < 0 || heads[i] >= hq)
            return ORC_EINVAL;
    if (n_threads < 1)
        n_threads = 1;
    orc_decode_job *jobs = calloc((size_t)n_threads, sizeof *jobs);
    if (!jobs)
        return ORC_EINVAL;
    for (int i = 0; i < n_threads; ++i) {
        orc_decode_job *j = &jobs[i];
        j->q = q; j->kc = k_cache; j->vc = v_cache; j->dtype = dtype;
        j->max_cache = max_cache; j->cache_len = cache_len;
        j->batch = batch; j->hq = hq; j->hkv = hkv; j->d = d;
        j->n_layers = n_layers; j->layer = layer;
        j->sink = sink; j->window = window; j->block = block;
        j->route = route; j->sm_scale = sm_scale;
        j->heads = heads; j->n_heads = n_heads;
        j->o = o; j->lse = lse; j->tid = i; j->n_threads = n_threads;
    }
    int rc = orc_run_threads(orc_decode_worker, jobs, sizeof *jobs, n_threads);
    free(jobs);
    return rc;
}
