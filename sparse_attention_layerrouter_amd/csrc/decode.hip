// decode.hip -- one decode step of one layer over the KV cache (gfx950).
//
// The new query token of every sequence sits at position n - 1 of its n-token
// cache and reuses the route bit chosen at prefill [thelatestinai paper page,
// Table 3: prefill routing, decode reuse].  FA layers read the whole cache; SA
// layers read only the sink blocks and the local window of blocks of query
// block (n - 1) / block [thelatestinai paper page, Table 6], which is a tiny,
// contiguous fraction of the cache -- the decode saving of layer-level routing
// [thelatestinai paper page, Figure 1(b)].
//
// Split-K: the kept tokens of a sequence are laid end to end (sink run, then
// window run) and cut into equal splits; workgroup (split, sequence, kv head)
// streams its split once for all G query heads of that KV head.  Inside a
// workgroup each wavefront walks 16-byte-per-lane coalesced rows (a full K or
// V row per 8/16/32 lanes), keeps an online softmax per (row slot, head), and
// the row slots and then the 4 wavefronts are merged with the log-sum-exp rule
// through LDS.  A second small kernel merges the splits in ascending order.
// Both merges use fixed orders, so results are bitwise reproducible.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

int decode_split_tokens(int max_kept_tokens)
{
    // about 64 splits per (sequence, kv head); 128..4096 tokens per split
    int st = (max_kept_tokens + 63) / 64;
    st = (st + 63) / 64 * 64;
    if (st < 128) st = 128;
    if (st > 4096) st = 4096;
    return st;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kUnroll = 4;  // rows per lane per iteration

template <typename TE>
__device__ __forceinline__ void widen(const u32x4 &w, float *out)
{
    if constexpr (sizeof(TE) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(w[i]);
            out[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
    }
}

// Physical cache position of kept-token index v (sink run then window run).
__device__ __forceinline__ int phys_of(int v, int sink_len, int win_start)
{
    return v < sink_len ? v : win_start + (v - sink_len);
}

template <typename TE, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const TE *__restrict__ q, const TE *__restrict__ k_new, const TE *__restrict__ v_new,
    TE *__restrict__ k_cache, TE *__restrict__ v_cache, int max_cache,
    const int32_t *__restrict__ cache_len, const uint8_t *__restrict__ route, int n_layers,
    int layer, int hq, int hkv, SparseRule rule, float scale_log2, int split_tokens, int n_splits,
    float *__restrict__ o_part, float *__restrict__ lse_part)
{
    constexpr int EPL = 16 / sizeof(TE);   // elements per lane (16 bytes)
    constexpr int LPR = D / EPL;           // lanes per row
    constexpr int TPI = 64 / LPR;          // rows per wavefront load
    constexpr int CHUNK = TPI * kUnroll;   // rows per wavefront iteration

    __shared__ float sm_m[kWaves][G];
    __shared__ float sm_l[kWaves][G];
    __shared__ float sm_acc[kWaves][G][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane / LPR;  // row slot
    const int c = lane % LPR;  // 16-byte chunk of the row

    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / hkv, kvh = unit % hkv;
    const int n = cache_len[b];
    if (n < 1 || n > max_cache) return;  // merge kernel writes NaN for this sequence

    const bool is_fa = MODE == kModeFA ? true
                       : MODE == kModeSA ? false
                                         : route[(size_t)b * n_layers + layer] != 0;
    int sink_len, win_start;
    if (is_fa) {
        sink_len = n;
        win_start = n;
    } else {
        const int i_q = (n - 1) >> rule.bk_log2;
        sink_len = min(rule.ns << rule.bk_log2, n);
        win_start = max(rule.ns << rule.bk_log2, (i_q - rule.nw + 1) << rule.bk_log2);
        win_start = min(win_start, n);
    }
    const int kept = sink_len + (n - win_start);
    const int v0 = split * split_tokens;
    const int v1 = min(v0 + split_tokens, kept);

    // q of the G heads, this lane's 16-byte chunk, pre-scaled into the exp2 domain
    float qv[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const TE *qr = q + ((size_t)b * hq + kvh * G + h) * D + c * EPL;
        float tmp[EPL];
        widen<TE>(*(const u32x4 *)qr, tmp);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[h][e] = tmp[e] * scale_log2;
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }

    const size_t cache_base = ((size_t)b * hkv + kvh) * (size_t)max_cache * D;
    const TE *kc = k_cache + cache_base;
    const TE *vc = v_cache + cache_base;
    const TE *kn = k_new ? k_new + ((size_t)b * hkv + kvh) * D : nullptr;
    const TE *vn = v_new ? v_new + ((size_t)b * hkv + kvh) * D : nullptr;

    for (int cv = v0 + wave * CHUNK; cv < v1; cv += kWaves * CHUNK) {
        u32x4 kw[kUnroll], vw[kUnroll];
        int pos[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int vi = cv + u * TPI + r;
            ok[u] = vi < v1;
            pos[u] = ok[u] ? phys_of(vi, sink_len, win_start) : 0;
            const bool fresh = ok[u] && kn && pos[u] == n - 1;
            const TE *kp = fresh ? kn + c * EPL : kc + (size_t)pos[u] * D + c * EPL;
            const TE *vp = fresh ? vn + c * EPL : vc + (size_t)pos[u] * D + c * EPL;
            kw[u] = ok[u] ? *(const u32x4 *)kp : u32x4{0, 0, 0, 0};
            vw[u] = ok[u] ? *(const u32x4 *)vp : u32x4{0, 0, 0, 0};
            if (fresh) {  // append the new token to the cache
                *(u32x4 *)(k_cache + cache_base + (size_t)pos[u] * D + c * EPL) = kw[u];
                *(u32x4 *)(v_cache + cache_base + (size_t)pos[u] * D + c * EPL) = vw[u];
            }
        }
        // scores (log2 domain), reduced over the LPR lanes of each row
        float s[kUnroll][G];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float kf[EPL];
            widen<TE>(kw[u], kf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float part = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) part += qv[h][e] * kf[e];
                part = group_sum<LPR>(part);
                s[u][h] = ok[u] ? part : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, s[u][h]);
            const float m_new = fmaxf(m[h], mx);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = fast_exp2(m[h] - m_use);
            float p[kUnroll];
            float ps = 0.0f;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                p[u] = fast_exp2(s[u][h] - m_use);
                ps += p[u];
            }
            l[h] = l[h] * alpha + ps;
            m[h] = m_new;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float vf[EPL];
                widen<TE>(vw[u], vf);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] += p[u] * vf[e];
            }
        }
    }

    // merge the TPI row slots of the wavefront (lanes c, c+LPR, ...) into slot 0
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mo = __shfl_xor(m[h], off);
            float lo = __shfl_xor(l[h], off);
            const float M = fmaxf(m[h], mo);
            const float Mu = M == -INFINITY ? 0.0f : M;
            const float fa_ = fast_exp2(m[h] - Mu), fb = fast_exp2(mo - Mu);
            l[h] = l[h] * fa_ + lo * fb;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float ao = __shfl_xor(acc[h][e], off);
                acc[h][e] = acc[h][e] * fa_ + ao * fb;
            }
            m[h] = M;
        }
    }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][h][c * EPL + e] = acc[h][e];
            if (c == 0) {
                sm_m[wave][h] = m[h];
                sm_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    // merge the 4 wavefronts in order; write this split's partial (o, lse)
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
        const float Mu = M == -INFINITY ? 0.0f : M;
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(sm_m[w][h] - Mu);
            L += sm_l[w][h] * f;
            O += sm_acc[w][h][d] * f;
        }
        const size_t row = ((size_t)b * hq + kvh * G + h) * n_splits + split;
        o_part[row * D + d] = L > 0.0f ? O / L : 0.0f;
        if (d == 0) lse_part[row] = L > 0.0f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
}

// o[b][h] = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, ascending s.
template <typename TE>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    const int32_t *__restrict__ cache_len, int max_cache, int hq, int D, int n_splits,
    TE *__restrict__ o, float *__restrict__ lse)
{
    const int bh = blockIdx.x;
    const int b = bh / hq;
    const int n = cache_len[b];
    const bool bad = n < 1 || n > max_cache;
    const float *lp = lse_part + (size_t)bh * n_splits;
    float M = -INFINITY;
    if (!bad)
        for (int s = 0; s < n_splits; ++s) M = fmaxf(M, lp[s]);
    float W = 0.0f;
    if (!bad)
        for (int s = 0; s < n_splits; ++s) W += lp[s] == -INFINITY ? 0.0f : __expf(lp[s] - M);
    const float inv = 1.0f / W;
    for (int d = threadIdx.x; d < D; d += 64) {
        float acc = 0.0f;
        if (!bad)
            for (int s = 0; s < n_splits; ++s) {
                if (lp[s] == -INFINITY) continue;
                acc += __expf(lp[s] - M) * o_part[((size_t)bh * n_splits + s) * D + d];
            }
        const float val = bad ? __builtin_nanf("") : acc * inv;
        if constexpr (sizeof(TE) == 2)
            ((uint16_t *)o)[(size_t)bh * D + d] = to_bf16(val);
        else
            ((float *)o)[(size_t)bh * D + d] = val;
    }
    if (lse && threadIdx.x == 0) lse[bh] = bad ? __builtin_nanf("") : M + __logf(W);
}

template <typename TE, int D, int G>
hipError_t launch_split(const DecodeArgs &a, hipStream_t stream, const SparseRule &r,
                        float scale_log2)
{
    dim3 grid(a.n_splits, a.batch * a.hkv);
#define FA_DECODE_ARGS                                                                         \
    (const TE *)a.q, (const TE *)a.k_new, (const TE *)a.v_new, (TE *)a.k_cache,                 \
        (TE *)a.v_cache, a.max_cache, a.cache_len, a.route, a.n_layers, a.layer, a.hq, a.hkv, r, \
        scale_log2, a.split_tokens, a.n_splits, a.o_part, a.lse_part
    if (a.mode == kModeFA)
        decode_split_kernel<TE, D, G, kModeFA><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
    else if (a.mode == kModeSA)
        decode_split_kernel<TE, D, G, kModeSA><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
    else
        decode_split_kernel<TE, D, G, kModeMixed><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
#undef FA_DECODE_ARGS
    return hipGetLastError();
}

template <typename TE, int D>
hipError_t launch_by_g(const DecodeArgs &a, hipStream_t stream, const SparseRule &r,
                       float scale_log2)
{
    switch (a.hq / a.hkv) {
    case 1: return launch_split<TE, D, 1>(a, stream, r, scale_log2);
    case 2: return launch_split<TE, D, 2>(a, stream, r, scale_log2);
    case 4: return launch_split<TE, D, 4>(a, stream, r, scale_log2);
    case 8: return launch_split<TE, D, 8>(a, stream, r, scale_log2);
    case 16: return launch_split<TE, D, 16>(a, stream, r, scale_log2);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_g_supported(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    SparseRule r{a.ns, a.nw, a.bk_log2};
    const float scale_log2 = a.sm_scale * kLog2e;
    hipError_t e;
    if (a.bf16)
        e = a.d == 128 ? launch_by_g<uint16_t, 128>(a, stream, r, scale_log2)
                       : launch_by_g<uint16_t, 64>(a, stream, r, scale_log2);
    else
        e = a.d == 128 ? launch_by_g<float, 128>(a, stream, r, scale_log2)
                       : launch_by_g<float, 64>(a, stream, r, scale_log2);
    if (e != hipSuccess) return e;
    if (a.bf16)
        decode_merge_kernel<uint16_t><<<a.batch * a.hq, 64, 0, stream>>>(
            a.o_part, a.lse_part, a.cache_len, a.max_cache, a.hq, a.d, a.n_splits, (uint16_t *)a.o,
            a.lse);
    else
        decode_merge_kernel<float><<<a.batch * a.hq, 64, 0, stream>>>(
            a.o_part, a.lse_part, a.cache_len, a.max_cache, a.hq, a.d, a.n_splits, (float *)a.o,
            a.lse);
    return hipGetLastError();
}

}  // namespace fa
