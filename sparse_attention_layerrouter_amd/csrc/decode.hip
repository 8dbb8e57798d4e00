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
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
// The cache is streamed once per step and never re-read by it: its loads carry
// the non-temporal hint (measured ~11 % faster streaming on MI355X), which is
// the cache-policy bit 2 of the LDS-direct copy.
constexpr int kNonTemporal = 2;
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

// Row of position pos in a compact SA ring cache of sink + window tokens: the
// sink tokens keep their positions; window block j (j >= ns) lives in ring
// block (j - ns) mod nw, so the newest block overwrites the one that just left
// the window.
__device__ __forceinline__ int ring_slot(int pos, const SparseRule &r)
{
    const int sink_tok = r.ns << r.bk_log2;
    if (pos < sink_tok) return pos;
    const int j = pos >> r.bk_log2;
    return sink_tok + (((j - r.ns) % r.nw) << r.bk_log2) + (pos & ((1 << r.bk_log2) - 1));
}

// Row of position pos in the cache: the position itself, or its ring slot.
template <bool RING>
__device__ __forceinline__ int cache_row(int pos, const SparseRule &r)
{
    if constexpr (RING) return ring_slot(pos, r);
    else return pos;
}

template <typename TE, int D, int G, int MODE, bool RING>
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
    if (n < 1 || (!RING && n > max_cache)) return;  // merge kernel writes NaN for this sequence

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
            const size_t row = (size_t)cache_row<RING>(pos[u], rule);
            const TE *kp = fresh ? kn + c * EPL : kc + row * D + c * EPL;
            const TE *vp = fresh ? vn + c * EPL : vc + row * D + c * EPL;
            kw[u] = ok[u] ? __builtin_nontemporal_load((const u32x4 *)kp) : u32x4{0, 0, 0, 0};
            vw[u] = ok[u] ? __builtin_nontemporal_load((const u32x4 *)vp) : u32x4{0, 0, 0, 0};
            if (fresh) {  // append the new token to the cache
                *(u32x4 *)(k_cache + cache_base + row * D + c * EPL) = kw[u];
                *(u32x4 *)(v_cache + cache_base + row * D + c * EPL) = vw[u];
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

// ---------------------------------------------------------------------------
// bf16 decode on the matrix cores.
//
// Per wavefront and 32-token chunk of its split:
//   S^T = K Q^T   on v_mfma_f32_16x16x32_bf16: A = K (lane l: token l%16 of a
//                 16-token half, 8 consecutive d), loaded straight from the
//                 cache into registers (each instruction reads 64 contiguous
//                 bytes of 16 rows); B = Q^T (lane l: head l%16, zero for
//                 l%16 >= G), loaded once.  C lane l: head l%16, tokens
//                 4*(l/16) + j of the half.
//   softmax       per head over the lane's 8 tokens, lazy reference max.
//   O^T += V^T P^T on the same MFMA: P^T is the lane's own C values (head l%16,
//                 tokens 4*(l/16)+j of both halves -> k index 8*(l/16) + e);
//                 V rows go global -> LDS (global_load_lds_dwordx4, swizzled)
//                 and V^T comes back through ds_read_b64_tr_b16.
// The chunk loop is software pipelined: the K registers and V LDS buffer of
// chunk i+1 are requested before chunk i is computed.  The 4 wavefronts of the
// workgroup take interleaved chunks and are merged with the log-sum-exp rule.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

constexpr int kDecChunk = 32;              // tokens per wavefront iteration
constexpr float kDecRescaleSlack = 8.0f;   // log2 units

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// V tile swizzle: 16-byte chunk c of row r is stored at chunk c ^ (2 * (r % 8)),
// so the 8 rows x 32 bytes a 32-lane transposed read touches hit disjoint banks.
template <int D>
__device__ __forceinline__ int dec_swz(int r) { return (2 * (r & 7)) & (D / 8 - 1); }

template <int D>
struct DecChunkRegs {
    u32x4 k[2][D / 32];   // [half][d step] K operand
};

// ONE: every wave takes at most one chunk (splits of kWaves * kDecChunk tokens,
// e.g. every split of an SA layer's sink + window span): no second register set
// or V buffer, so four workgroups fit per CU and a short layer's splits run in
// about one round.  The per-chunk arithmetic and the merges are the same.
template <int D, int G, int MODE, bool RING, bool ONE>
__global__ __launch_bounds__(kThreads, ONE ? 5 : 2) void decode_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, uint16_t *__restrict__ k_cache,
    uint16_t *__restrict__ v_cache, int max_cache, const int32_t *__restrict__ cache_len,
    const uint8_t *__restrict__ route, int n_layers, int layer, int hq, int hkv, SparseRule rule,
    float scale_log2, int split_tokens, int n_splits, float *__restrict__ o_part,
    float *__restrict__ lse_part)
{
    constexpr int CH = D / 8;                 // 16-byte chunks per row
    constexpr int RPI = 64 / CH;              // V rows per global_load_lds (1 KiB)
    constexpr int VINS = kDecChunk / RPI;     // V copies per chunk per wave
    constexpr int VBYTES = kDecChunk * D * 2; // one wave's V buffer
    constexpr int NKS = D / 32;               // d steps of the QK product
    static_assert(G >= 1 && G <= 16, "GQA ratio");
    // V buffers: [wave] x 2, two separate arrays so that reads of the current
    // chunk provably do not alias the copies into the next one
    // ONE with G <= 8 keeps its whole LDS within the 32 KiB V buffer (the merge
    // scratch then lives in it too), so five workgroups fit per CU
    constexpr bool kPack = ONE && G <= 8;
    constexpr int HS = kPack ? G : 16;  // head slots of the merge scratch
    static_assert(kWaves * HS * D * 4 + (kPack ? 2 * kWaves * 16 * 4 : 0) <= kWaves * VBYTES,
                  "merge scratch fits the V buffers");
    __shared__ __attribute__((aligned(1024))) char vbuf0[kWaves][VBYTES];
    // (the unused arrays of a variant are never referenced and take no LDS)
    __shared__ __attribute__((aligned(1024))) char vbuf1[ONE ? 1 : kWaves][ONE ? 16 : VBYTES];
    __shared__ float sm_m_s[kPack ? 1 : kWaves * 16];
    __shared__ float sm_l_s[kPack ? 1 : kWaves * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;   // head (C/B operands) or token (A operand)
    const int g4 = lane >> 4;    // 16-lane group

    const int split = blockIdx.x;
    const int unit = blockIdx.y;
    const int b = unit / hkv, kvh = unit % hkv;
    const int n = cache_len[b];
    if (n < 1 || (!RING && n > max_cache)) return;  // the merge kernel writes NaN for it

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

    const size_t cache_base = ((size_t)b * hkv + kvh) * (size_t)max_cache * D;
    const uint16_t *kc = k_cache + cache_base;
    const uint16_t *vc = v_cache + cache_base;
    const uint16_t *kn = k_new ? k_new + ((size_t)b * hkv + kvh) * D : nullptr;
    const uint16_t *vn = v_new ? v_new + ((size_t)b * hkv + kvh) * D : nullptr;
    // the workgroup whose split holds the new token appends it to the cache;
    // every read of that position below goes to k_new / v_new instead
    if (kn && v0 <= kept - 1 && kept - 1 < v1 && tid < CH) {
        const size_t row = (size_t)cache_row<RING>(n - 1, rule);
        *(u32x4 *)(k_cache + cache_base + row * D + tid * 8) = *(const u32x4 *)(kn + tid * 8);
        *(u32x4 *)(v_cache + cache_base + row * D + tid * 8) = *(const u32x4 *)(vn + tid * 8);
    }

    // physical row address of kept-token index v (clamped into the split)
    auto row_ptr = [&](const uint16_t *cache, const uint16_t *fresh, int vi) -> const uint16_t * {
        const int vv = min(vi, v1 - 1);
        const int pos = vv < sink_len ? vv : win_start + (vv - sink_len);
        return (fresh && pos == n - 1) ? fresh : cache + (size_t)cache_row<RING>(pos, rule) * D;
    };
    auto issue = [&](int cv, DecChunkRegs<D> &r, char *vdst) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint16_t *kp = row_ptr(kc, kn, cv + hh * 16 + l16) + g4 * 8;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                r.k[hh][ks] = __builtin_nontemporal_load((const u32x4 *)(kp + ks * 32));
        }
#pragma unroll
        for (int i = 0; i < VINS; ++i) {
            const int row = i * RPI + lane / CH;
            const int c = lane % CH;
            const uint16_t *vp = row_ptr(vc, vn, cv + row) + ((c ^ dec_swz<D>(row)) << 3);
            __builtin_amdgcn_global_load_lds((const void *)vp, (lds_void_t *)(vdst + i * 1024), 16, 0,
                                             kNonTemporal);
        }
    };

    // Q^T operand: lane l holds head l%16 (zero past G), d = ks*32 + 8*(l/16) .. +8
    bf16x8 qreg[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4 w = {0, 0, 0, 0};
        if (l16 < G) w = *(const u32x4 *)(q + ((size_t)b * hq + kvh * G + l16) * D + ks * 32 + g4 * 8);
        qreg[ks] = __builtin_bit_cast(bf16x8, w);
    }

    f32x4 oacc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.0f;

    // transposed V read: lane (group g4, a = l16/4, bq = l16%4) points at row
    // K0 + a, d columns C0 + 4*bq, and receives rows K0..K0+3 at d = C0 + l16
    const int tr_a = l16 >> 2;
    const int tr_b = l16 & 3;

    auto compute = [&](int cv, const DecChunkRegs<D> &r, const char *vsrc) {
        f32x4 st[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            st[hh] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                st[hh] = mfma16(__builtin_bit_cast(bf16x8, r.k[hh][ks]), qreg[ks], st[hh]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = cv + hh * 16 + 4 * g4 + j < v1;
                st[hh][j] = ok ? st[hh][j] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, st[hh][j]);
            }
        mx = fmaxf(mx, xor16(mx));
        mx = max_xor32(mx);
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kDecRescaleSlack) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float p[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[hh][j] = fast_exp2(st[hh][j] - m_use);
                l_run += p[hh][j];
            }
        const u32x4 pw = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const int r0 = 4 * g4 + tr_a;   // rows of half 0; half 1 is r0 + 16
        const int r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const int col = dt * 16 + 4 * tr_b;
            const int off0 = r0 * (D * 2) + (((col >> 3) ^ dec_swz<D>(r0)) << 4) + (col & 7) * 2;
            const int off1 = r1 * (D * 2) + (((col >> 3) ^ dec_swz<D>(r1)) << 4) + (col & 7) * 2;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(vsrc + off0));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t *)(vsrc + off1));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 aw = {lo2[0], lo2[1], hi2[0], hi2[1]};
            oacc[dt] = mfma16(__builtin_bit_cast(bf16x8, aw), pb, oacc[dt]);
        }
    };

    if constexpr (ONE) {
        const int cv = v0 + wave * kDecChunk;
        if (cv < v1) {
            DecChunkRegs<D> ra;
            issue(cv, ra, vbuf0[wave]);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            compute(cv, ra, vbuf0[wave]);
        }
    } else {
    // software-pipelined chunk loop, unrolled by two so each step uses fixed buffers
    DecChunkRegs<D> ra, rb;
    const int stride = kWaves * kDecChunk;
    int cv = v0 + wave * kDecChunk;
    if (cv < v1) issue(cv, ra, vbuf0[wave]);
    while (cv < v1) {
        const int cn = cv + stride;
        if (cn < v1) issue(cn, rb, vbuf1[wave]);
        if (cn < v1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NKS + VINS) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        compute(cv, ra, vbuf0[wave]);
        if (cn >= v1) break;
        const int cm = cn + stride;
        if (cm < v1) issue(cm, ra, vbuf0[wave]);
        if (cm < v1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NKS + VINS) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        compute(cn, rb, vbuf1[wave]);
        cv = cm;
    }
    }

    // per-head totals of this wavefront: lanes l16 + 16*g4 share head l16
    float l_w = l_run + xor16(l_run);
    l_w = sum_xor32(l_w);
    // O^T: lane holds the finished sums for d = dt*16 + 4*g4 + j of head l16
    __syncthreads();  // every wave is done with its V buffers: reuse them for the merge
    float *sm_o = (float *)&vbuf0[0][0];   // [wave][HS][D] floats (<= 32 KiB at D = 128)
    float *sm_m = kPack ? sm_o + kWaves * HS * D : sm_m_s;  // [wave][16]
    float *sm_l = kPack ? sm_m + kWaves * 16 : sm_l_s;      // [wave][16]
    if (l16 < HS) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm_o[((size_t)wave * HS + l16) * D + dt * 16 + 4 * g4 + j] = oacc[dt][j];
    }
    if (g4 == 0) {
        sm_m[wave * 16 + l16] = m_run;
        sm_l[wave * 16 + l16] = l_w;
    }
    __syncthreads();

    // merge the 4 wavefronts in order; write this split's partial (o, lse)
    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 16 + h]);
        const float Mu = M == -INFINITY ? 0.0f : M;
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(sm_m[w * 16 + h] - Mu);
            L += sm_l[w * 16 + h] * f;
            O += sm_o[((size_t)w * HS + h) * D + d] * f;
        }
        const size_t row = ((size_t)b * hq + kvh * G + h) * n_splits + split;
        o_part[row * D + d] = L > 0.0f ? O / L : 0.0f;
        if (d == 0) lse_part[row] = L > 0.0f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
}

// o[b][h] = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, M = max_s lse_s.
// One workgroup per (sequence, query head), one thread per output element d.
// Each wave handles the splits 64 at a time: lane s holds split s's lse and
// weight, the max and the weight sum are fixed DPP / swizzle / permlane trees
// (no LDS, no barrier), and every thread requests its 64 o partials of the chunk
// (at clamped addresses, without branches) together with the lse values, so one
// memory round trip feeds the whole chunk.  The weighted sum runs in ascending
// s with the weight read from its lane, so the result does not depend on timing.
__device__ __forceinline__ float wave_max(float x) { return max_xor32(group_max<32>(x)); }
__device__ __forceinline__ float wave_sum(float x) { return sum_xor32(group_sum<32>(x)); }

template <typename TE, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    const int32_t *__restrict__ cache_len, int max_cache, int hq, int n_splits,
    TE *__restrict__ o, float *__restrict__ lse)
{
    static_assert(D % 64 == 0, "whole waves");
    const int bh = blockIdx.x;
    const int d = threadIdx.x;
    const int lane = d & 63;
    const float *lp = lse_part + (size_t)bh * n_splits;
    const float *op = o_part + (size_t)bh * n_splits * D + d;

    // the first chunk's partials are requested before the lse values are even
    // reduced: they do not depend on them
    float x[64];
    {
        const int cnt = min(64, n_splits);
#pragma unroll
        for (int u = 0; u < 64; ++u) x[u] = op[(size_t)min(u, cnt - 1) * D];
    }
    float m = -INFINITY;
    for (int s = lane; s < n_splits; s += 64) m = fmaxf(m, lp[s]);
    const float M = wave_max(m);
    const float Mu = M == -INFINITY ? 0.0f : M;
    float W = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
        const int cnt = min(64, n_splits - s0);
        if (s0 > 0) {  // caches of more than 64 splits
#pragma unroll
            for (int u = 0; u < 64; ++u) x[u] = op[(size_t)(s0 + min(u, cnt - 1)) * D];
        }
        const float ls = lane < cnt ? lp[s0 + lane] : -INFINITY;
        const float w = ls == -INFINITY ? 0.0f : __expf(ls - Mu);
        W += wave_sum(w);
#pragma unroll
        for (int u = 0; u < 64; ++u)
            acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u)) *
                   x[u];
    }
    const int n = cache_len[bh / hq];
    const bool bad = n < 1 || n > max_cache;  // max_cache: INT_MAX for ring caches
    const float val = bad ? __builtin_nanf("") : acc / W;
    if constexpr (sizeof(TE) == 2)
        ((uint16_t *)o)[(size_t)bh * D + d] = to_bf16(val);
    else
        ((float *)o)[(size_t)bh * D + d] = val;
    if (lse && d == 0) lse[bh] = bad ? __builtin_nanf("") : M + __logf(W);
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
    if (a.ring)
        decode_split_kernel<TE, D, G, kModeSA, true><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
    else if (a.mode == kModeFA)
        decode_split_kernel<TE, D, G, kModeFA, false><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
    else if (a.mode == kModeSA)
        decode_split_kernel<TE, D, G, kModeSA, false><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
    else
        decode_split_kernel<TE, D, G, kModeMixed, false><<<grid, kThreads, 0, stream>>>(FA_DECODE_ARGS);
#undef FA_DECODE_ARGS
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_bf16(const DecodeArgs &a, hipStream_t stream, const SparseRule &r,
                       float scale_log2)
{
    dim3 grid(a.n_splits, a.batch * a.hkv);
#define FA_DEC16_ARGS                                                                          \
    (const uint16_t *)a.q, (const uint16_t *)a.k_new, (const uint16_t *)a.v_new,                 \
        (uint16_t *)a.k_cache, (uint16_t *)a.v_cache, a.max_cache, a.cache_len, a.route,          \
        a.n_layers, a.layer, a.hq, a.hkv, r, scale_log2, a.split_tokens, a.n_splits, a.o_part,    \
        a.lse_part
    if (a.split_tokens == kWaves * kDecChunk) {  // one chunk per wave
        if (a.ring)
            decode_bf16_kernel<D, G, kModeSA, true, true><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
        else if (a.mode == kModeFA)
            decode_bf16_kernel<D, G, kModeFA, false, true><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
        else if (a.mode == kModeSA)
            decode_bf16_kernel<D, G, kModeSA, false, true><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
        else
            decode_bf16_kernel<D, G, kModeMixed, false, true><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
    } else if (a.ring) {
        decode_bf16_kernel<D, G, kModeSA, true, false><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
    } else if (a.mode == kModeFA) {
        decode_bf16_kernel<D, G, kModeFA, false, false><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
    } else if (a.mode == kModeSA) {
        decode_bf16_kernel<D, G, kModeSA, false, false><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
    } else {
        decode_bf16_kernel<D, G, kModeMixed, false, false><<<grid, kThreads, 0, stream>>>(FA_DEC16_ARGS);
    }
#undef FA_DEC16_ARGS
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_by_g(const DecodeArgs &a, hipStream_t stream, const SparseRule &r,
                            float scale_log2)
{
    switch (a.hq / a.hkv) {
    case 1: return launch_bf16<D, 1>(a, stream, r, scale_log2);
    case 2: return launch_bf16<D, 2>(a, stream, r, scale_log2);
    case 4: return launch_bf16<D, 4>(a, stream, r, scale_log2);
    case 8: return launch_bf16<D, 8>(a, stream, r, scale_log2);
    case 16: return launch_bf16<D, 16>(a, stream, r, scale_log2);
    default: return hipErrorInvalidValue;
    }
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
    SparseRule r{a.ns, a.nw, a.bk_log2, 0};
    const float scale_log2 = a.sm_scale * kLog2e;
    hipError_t e;
    if (a.bf16)
        e = a.d == 128 ? launch_bf16_by_g<128>(a, stream, r, scale_log2)
                       : launch_bf16_by_g<64>(a, stream, r, scale_log2);
    else
        e = a.d == 128 ? launch_by_g<float, 128>(a, stream, r, scale_log2)
                       : launch_by_g<float, 64>(a, stream, r, scale_log2);
    if (e != hipSuccess) return e;
    const int max_len = a.ring ? 0x7fffffff : a.max_cache;
#define FA_MERGE(TE, DD)                                                                      \
    decode_merge_kernel<TE, DD><<<a.batch * a.hq, DD, 0, stream>>>(                            \
        a.o_part, a.lse_part, a.cache_len, max_len, a.hq, a.n_splits, (TE *)a.o, a.lse)
    if (a.bf16) {
        if (a.d == 128) FA_MERGE(uint16_t, 128);
        else FA_MERGE(uint16_t, 64);
    } else {
        if (a.d == 128) FA_MERGE(float, 128);
        else FA_MERGE(float, 64);
    }
#undef FA_MERGE
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation decode entry point: the split partials live in
// this file-scope device array (one copy per GPU the library runs on, held until
// the process ends) instead of a caller workspace.  Host code never uses the
// array's name as an address: on first use on a device its device address is
// looked up once with that device current and kept per device.  Nothing in it
// has to start at zero (every split writes its partial before the merge reads
// it); calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char fa_decode_scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

hipError_t decode_scratch_ptr(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipErrorInvalidDevice;  // the stream's device must be current
    }
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(fa_decode_scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode_noalloc(DecodeArgs a, size_t o_bytes, hipStream_t stream)
{
    void *base = nullptr;
    hipError_t e = decode_scratch_ptr(stream, &base);
    if (e != hipSuccess) return e;
    a.o_part = (float *)base;
    a.lse_part = (float *)((char *)base + o_bytes);
    return launch_decode(a, stream);
}

namespace {

// Copy the tokens an SA layer keeps for the next decode query of every sequence
// (position T_b, query block i = T_b / block) from the packed prefill K/V into
// the compact ring cache: positions [0, min(sink, T_b)) and the window blocks
// max(ns, i - nw + 1) .. i below T_b.  One thread moves 16 bytes.
template <typename TE, int D>
__global__ __launch_bounds__(256) void kv_compact_kernel(
    const TE *__restrict__ k, const TE *__restrict__ v, const int32_t *__restrict__ cu, int hkv,
    SparseRule rule, TE *__restrict__ k_ring, TE *__restrict__ v_ring, int ring)
{
    constexpr int EPL = 16 / sizeof(TE);
    constexpr int LPR = D / EPL;            // threads per row
    constexpr int ROWS = 256 / LPR;         // rows per workgroup
    const int unit = blockIdx.y;
    const int b = unit / hkv, kvh = unit % hkv;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    const int vi = blockIdx.x * ROWS + threadIdx.x / LPR;  // kept-token index
    const int c = threadIdx.x % LPR;
    if (T <= 0) return;
    const int i_q = T >> rule.bk_log2;
    const int sink_tok = rule.ns << rule.bk_log2;
    const int sink_len = min(sink_tok, T);
    const int win_start = min(max(sink_tok, (i_q - rule.nw + 1) << rule.bk_log2), T);
    const int kept = sink_len + (T - win_start);
    if (vi >= kept) return;
    const int pos = vi < sink_len ? vi : win_start + (vi - sink_len);
    const size_t src = ((size_t)(start + pos) * hkv + kvh) * D + c * EPL;
    const size_t dst = (((size_t)b * hkv + kvh) * ring + ring_slot(pos, rule)) * D + c * EPL;
    *(u32x4 *)(k_ring + dst) = *(const u32x4 *)(k + src);
    *(u32x4 *)(v_ring + dst) = *(const u32x4 *)(v + src);
}

template <typename TE, int D>
hipError_t launch_compact_t(const CompactArgs &a, hipStream_t stream)
{
    constexpr int ROWS = 256 / (D / (16 / sizeof(TE)));
    SparseRule r{a.ns, a.nw, a.bk_log2, 0};
    dim3 grid((a.ring + ROWS - 1) / ROWS, a.batch * a.hkv);
    kv_compact_kernel<TE, D><<<grid, 256, 0, stream>>>((const TE *)a.k, (const TE *)a.v,
                                                        a.cu_seqlens, a.hkv, r, (TE *)a.k_ring,
                                                        (TE *)a.v_ring, a.ring);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_compact(const CompactArgs &a, hipStream_t stream)
{
    if (a.bf16) return a.d == 128 ? launch_compact_t<uint16_t, 128>(a, stream)
                                  : launch_compact_t<uint16_t, 64>(a, stream);
    return a.d == 128 ? launch_compact_t<float, 128>(a, stream) : launch_compact_t<float, 64>(a, stream);
}

}  // namespace fa
