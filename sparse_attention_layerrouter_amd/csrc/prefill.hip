// prefill.hip -- prefill attention of one layer for FA and SA sequences (gfx950).
//
// FA layers run dense causal GQA attention (the FlashAttention-2 dense path of
// [thelatestinai paper page, Table 6]; query head h reads KV head h / G as
// `repeat_kv` does in the codewithpapers function list).  SA layers run the
// streaming block-sparse form: only the sink blocks and the local window of
// blocks are visited [thelatestinai paper page, Table 6], so their KV tiles
// are two contiguous runs and every skipped tile is never loaded.
//
// bf16 kernel (head_dim 128 or 64): one workgroup of 4 wavefronts owns 128
// query rows that share one KV head (GQA stacking: 4 heads x 32 positions when
// G >= 4), so every K/V tile staged in LDS serves 128 rows.  Per 64-key tile:
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T in registers);
//   online softmax in the exp2 domain, row statistics per lane;
//   O^T += V^T P^T on the same MFMA; P^T comes straight out of the S^T
//   accumulators (no cross-lane movement) and V^T is staged transposed in LDS.
// K is stored row-major with a 16-byte XOR swizzle, V^T with an 8-byte XOR
// swizzle; both make the MFMA operand reads and the tile writes bank-conflict
// free.  Global->register prefetch of tile i+1 overlaps the MFMAs of tile i.
// The causal diagonal and the lower window edge are masked per element, all
// other kept tiles run unmasked.
//
// Generic kernel (fp32, and bf16 shapes the MFMA kernel does not cover): one
// thread per (query row, head), exact online softmax over the same kept
// ranges.  It is the correctness path for fp32 inputs.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBN = 64;        // keys per KV tile
constexpr int kThreads = 256;  // 4 wavefronts

// ---------------------------------------------------------------------------
// LDS layouts
// ---------------------------------------------------------------------------
// K tile: [64 keys][D] bf16, row stride D*2 bytes, 16-byte chunk c of key r
// stored at chunk c ^ (r % (D/8)).
template <int D>
__device__ __forceinline__ int k_lds_off(int key, int chunk)
{
    constexpr int CH = D / 8;
    return key * (D * 2) + ((chunk ^ (key & (CH - 1))) << 4);
}
// V^T tile: [D][64 keys] bf16, row stride 128 bytes, 8-byte slot s (4 keys) of
// row d stored at slot s ^ g(d), g(d) = (d % 16) ^ ((d / 8) % 16).
__device__ __forceinline__ int vt_lds_off(int d, int slot)
{
    int g = (d & 15) ^ ((d >> 3) & 15);
    return d * 128 + ((slot ^ g) << 3);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D>
struct TileRegs {
    // K: D/32 passes of one 16-byte chunk; V: D/32 passes of 4 keys x 8 d
    u32x4 k[D / 32];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &r, const uint16_t *__restrict__ kb,
                                          const uint16_t *__restrict__ vb, size_t row_stride,
                                          int k0, int T, int tid)
{
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int RPP = kThreads / CH;   // rows per pass
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        int key = tid / CH + RPP * i;
        int c = tid % CH;
        int s = k0 + key;
        if (s < T)
            r.k[i] = *(const u32x4 *)(kb + (size_t)s * row_stride + c * 8);
        else
            r.k[i] = u32x4{0, 0, 0, 0};
    }
    // V: unit = (4 keys, 8 d); D/8 * 16 units; threads past the unit count idle.
    constexpr int UNITS = CH * 16;
    if (tid < UNITS) {
        int c = tid % CH, kg = tid / CH;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int s = k0 + kg * 4 + j;
            if (s < T)
                r.v[j] = *(const u32x4 *)(vb + (size_t)s * row_stride + c * 8);
            else
                r.v[j] = u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &r, char *k_lds, char *vt_lds, int tid)
{
    constexpr int CH = D / 8;
    constexpr int RPP = kThreads / CH;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        int key = tid / CH + RPP * i;
        int c = tid % CH;
        *(u32x4 *)(k_lds + k_lds_off<D>(key, c)) = r.k[i];
    }
    constexpr int UNITS = CH * 16;
    if (tid < UNITS) {
        int c = tid % CH, kg = tid / CH;
        // r.v[j] holds key kg*4+j, d = 8c .. 8c+7 (two bf16 per dword).
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // d = 8c + 2w (low halves) and 8c + 2w + 1 (high halves)
            uint32_t a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
            uint32_t lo01 = __builtin_amdgcn_perm(a1, a0, 0x05040100);
            uint32_t lo23 = __builtin_amdgcn_perm(a3, a2, 0x05040100);
            uint32_t hi01 = __builtin_amdgcn_perm(a1, a0, 0x07060302);
            uint32_t hi23 = __builtin_amdgcn_perm(a3, a2, 0x07060302);
            int d0 = 8 * c + 2 * w;
            *(u32x2 *)(vt_lds + vt_lds_off(d0, kg)) = u32x2{lo01, lo23};
            *(u32x2 *)(vt_lds + vt_lds_off(d0 + 1, kg)) = u32x2{hi01, hi23};
        }
    }
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One workgroup: 4 waves x 32 query rows.  Wave w handles head
// h0 + w / WPH and positions p0 + (w % WPH) * 32 .. +32, WPH = 4 / HPW.
template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, const uint8_t *__restrict__ route, int n_layers, int layer,
    int hq, int hkv, int G, int hpw, int n_hgroups, int n_units, int n_ptiles,
    SparseRule rule, float scale_log2)
{
    __shared__ __attribute__((aligned(16))) char k_lds[kBN * D * 2];
    __shared__ __attribute__((aligned(16))) char vt_lds[D * kBN * 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // blockIdx -> (position tile, head group, unit) with the unit (sequence, kv
    // head) fastest, so consecutive workgroups -- which the dispatcher spreads
    // round-robin over the 8 XCDs -- keep one KV head per XCD when the unit
    // count is a multiple of 8.  Position tiles run last-first: the causal tail
    // tiles carry the most KV tiles and start first.
    int bid = blockIdx.x;
    const int unit = bid % n_units;
    bid /= n_units;
    const int hg = bid % n_hgroups;
    const int ptile = n_ptiles - 1 - bid / n_hgroups;
    const int b = unit / hkv, kvh = unit % hkv;

    const int start = cu[b];
    const int T = cu[b + 1] - start;
    const int wph = 4 / hpw;             // waves per head
    const int bm_pos = 32 * wph;         // positions per workgroup
    const int p0 = ptile * bm_pos;
    if (p0 >= T) return;
    const int p1 = min(p0 + bm_pos, T);
    const bool is_fa = MODE == kModeFA ? true
                       : MODE == kModeSA ? false
                                         : route[(size_t)b * n_layers + layer] != 0;

    const int h = kvh * G + hg * hpw + wave / wph;
    const int pw0 = p0 + (wave % wph) * 32;   // this wave's first position
    const bool wave_active = pw0 < T;
    const int pw_last = min(pw0 + 31, T - 1);  // last valid position of the wave

    // ---- Q^T operand in registers: lane holds row pw0 + l32, d = ks*16 + half*8 ..
    bf16x8 qreg[D / 16];
    {
        int t = min(pw0 + l32, T - 1);
        const uint16_t *qr = q + ((size_t)(start + t) * hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qr + ks * 16 + half * 8));
    }

    // ---- KV tile schedule: [0, nA) then [tB0, tB0 + nB)
    int a_end, b_begin;
    kept_ranges(p0, p1, is_fa, rule, a_end, b_begin);
    const int nA = (a_end + kBN - 1) / kBN;
    const int tB0 = max(nA, b_begin / kBN);
    const int tB1 = (p1 + kBN - 1) / kBN;
    const int nB = max(0, tB1 - tB0);
    const int n_tiles = nA + nB;

    const size_t row_stride = (size_t)hkv * D;
    const uint16_t *kb = k + ((size_t)start * hkv + kvh) * D;
    const uint16_t *vb = v + ((size_t)start * hkv + kvh) * D;

    // masking thresholds for this wave
    const int sink_tok = rule.ns << rule.bk_log2;
    const int win_lo_max = ((pw_last >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;
    const int my_t = min(pw0 + l32, T - 1);  // query position of this lane's row
    const int my_win_lo = ((my_t >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // running max, log2 domain
    float l_run = 0.0f;       // this lane's share of the row sum

    TileRegs<D> regs;
    if (n_tiles > 0) load_tile<D>(regs, kb, vb, row_stride, 0 * kBN, T, tid);

    for (int it = 0; it < n_tiles; ++it) {
        const int kt = it < nA ? it : tB0 + (it - nA);
        const int k0 = kt * kBN;
        __syncthreads();  // previous tile fully consumed
        store_tile<D>(regs, k_lds, vt_lds, tid);
        __syncthreads();
        if (it + 1 < n_tiles) {
            const int kn = (it + 1) < nA ? it + 1 : tB0 + (it + 1 - nA);
            load_tile<D>(regs, kb, vb, row_stride, kn * kBN, T, tid);
        }
        if (!wave_active || k0 > pw_last) continue;  // nothing visible for this wave

        // ---- S^T = K Q^T : two 32-key blocks
        f32x16 s[2];
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                int key = kb2 * 32 + l32;
                bf16x8 a = __builtin_bit_cast(
                    bf16x8, *(const u32x4 *)(k_lds + k_lds_off<D>(key, ks * 2 + half)));
                s[kb2] = mfma32(a, qreg[ks], s[kb2]);
            }
        }

        // ---- mask (causal diagonal, window lower edge, sequence tail)
        const bool need_mask = (k0 + kBN - 1 > pw0) ||
                               (!is_fa && k0 < win_lo_max && k0 + kBN > sink_tok);
        if (need_mask) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    int key = k0 + kb2 * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
                    bool vis = key <= my_t &&
                               (is_fa || key < sink_tok || key >= my_win_lo);
                    if (!vis) s[kb2][j] = -INFINITY;
                }
        }

        // ---- online softmax (exp2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb2][j]);
        mx = max_xor32(mx);
        const float m_new = fmaxf(m_run, mx * scale_log2);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.0f;
        uint32_t pk[2][8];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                float e0 = fast_exp2(s[kb2][j] * scale_log2 - m_use);
                float e1 = fast_exp2(s[kb2][j + 1] * scale_log2 - m_use);
                psum += e0 + e1;
                pk[kb2][j / 2] = pack_bf16x2(e0, e1);
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;

        // ---- O^T += V^T P^T : 4 k-steps of 16 keys
#pragma unroll
        for (int ksv = 0; ksv < 4; ++ksv) {
            const int kb2 = ksv >> 1, jb = (ksv & 1) * 4;
            u32x4 pw = {pk[kb2][jb], pk[kb2][jb + 1], pk[kb2][jb + 2], pk[kb2][jb + 3]};
            bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                int d = dt * 32 + l32;
                u32x2 lo = *(const u32x2 *)(vt_lds + vt_lds_off(d, 4 * ksv + half));
                u32x2 hi = *(const u32x2 *)(vt_lds + vt_lds_off(d, 4 * ksv + 2 + half));
                u32x4 aw = {lo[0], lo[1], hi[0], hi[1]};
                oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, aw), pb, oacc[dt]);
            }
        }
    }

    if (!wave_active) return;
    // ---- epilogue: O = O^T / l, lse = (m + log2 l) ln 2
    const float l_tot = sum_xor32(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int t = pw0 + l32;
    if (t < T) {
        uint16_t *orow = o + ((size_t)(start + t) * hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                int d = dt * 32 + 8 * jg + 4 * half;
                u32x2 w = {pack_bf16x2(oacc[dt][4 * jg] * inv, oacc[dt][4 * jg + 1] * inv),
                           pack_bf16x2(oacc[dt][4 * jg + 2] * inv, oacc[dt][4 * jg + 3] * inv)};
                *(u32x2 *)(orow + d) = w;
            }
        if (lse && half == 0)
            lse[(size_t)(start + t) * hq + h] = (m_run + fast_log2(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: one thread per (query row, head), exact online softmax.
// ---------------------------------------------------------------------------
template <typename TE, int D>
__device__ __forceinline__ float ld_elem(const TE *p, int i)
{
    if constexpr (sizeof(TE) == 2)
        return __uint_as_float((uint32_t)((const uint16_t *)p)[i] << 16);
    else
        return ((const float *)p)[i];
}

template <typename TE, int D, int MODE>
__global__ __launch_bounds__(64) void prefill_generic_kernel(
    const TE *__restrict__ q, const TE *__restrict__ k, const TE *__restrict__ v,
    TE *__restrict__ o, float *__restrict__ lse, const int32_t *__restrict__ cu,
    const uint8_t *__restrict__ route, int n_layers, int layer, int hq, int hkv,
    SparseRule rule, float scale_log2)
{
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    const int p0 = blockIdx.x * 64;
    if (p0 >= T) return;
    const int p1 = min(p0 + 64, T);
    const int t = min(p0 + (int)threadIdx.x, T - 1);
    const bool is_fa = MODE == kModeFA ? true
                       : MODE == kModeSA ? false
                                         : route[(size_t)b * n_layers + layer] != 0;
    const int G = hq / hkv;
    const int g = h / G;

    float qv[D], acc[D];
    const TE *qr = q + ((size_t)(start + t) * hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qv[c] = ld_elem<TE, D>(qr, c) * scale_log2;
        acc[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    int a_end, b_begin;
    kept_ranges(p0, p1, is_fa, rule, a_end, b_begin);
    for (int pass = 0; pass < 2; ++pass) {
        int s0 = pass == 0 ? 0 : b_begin;
        int s1 = pass == 0 ? a_end : p1;
        for (int s = s0; s < s1; ++s) {
            if (!visible(t, s, is_fa, rule)) continue;
            const TE *kr = k + ((size_t)(start + s) * hkv + g) * D;
            const TE *vr = v + ((size_t)(start + s) * hkv + g) * D;
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot += qv[c] * ld_elem<TE, D>(kr, c);
            float m_new = fmaxf(m, dot);
            float alpha = fast_exp2(m - m_new);
            float p = fast_exp2(dot - m_new);
            l = l * alpha + p;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = acc[c] * alpha + p * ld_elem<TE, D>(vr, c);
            m = m_new;
        }
    }
    if (p0 + (int)threadIdx.x >= T) return;
    const float inv = 1.0f / l;
    TE *orow = o + ((size_t)(start + t) * hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        if constexpr (sizeof(TE) == 2)
            ((uint16_t *)orow)[c] = to_bf16(acc[c] * inv);
        else
            ((float *)orow)[c] = acc[c] * inv;
    }
    if (lse) lse[(size_t)(start + t) * hq + h] = (m + fast_log2(l)) * kLn2;
}

template <typename TE, int D, int MODE>
hipError_t launch_generic(const PrefillArgs &a, hipStream_t stream, const SparseRule &r,
                          float scale_log2)
{
    dim3 grid((a.max_seqlen + 63) / 64, a.hq, a.batch);
    prefill_generic_kernel<TE, D, MODE><<<grid, 64, 0, stream>>>(
        (const TE *)a.q, (const TE *)a.k, (const TE *)a.v, (TE *)a.o, a.lse, a.cu_seqlens,
        a.route, a.n_layers, a.layer, a.hq, a.hkv, r, scale_log2);
    return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_mfma(const PrefillArgs &a, hipStream_t stream, const SparseRule &r,
                       float scale_log2)
{
    const int G = a.hq / a.hkv;
    const int hpw = G >= 4 ? 4 : G;
    const int n_hgroups = G / hpw;
    const int bm_pos = 32 * (4 / hpw);
    const int n_ptiles = (a.max_seqlen + bm_pos - 1) / bm_pos;
    const int n_units = a.batch * a.hkv;
    const long long n_wg = (long long)n_ptiles * n_hgroups * n_units;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    prefill_bf16_kernel<D, MODE><<<(unsigned)n_wg, kThreads, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o,
        a.lse, a.cu_seqlens, a.route, a.n_layers, a.layer, a.hq, a.hkv, G, hpw, n_hgroups,
        n_units, n_ptiles, r, scale_log2);
    return hipGetLastError();
}

bool prefill_mfma_supported(int d, int G)
{
    return (d == 128 || d == 64) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

template <int MODE>
hipError_t launch_mode(const PrefillArgs &a, hipStream_t stream, const SparseRule &r,
                       float scale_log2)
{
    const int G = a.hq / a.hkv;
    if (a.bf16 && prefill_mfma_supported(a.d, G)) {
        if (a.d == 128) return launch_mfma<128, MODE>(a, stream, r, scale_log2);
        return launch_mfma<64, MODE>(a, stream, r, scale_log2);
    }
    if (a.bf16) {
        if (a.d == 128) return launch_generic<uint16_t, 128, MODE>(a, stream, r, scale_log2);
        return launch_generic<uint16_t, 64, MODE>(a, stream, r, scale_log2);
    }
    if (a.d == 128) return launch_generic<float, 128, MODE>(a, stream, r, scale_log2);
    return launch_generic<float, 64, MODE>(a, stream, r, scale_log2);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    SparseRule r{a.ns, a.nw, a.bk_log2};
    const float scale_log2 = a.sm_scale * kLog2e;
    switch (a.mode) {
    case kModeFA: return launch_mode<kModeFA>(a, stream, r, scale_log2);
    case kModeSA: return launch_mode<kModeSA>(a, stream, r, scale_log2);
    default: return launch_mode<kModeMixed>(a, stream, r, scale_log2);
    }
}

}  // namespace fa
