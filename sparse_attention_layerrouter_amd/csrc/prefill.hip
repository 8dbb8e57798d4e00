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
//   accumulators (no cross-lane movement) and V^T is read from the row-major
//   V tile by the transposing LDS read ds_read_b64_tr_b16.
// K and V tiles go global -> LDS directly (global_load_lds_dwordx4) into a
// double buffer, each with a 16-byte XOR swizzle chosen so the MFMA operand
// reads are bank-conflict free; the copy of tile i+1 is in flight while tile i
// is computed.
// The causal diagonal and the lower window edge are masked per element, all
// other kept tiles run unmasked.
//
// Generic kernel (fp32, and bf16 shapes the MFMA kernel does not cover): one
// thread per (query row, head), exact online softmax over the same kept
// ranges.  It is the correctness path for fp32 inputs.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBN = 64;        // keys per KV tile
constexpr int kThreads = 256;  // 4 wavefronts
constexpr float kRescaleSlack = 8.0f;  // log2 units

// ---------------------------------------------------------------------------
// LDS layout
// ---------------------------------------------------------------------------
// Each K or V tile is [64 keys][D] bf16, row-major (D*2 bytes per row), and is
// written straight from global memory by global_load_lds_dwordx4: wave
// instruction i fills 1 KiB, lane l's 16 bytes landing at byte 16*l, i.e. row
// l / (D/8), chunk l % (D/8).  The lane chooses WHICH global chunk it fetches,
// so the tile can be stored swizzled: physical chunk c of row r holds logical
// chunk c ^ f(r).
//   K, read by ds_read_b128 with 16 rows per bank sweep at one logical chunk:
//     fK(r) = r % (D/8)  -> the 16 rows hit 16 distinct chunks.
//   V, read by ds_read_b64_tr_b16 with 4 rows x 32 bytes per 16-lane group:
//     fV(r) = 4 (r % 4)  -> the 4 rows of a group land in disjoint chunk pairs.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return (4 * (r & 3)) & (D / 8 - 1); }

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk, int swz)
{
    return row * (D * 2) + ((chunk ^ swz) << 4);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;

// Asynchronous global -> LDS copies of one 64-key K tile and V tile.  Wave
// instruction i of wave w fills 1 KiB block (w * NI + i) of a tile: lane l lands
// at row (block * RPI + l / CH), chunk l % CH, and fetches the logical chunk the
// swizzle stores there.  The copies are buffer loads: the tile base lives in a
// scalar buffer descriptor and each lane's byte offset inside a full tile is a
// fixed 32-bit register, so moving to the next tile costs no vector work.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

template <int D>
struct TileLoader {
    static constexpr int CH = D / 8;              // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;           // rows per wave instruction (1 KiB)
    static constexpr int NI = kBN / (RPI * 4);    // instructions per wave per tensor
    uint32_t off_k[NI], off_v[NI];                // byte offsets inside a full tile
    int row[NI];                                  // tile row of each instruction
    int lds_blk;                                  // first 1 KiB block of this wave
    uint32_t chunk_k[NI], chunk_v[NI];

    __device__ __forceinline__ void init(int wave, int lane, size_t row_stride)
    {
        const int c = lane % CH;
        lds_blk = wave * NI;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            row[i] = (lds_blk + i) * RPI + lane / CH;
            chunk_k[i] = (uint32_t)((c ^ swz_k<D>(row[i])) << 4);
            chunk_v[i] = (uint32_t)((c ^ swz_v<D>(row[i])) << 4);
            off_k[i] = (uint32_t)(row[i] * row_stride * 2) + chunk_k[i];
            off_v[i] = (uint32_t)(row[i] * row_stride * 2) + chunk_v[i];
        }
    }

    // rows k0 .. k0+63 of K and V (bases of the KV head) into dst_k / dst_v;
    // rows past the sequence end are clamped to T - 1 (always masked)
    __device__ __forceinline__ void issue(char *dst_k, char *dst_v, const uint16_t *__restrict__ kb,
                                          const uint16_t *__restrict__ vb, size_t row_stride,
                                          int k0, int T) const
    {
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kb + (size_t)k0 * row_stride), (short)0, 0x7fffffff, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vb + (size_t)k0 * row_stride), (short)0, 0x7fffffff, kRsrcWord3);
        if (k0 + kBN <= T) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (lds_void *)(dst_k + (lds_blk + i) * 1024), 16, (int)off_k[i], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (lds_void *)(dst_v + (lds_blk + i) * 1024), 16, (int)off_v[i], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const uint32_t r = (uint32_t)min(row[i], T - 1 - k0) * (uint32_t)(row_stride * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (lds_void *)(dst_k + (lds_blk + i) * 1024), 16, (int)(r + chunk_k[i]), 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (lds_void *)(dst_v + (lds_blk + i) * 1024), 16, (int)(r + chunk_v[i]), 0, 0, 0);
            }
        }
    }
};

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
    constexpr int TILE_BYTES = kBN * D * 2;
    // [buffer][K, V] tiles, double-buffered
    __shared__ __attribute__((aligned(1024))) char lds[2 * 2 * TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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
    TileLoader<D> loader;
    loader.init(wave, lane, row_stride);
    loader.issue(lds, lds + TILE_BYTES, kb, vb, row_stride, 0, T);

    // ---- Q^T operand in registers: lane holds row pw0 + l32, d = ks*16 + half*8 ..
    bf16x8 qreg[D / 16];
    {
        int t = min(pw0 + l32, T - 1);
        const uint16_t *qr = q + ((size_t)(start + t) * hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qreg[ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qr + ks * 16 + half * 8));
    }

    // masking thresholds for this wave
    const int sink_tok = rule.ns << rule.bk_log2;
    const int win_lo_max = ((pw_last >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;
    const int my_t = min(pw0 + l32, T - 1);  // query position of this lane's row
    const int my_win_lo = ((my_t >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;

    // Per-lane LDS byte offsets, fixed for the whole kernel (the buffer and the
    // 32-key block only add constants, which become instruction offsets):
    //   K operand of d step ks: key l32 (+32 for the second block), logical
    //   chunk 2 ks + half, stored at chunk ^ swz_k(key) -- swz_k(key) depends on
    //   l32 only.
    //   V^T operand of d block dt: the transposed read of lane (a = (l%16)/4,
    //   bq = l%4) points at key row 4 half + a (+16 per k step, +8 for the upper
    //   4 keys), d columns C0 + 4 bq .. +3 with C0 = 32 dt + 16 ((l/16) % 2); the
    //   instruction hands lane l the 4 keys of its group at d = C0 + l%16.  The
    //   V swizzle depends on key row % 4 = a only.
    uint32_t koff[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        koff[ks] = (uint32_t)tile_off<D>(l32, ks * 2 + half, swz_k<D>(l32));
    uint32_t voff[D / 32];
    {
        const int tr_a = (lane & 15) >> 2;
        const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int r0 = 4 * half + tr_a;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int col = dt * 32 + tr_col;
            voff[dt] = (uint32_t)(tile_off<D>(r0, col >> 3, swz_v<D>(r0)) + (col & 7) * 2);
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // reference max, log2 domain
    float l_run = 0.0f;       // this lane's share of the row sum

    // One KV tile; BUF (the LDS buffer it sits in) is a compile-time constant so
    // every LDS address is a fixed register plus an instruction offset.
    auto tile_step = [&](auto buf_tag, int it) {
        constexpr int BUF = decltype(buf_tag)::value;
        const int kt = it < nA ? it : tB0 + (it - nA);
        const int k0 = kt * kBN;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile `it` landed; the other buffer is free again
        if (it + 1 < n_tiles) {
            const int kn = (it + 1) < nA ? it + 1 : tB0 + (it + 1 - nA);
            char *nk = lds + (1 - BUF) * 2 * TILE_BYTES;
            loader.issue(nk, nk + TILE_BYTES, kb, vb, row_stride, kn * kBN, T);
        }
        if (!wave_active || k0 > pw_last) return;  // nothing visible for this wave
        constexpr uint32_t kbase = BUF * 2 * TILE_BYTES;
        constexpr uint32_t vbase = kbase + TILE_BYTES;

        // ---- S^T = K Q^T : two 32-key blocks
        f32x16 s[2];
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const uint32_t off = koff[ks] + kbase + kb2 * 32 * D * 2;
                bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4 *)(lds + off));
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

        // ---- online softmax (exp2 domain) with a lazily moved reference max:
        // the reference m_ref only moves when a row's tile max exceeds it by more
        // than kRescaleSlack (log2 units), so p = 2^(s - m_ref) <= 2^kRescaleSlack
        // and the O / l rescale runs on few tiles.  O / l is independent of the
        // reference, so the result is the same softmax.
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[kb2][j]);
        mx = max_xor32(mx) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.0f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
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
        l_run += psum;

        // ---- O^T += V^T P^T : 4 k-steps of 16 keys.  P^T for k-step ksv is the
        // lane's own S^T values 8*(ksv%2) .. +8 of block ksv/2: k index
        // 8*half + e <-> key 16*ksv + 8*(e/4) + 4*half + e%4.
#pragma unroll
        for (int ksv = 0; ksv < 4; ++ksv) {
            const int kb2 = ksv >> 1, jb = (ksv & 1) * 4;
            u32x4 pw = {pk[kb2][jb], pk[kb2][jb + 1], pk[kb2][jb + 2], pk[kb2][jb + 3]};
            bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const uint32_t off_lo = voff[dt] + vbase + ksv * 16 * D * 2;
                const uint32_t off_hi = off_lo + 8 * D * 2;
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(lds + off_lo));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(lds + off_hi));
                u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                u32x4 aw = {lo2[0], lo2[1], hi2[0], hi2[1]};
                oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, aw), pb, oacc[dt]);
            }
        }
    };

    for (int it = 0; it < n_tiles; it += 2) {
        tile_step(std::integral_constant<int, 0>{}, it);
        if (it + 1 < n_tiles) tile_step(std::integral_constant<int, 1>{}, it + 1);
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
