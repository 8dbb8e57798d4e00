// prefill.hip -- prefill attention of one layer for FA and SA sequences (gfx950).
//
// FA layers run dense causal GQA attention (the FlashAttention-2 dense path of
// [thelatestinai paper page, Table 6]; query head h reads KV head h / G as
// `repeat_kv` does in the codewithpapers function list).  SA layers run the
// streaming block-sparse form: only the sink blocks and the local window of
// blocks are visited [thelatestinai paper page, Table 6], so their KV tiles
// are two contiguous runs and every skipped tile is never loaded.
//
// bf16 kernel (head_dim 128 or 64): one workgroup of 8 wavefronts owns 256
// query rows that share one KV head (GQA stacking: 4 heads x 64 positions when
// G >= 4), so every K/V tile staged in LDS serves 256 rows.  Per 64-key tile
// and wave (32 query rows, two row groups of 16):
//   S^T = K Q^T  on v_mfma_f32_16x16x32_bf16 (K from LDS, Q^T in registers),
//   each K fragment read once for both row groups;
//   online softmax in the exp2 domain, row statistics per lane and row group;
//   O^T += V^T P^T on the same MFMA, each V^T fragment read once for both row
//   groups; P^T comes straight out of the S^T accumulators (no cross-lane
//   movement) and V^T is read from the row-major V tile by the transposing
//   LDS read ds_read_b64_tr_b16.
// The 16x16x32 product moves a quarter of the accumulator bytes per flop of
// the 32x32x16 one: under the board's power limit the kernel then runs at a
// higher clock for the same LDS bytes and VALU work per flop.
// The 8 waves form two groups that ping-pong: while one group's softmax keeps
// the vector ALUs busy, the other group's QK and PV products keep the matrix
// cores of the same SIMDs busy (one wave of each group per SIMD); a single
// wave cannot overlap the two itself, because its softmax depends on its own
// QK and its PV on its own softmax.
// K and V tiles go global -> LDS directly (buffer_load ... lds) into a double
// buffer, each with a 16-byte XOR swizzle chosen so the MFMA operand reads are
// bank-conflict free; the copies of the next tiles are in flight while the
// current ones are computed.  The causal diagonal and the lower window edge
// are masked per element, all other kept tiles run unmasked.
//
// Generic kernel (fp32, and bf16 shapes the MFMA kernel does not cover): one
// thread per (query row, head), exact online softmax over the same kept
// ranges.  It is the correctness path for fp32 inputs.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBN = 64;                // keys per KV tile
constexpr int kWaves = 8;              // two ping-pong groups of 4 wavefronts
constexpr int kThreads = 64 * kWaves;
constexpr float kFastLimit = 65536.0f;  // largest p without a rescale

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
//   V, read by ds_read_b64_tr_b16 with 4 rows x 32 bytes per 16-lane group,
//   the two groups of a 32-lane bank sweep 4 rows apart at the same columns:
//     fV(r) = 4 (r % 4) ^ 2 ((r / 4) % 2)  -> the 8 rows of a sweep land in
//     disjoint chunk pairs.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return (4 * (r & 3) ^ 2 * ((r >> 2) & 1)) & (D / 8 - 1); }

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

// Asynchronous global -> LDS copies of one 64-key K or V tile by the 4 waves of
// ping-pong group 0.  Wave instruction i of wave w fills 1 KiB block (w * NI + i)
// of the tile: lane l lands at row (block * RPI + l / CH), chunk l % CH, and
// fetches the logical chunk the swizzle stores there.  The copies are buffer
// loads: the tile base lives in a scalar buffer descriptor and each lane's byte
// offset inside a full tile is a fixed 32-bit register, so a copy costs no
// vector work.  The descriptor's size ends at the sequence end: rows past it
// read as zero (and are masked).
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kLoadWaves = 4;

template <int D, bool IS_V>
struct TileLoader {
    static constexpr int CH = D / 8;                     // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;                  // rows per wave instruction (1 KiB)
    static constexpr int NI = kBN / (RPI * kLoadWaves);  // instructions per wave
    static_assert(NI >= 1 && NI * RPI * kLoadWaves == kBN, "tile split over the waves");
    uint32_t off[NI];    // byte offset inside a full tile
    int lds_blk;         // first 1 KiB block of this wave

    __device__ __forceinline__ void init(int wave, int lane, size_t row_stride)
    {
        const int c = lane % CH;
        lds_blk = wave * NI;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = (lds_blk + i) * RPI + lane / CH;
            const int chunk = c ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
            off[i] = (uint32_t)(row * row_stride * 2) + (uint32_t)(chunk << 4);
        }
    }

    // descriptor of rows k0 .. T-1 of one KV head (an empty range when k0 >= T:
    // in mode XA the second 64-key tile of a sequence's last block can start
    // past its end, and a negative count would lift the range check)
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *__restrict__ base,
                                                               size_t row_stride, int k0, int T)
    {
        const long long bytes = (long long)max(T - k0, 0) * (long long)row_stride * 2;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (size_t)k0 * row_stride), (short)0,
                                                 (int)min(bytes, 0x7fffffffLL), kRsrcWord3);
    }

    __device__ __forceinline__ void issue_one(int i, char *dst, __amdgpu_buffer_rsrc_t r) const
    {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + (lds_blk + i) * 1024), 16,
                                                 (int)off[i], 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int V>
using ic = std::integral_constant<int, V>;

// One workgroup: two groups of 4 waves, 32 query rows per wave.  In group g,
// wave w handles head h0 + w / WPH and positions p0 + g * GP + (w % WPH) * 32
// .. +32, WPH = 4 / HPW, GP = 32 * WPH.
//
// Ping-pong: a wave's work on KV tile t is an MFMA block M_t (O^T += V^T P^T
// of tile t-1, then S^T = K Q^T of tile t) followed by a VALU block V_t (mask,
// online softmax, P of tile t).  Group 0 runs M_0 V_0 M_1 V_1 ..., group 1 the
// same one phase later, and every even phase starts at a workgroup barrier, so
// while one group's softmax occupies the vector ALUs the other group's products
// occupy the matrix cores of the same SIMDs.  The barriers also order the
// double-buffered tiles: at phase 2j every wave waits for the copies it issued
// at phase 2j-2 (K of tile j, V of tile j-1) and issues K of tile j+1 and V of
// tile j into the buffers whose previous tiles were last read at phase 2j-1
// (every wave drains its LDS reads before the barrier).  Odd phases need no
// barrier: nothing is copied there, and the pair of blocks between two even
// barriers keeps the groups one block apart on its own (a barrier there
// measured 1.6 % slower).
template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ cu_k,
    const uint8_t *__restrict__ route, int n_layers, int layer,
    int hq, int hkv, int G, int hpw, int n_hgroups, int n_units, int n_ptiles,
    SparseRule rule, float scale_log2, const uint32_t *__restrict__ xa_mask, int xa_nqb,
    int xa_nw)
{
    constexpr int TILE_BYTES = kBN * D * 2;
    constexpr bool XA = MODE == kModeXA;
    // XA: kept-block words of the workgroup's heads, their union as a block list
    // (entry: block index | bit 16 + hh set when head hh keeps the block)
    __shared__ uint32_t xa_head[XA ? 4 : 1][XA ? 128 : 1];
    __shared__ uint32_t xa_list[XA ? 4096 : 1];
    __shared__ int xa_pre[XA ? 129 : 1];
    // separate arrays per buffer: the compiler can then tell that reads of one
    // buffer never wait for the asynchronous copies into the other
    __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = wave >> 2;
    const int wq = wave & 3;
    const int half = lane >> 5;
    const int l32 = lane & 31;

    // blockIdx -> (unit (sequence, kv head), head group, position tile).  The
    // dispatcher deals consecutive workgroups round-robin to the 8 XCDs, each
    // with its own L2.  When the unit count is a multiple of 8, XCD x (blockIdx
    // mod 8) walks the units 8u + x one at a time, all of a unit's workgroups
    // before the next, so its CUs stream one KV head's tiles in step and share
    // them in L2 (a varlen batch would otherwise interleave its sequences on
    // every XCD).  Otherwise the unit is the fastest index.  Within a unit,
    // position tiles run last-first: the causal tail tiles carry the most KV
    // tiles and start first.
    int unit, hg, ptile;
    if (n_units % 8 == 0) {  // uniform
        const int m = blockIdx.x >> 3;
        const int per_unit = n_hgroups * n_ptiles;
        const int u = m / per_unit, rem = m - u * per_unit;
        unit = 8 * u + (blockIdx.x & 7);
        hg = rem % n_hgroups;
        ptile = n_ptiles - 1 - rem / n_hgroups;
    } else {
        int bid = blockIdx.x;
        unit = bid % n_units;
        bid /= n_units;
        hg = bid % n_hgroups;
        ptile = n_ptiles - 1 - bid / n_hgroups;
    }
    const int b = unit / hkv, kvh = unit % hkv;

    // Query rows of sequence b are cu[b] .. cu[b+1]-1 and its keys cu_k[b] ..
    // cu_k[b+1]-1; the Tq queries are the last Tq of the T tokens, so query row
    // r sits at position q_off + r (q_off = 0 when queries and keys coincide).
    const int start_q = cu[b];
    const int Tq = cu[b + 1] - start_q;
    const int start = cu_k[b];
    const int T = cu_k[b + 1] - start;
    const int q_off = T - Tq;
    const int wph = 4 / hpw;        // waves per head in a group
    const int gpos = 32 * wph;      // positions per group
    const int r0 = ptile * 2 * gpos;
    if (r0 >= Tq) return;           // uniform: the whole workgroup leaves
    const int h = kvh * G + hg * hpw + wq / wph;
    if (q_off < 0) {                // more queries than keys: NaN rows, nothing read
        const int r = r0 + grp * gpos + (wq % wph) * 32 + l32;
        if (r < Tq) {
            uint16_t *orow = o + ((size_t)(start_q + r) * hq + h) * D;
            for (int d = half; d < D; d += 2) orow[d] = 0x7fc0u;
            if (lse && half == 0) lse[(size_t)(start_q + r) * hq + h] = __builtin_nanf("");
        }
        return;
    }
    const int p0 = q_off + r0;      // positions of this workgroup: p0 .. p1-1
    const int p1 = min(p0 + 2 * gpos, T);
    const bool is_fa = MODE == kModeFA || MODE == kModeXA ? true
                       : MODE == kModeSA ? false
                                         : route[(size_t)b * n_layers + layer] != 0;
    // Triangle attention: rows at or past tail0 keep every key (the whole
    // sequence when is_fa); otherwise only the sink and window blocks
    const int tail0 = is_fa ? 0 : dense_tail_start(T, rule);

    const int pw0 = p0 + grp * gpos + (wq % wph) * 32;  // this wave's first position
    const bool wave_active = pw0 < T;
    const int pw_last = min(pw0 + 31, T - 1);  // last valid position of the wave
    // (is_fa first: FA and XA kernels fold every dense-tail test away)
    const bool w_dense_any = is_fa || pw_last >= tail0;  // some row of the wave keeps every key
    const bool w_dense_all = is_fa || pw0 >= tail0;      // every row does

    // ---- KV tile schedule: [0, nA) then [tB0, tB0 + nB); in mode XA the kept
    // blocks of the workgroup's query block (all its positions lie in one block),
    // the union over its heads in ascending order, each block kBN-tiled.
    int nA = 0, tB0 = 0, n_tiles = 0;
    if constexpr (XA) {
        const int qi = p0 >> rule.bk_log2;
        const size_t hstep = (size_t)xa_nqb * xa_nw;
        const uint32_t *mrow =
            xa_mask + (((size_t)b * hq + kvh * G + hg * hpw) * xa_nqb + qi) * xa_nw;
        for (int w = tid; w < xa_nw; w += kThreads) {
            uint32_t u = 0;
            for (int hh = 0; hh < hpw; ++hh) {
                const uint32_t x = mrow[hh * hstep + w];
                xa_head[hh][w] = x;
                u |= x;
            }
            xa_pre[w + 1] = __builtin_popcount(u);
        }
        __syncthreads();
        if (tid == 0) {
            xa_pre[0] = 0;
            for (int w = 0; w < xa_nw; ++w) xa_pre[w + 1] += xa_pre[w];
        }
        __syncthreads();
        for (int w = tid; w < xa_nw; w += kThreads) {
            uint32_t hw[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) hw[hh] = hh < hpw ? xa_head[hh][w] : 0u;
            uint32_t u = (hw[0] | hw[1]) | (hw[2] | hw[3]);
            int o = xa_pre[w];
            while (u) {
                const int bit = __builtin_ctz(u);
                uint32_t e = (uint32_t)(32 * w + bit);
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) e |= ((hw[hh] >> bit) & 1u) << (16 + hh);
                xa_list[o++] = e;
                u &= u - 1;
            }
        }
        __syncthreads();
        n_tiles = __builtin_amdgcn_readfirstlane(xa_pre[xa_nw]) << (rule.bk_log2 - 6);
    } else {
        int a_end, b_begin;
        kept_ranges(p0, p1, is_fa || p1 - 1 >= tail0, rule, a_end, b_begin);
        nA = (a_end + kBN - 1) / kBN;
        tB0 = max(nA, b_begin / kBN);
        const int tB1 = (p1 + kBN - 1) / kBN;
        n_tiles = nA + max(0, tB1 - tB0);
    }
    // XA: list entries xa_base .. xa_base+63 live in one VGPR, entry xa_base + l
    // in lane l, so a tile's entry is a lane read: no LDS round trip, and no LDS
    // wait, inside the tile pipeline.  xa_window(t0), at the top of each round
    // of phases (right after its barrier, when no LDS read is in flight), moves
    // the window, with one LDS read, when the entries of tiles t0 .. t0+2 (all
    // the round looks up) leave it: once per 62 blocks as the tiles ascend.
    // Tile indices are clamped to [0, n_tiles - 1], as every lookup is.
    uint32_t xa_win = 0u;
    int xa_base = 1 << 30;
    auto xa_window = [&](int t0) __attribute__((always_inline)) {
        const int sh = rule.bk_log2 - 6;  // kBN = 64 keys per tile
        const int lo = max(min(t0, n_tiles - 1), 0) >> sh;
        const int hi = max(min(t0 + 2, n_tiles - 1), 0) >> sh;
        if (lo < xa_base || hi >= xa_base + 64) {  // uniform
            xa_base = lo;
            xa_win = xa_list[min(lo + lane, 4095)];
        }
    };
    auto xa_entry = [&](int t) __attribute__((always_inline)) {
        const int e = max(t, 0) >> (rule.bk_log2 - 6);
        return (uint32_t)__builtin_amdgcn_readlane((int)xa_win, e - xa_base);
    };
    // first key of tile t; in mode XA from its list entry ent
    auto tile_k0e = [&](int t, uint32_t ent) __attribute__((always_inline)) {
        if constexpr (XA) {
            const int sh = rule.bk_log2 - 6;
            return ((int)(ent & 0xffffu) << rule.bk_log2) + ((t & ((1 << sh) - 1)) << 6);
        } else {
            return (t < nA ? t : tB0 + (t - nA)) * kBN;
        }
    };
    auto tile_k0 = [&](int t) __attribute__((always_inline)) {
        if constexpr (XA) return tile_k0e(t, xa_entry(t));
        else return tile_k0e(t, 0u);
    };
    if constexpr (XA) xa_window(0);

    const size_t row_stride = (size_t)hkv * D;
    const uint16_t *kb = k + ((size_t)start * hkv + kvh) * D;
    const uint16_t *vb = v + ((size_t)start * hkv + kvh) * D;
    TileLoader<D, false> lk;
    TileLoader<D, true> lv;
    lk.init(wq, lane, row_stride);
    lv.init(wq, lane, row_stride);
    // The first K tile is requested at once.  The V buffers are cleared once: a
    // copy past the sequence end may leave rows unwritten, and P = 0 times a
    // stale NaN pattern would still be NaN (the first MFMA block multiplies a zero
    // P with v_lds1).  K rows past the end need no clearing: their scores are
    // masked to -inf whatever they hold.  The clear is complete before the first
    // phase barrier (which waits for every wave's LDS accesses).
    if (grp == 0) {
        const __amdgpu_buffer_rsrc_t r0 = lk.rsrc(kb, row_stride, tile_k0(0), T);
#pragma unroll
        for (int i = 0; i < lk.NI; ++i) lk.issue_one(i, k_lds0, r0);
    }
    for (int i = tid; i < TILE_BYTES / 16; i += kThreads) {
        *(u32x4 *)(v_lds0 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
        *(u32x4 *)(v_lds1 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- Q^T operand in registers: B operand of the 16x16x32 products, lane l
    // holds row pw0 + 16 rg + l%16, d = 32 ks + 8 (l/16) .. +7
    const int c16 = lane & 15, g4 = lane >> 4;
    bf16x8 qreg[2][D / 32];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
        const int t = min(pw0 + 16 * rg + c16, T - 1);
        const uint16_t *qr = q + ((size_t)(start_q + t - q_off) * hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            qreg[rg][ks] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qr + ks * 32 + g4 * 8));
    }

    // masking thresholds for this wave and for the lane's two rows
    const int sink_tok = rule.ns << rule.bk_log2;
    const int win_lo_min = ((pw0 >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;
    const int win_lo_max = ((pw_last >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;
    int my_t[2], my_win_lo[2];
    bool my_dense[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
        my_t[rg] = min(pw0 + 16 * rg + c16, T - 1);
        my_win_lo[rg] = ((my_t[rg] >> rule.bk_log2) - rule.nw + 1) << rule.bk_log2;
        my_dense[rg] = is_fa || my_t[rg] >= tail0;
    }
    // does any row of this wave see a key of the tile at k0 (list entry ent)?
    auto wave_sees = [&](int k0, uint32_t ent) __attribute__((always_inline)) {
        if constexpr (XA) {  // this wave's head kept the tile's block
            return wave_active && k0 <= pw_last && ((ent >> (16 + wq / wph)) & 1u) != 0;
        } else {
            return wave_active && k0 <= pw_last &&
                   (w_dense_any || k0 < sink_tok || k0 + kBN > win_lo_min);
        }
    };

    // Per-lane LDS byte offsets, fixed for the whole kernel (the key group, the
    // d step and the k step only add constants):
    //   K operand (A of a 16x16x32 product) of key group kg, d step ks: key
    //   16 kg + l%16, logical chunk 4 ks + l/16, stored at chunk ^ swz_k(key),
    //   which depends on l%16 only.
    //   V^T operand of d group dg, k step ksv: the transposed read of lane
    //   (a = (l%16)/4, bq = l%4) points at key row 4 (l/16) + a (+32 per k step,
    //   +16 for the upper 4 keys), d columns 16 dg + 4 bq .. +3; the instruction
    //   hands lane l the 4 keys of its group at d = 16 dg + l%16.  The V swizzle
    //   depends on key row % 8, i.e. on l.
    uint32_t koff[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
        koff[ks] = (uint32_t)tile_off<D>(c16, ks * 4 + g4, swz_k<D>(c16));
    uint32_t voff[D / 16];
    {
        const int r0 = 4 * g4 + (c16 >> 2);
#pragma unroll
        for (int dg = 0; dg < D / 16; ++dg) {
            const int col = dg * 16 + 4 * (c16 & 3);
            voff[dg] = (uint32_t)(tile_off<D>(r0, col >> 3, swz_v<D>(r0)) + (col & 7) * 2);
        }
    }

    // O^T accumulators: oacc[dg][rg], lane l holds row 16 rg + l%16 at
    // d = 16 dg + 4 (l/16) .. +3.  Row statistics per lane and row group.
    f32x4 oacc[D / 16][2];
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) oacc[i][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};  // reference max, log2 domain
    float m_ref[2] = {0.0f, 0.0f};            // the reference the scores are shifted by
    float p_lim[2] = {-1.0f, -1.0f};          // fast-path bound on a lane's sum (-1: none yet)
    float l_run[2] = {0.0f, 0.0f};            // this lane's share of the row sum
    // S^T of the current tile: s[kg][rg], lane l holds row 16 rg + l%16 at keys
    // 16 kg + 4 (l/16) .. +3
    f32x4 s[4][2];
    uint32_t pk[2][2][4];     // P of the previous tile, bf16 pairs, [k step][rg] (0: none)
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int j = 0; j < 4; ++j) pk[a2][rg][j] = 0u;
    bool s_live = false;      // s holds a tile this wave sees
    int k0_live = 0;          // first key of the tile in s

    // ---- MFMA block of tile t: S^T = K Q^T of tile t, O^T += V^T P^T of tile t-1
    // P^T for k step ksv and row group rg is the lane's own S^T values of key
    // groups 2 ksv and 2 ksv + 1: k index 8 (l/16) + e <-> key
    // 32 ksv + 16 (e/4) + 4 (l/16) + e%4, the order the V^T reads follow.
    auto k_operand = [&](const char *k_lds, int ks, int kg) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, *(const u32x4 *)(k_lds + koff[ks] + kg * 16 * D * 2));
    };
    auto v_operand = [&](const char *v_lds, int ksv, int dg) __attribute__((always_inline)) {
        const char *plo = v_lds + voff[dg] + ksv * 32 * D * 2;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)plo);
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(plo + 16 * D * 2));
        u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        u32x4 aw = {lo2[0], lo2[1], hi2[0], hi2[1]};
        return __builtin_bit_cast(bf16x8, aw);
    };
    auto p_operand = [&](int ksv, int rg) __attribute__((always_inline)) {
        u32x4 pw = {pk[ksv][rg][0], pk[ksv][rg][1], pk[ksv][rg][2], pk[ksv][rg][3]};
        return __builtin_bit_cast(bf16x8, pw);
    };
    // Both products run as one pipeline of operand fragments: fragment f is a K
    // fragment (f even) or a V^T fragment (f odd), each read from LDS kLook
    // fragments ahead and used by the two products of its row groups;
    // scheduling barriers pin the order.  The block has no branches: a tile this
    // wave does not see still runs QK (the result is dropped) and its P is
    // zero, so PV adds exactly 0.
    //
    // When LD is set (group 0 at even phases 2j) the block also issues the
    // copies of K of tile j+1 and V of tile j, one every two fragments, so the
    // memory pipeline drains while the matrix cores work and group 1's softmax
    // is not interrupted.  Past the last tile the copies have an empty range
    // (their buffers are not read again).
    auto block_mfma = [&](auto ld_tag, const char *k_lds, const char *v_lds, int t, char *kdst,
                          char *vdst) __attribute__((always_inline)) {
        constexpr bool LD = decltype(ld_tag)::value != 0;
        constexpr int NKS = D / 32;        // d steps of QK
        constexpr int NKF = 4 * NKS;       // K fragments (4 key groups)
        constexpr int NDG = D / 16;        // d groups of PV
        constexpr int NVF = 2 * NDG;       // V^T fragments (2 k steps)
        static_assert(NKF == NVF, "K and V fragments interleave one to one");
        constexpr int NF = NKF + NVF;
        constexpr int kLook = 6;
        constexpr int NLD = lk.NI + lv.NI;
        static_assert(2 * NLD <= NF, "copies fit between the fragments");
        const int tc = min(t, n_tiles - 1);
        const uint32_t ent = XA ? xa_entry(tc) : 0u;
        const int k0_t = tile_k0e(tc, ent);
        k0_live = k0_t;
        s_live = t < n_tiles && wave_sees(k0_t, ent);
        __amdgpu_buffer_rsrc_t rk, rv;
        if constexpr (LD) {
            rk = lk.rsrc(kb, row_stride, tile_k0(min(t + 1, n_tiles - 1)), t + 1 < n_tiles ? T : 0);
            rv = lv.rsrc(vb, row_stride, k0_t, t < n_tiles ? T : 0);
        }
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) s[kg][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 ops[NF];
        // K fragment i: key group i / NKS, d step i % NKS (consecutive K
        // fragments extend one S chain); V^T fragment i: d group i % NDG, k step
        // i / NDG
        auto load_op = [&](int f) __attribute__((always_inline)) {
            const int i = f >> 1;
            if ((f & 1) == 0) ops[f] = k_operand(k_lds, i % NKS, i / NKS);
            else ops[f] = v_operand(v_lds, i / NDG, i % NDG);
        };
#pragma unroll
        for (int f = 0; f < kLook; ++f) load_op(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int i = f >> 1;
            if ((f & 1) == 0) {
                const int ks = i % NKS, kg = i / NKS;
#pragma unroll
                for (int rg = 0; rg < 2; ++rg) s[kg][rg] = mfma16(ops[f], qreg[rg][ks], s[kg][rg]);
            } else {
                const int dg = i % NDG, ksv = i / NDG;
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
                    oacc[dg][rg] = mfma16(ops[f], p_operand(ksv, rg), oacc[dg][rg]);
            }
            if (f + kLook < NF) load_op(f + kLook);
            if constexpr (LD) {
                if ((f & 1) == 1 && (f >> 1) < NLD) {
                    const int c = f >> 1;
                    if (c < lk.NI) lk.issue_one(c, kdst, rk);
                    else lv.issue_one(c - lk.NI, vdst, rv);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- VALU block of tile t: mask, online softmax, P = bf16(2^(s - m))
    auto block_valu = [&](int t) __attribute__((always_inline)) {
        if (!s_live) {
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                    for (int j = 0; j < 4; ++j) pk[a2][rg][j] = 0u;
            return;
        }
        const int k0 = k0_live;  // tile t's first key, from its MFMA block
        // mask (causal diagonal, window lower edge, sequence tail)
        const bool need_mask = (k0 + kBN - 1 > pw0) ||
                               (!w_dense_all && k0 < win_lo_max && k0 + kBN > sink_tok);
        if (need_mask) {
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = k0 + 16 * kg + 4 * g4 + j;
                        const bool vis = key <= my_t[rg] &&
                                         (my_dense[rg] || key < sink_tok || key >= my_win_lo[rg]);
                        if (!vis) s[kg][rg][j] = -INFINITY;
                    }
        }
        // online softmax (exp2 domain) against a lazily moved reference m_ref,
        // per row group: the fast path p = 2^(s scale - m_ref) holds while no
        // lane's partial row sum exceeds kFastLimit (which bounds every p it
        // holds) and every row has a reference; otherwise the tile max moves the
        // reference, O and l are rescaled and p is recomputed.  O / l does not
        // depend on the reference.
        const float m_use[2] = {m_ref[0], m_ref[1]};
#pragma unroll
        for (int kg = 0; kg < 4; ++kg)
#pragma unroll
            for (int rg = 0; rg < 2; ++rg)
#pragma unroll
                for (int j = 0; j < 4; ++j) s[kg][rg][j] = s[kg][rg][j] * scale_log2 - m_use[rg];
        __builtin_amdgcn_sched_barrier(0);
        float e[2][16];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
            for (int i = 0; i < 16; ++i) e[rg][i] = fast_exp2(s[i >> 2][rg][i & 3]);
        __builtin_amdgcn_sched_barrier(0);
        auto row_sum = [&](int rg) __attribute__((always_inline)) {
            float q1[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q1[i] = e[rg][2 * i] + e[rg][2 * i + 1];
#pragma unroll
            for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < w; ++i) q1[i] = q1[i] + q1[i + w];
            return q1[0];
        };
        float psum[2] = {row_sum(0), row_sum(1)};
        // NaN, or no reference yet: not fast
        const bool fast = psum[0] <= p_lim[0] && psum[1] <= p_lim[1];
        if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
                float m1[4];
#pragma unroll
                for (int kg = 0; kg < 4; ++kg)
                    m1[kg] = fmaxf(fmaxf(s[kg][rg][0], s[kg][rg][1]),
                                   fmaxf(s[kg][rg][2], s[kg][rg][3]));
                float mx = fmaxf(fmaxf(m1[0], m1[1]), fmaxf(m1[2], m1[3]));
                mx = row4_max(mx) + m_use[rg];   // tile max in the log2 domain
                const float m_new = fmaxf(m_run[rg], mx);
                const float alpha =
                    fast_exp2(m_run[rg] - (m_new == -INFINITY ? 0.0f : m_new));
                l_run[rg] *= alpha;
#pragma unroll
                for (int i = 0; i < D / 16; ++i) oacc[i][rg] *= alpha;
                m_run[rg] = m_new;
                m_ref[rg] = m_new == -INFINITY ? 0.0f : m_new;
                p_lim[rg] = m_new == -INFINITY ? -1.0f : kFastLimit;
                const float shift = m_use[rg] - m_ref[rg];
#pragma unroll
                for (int i = 0; i < 16; ++i) e[rg][i] = fast_exp2(s[i >> 2][rg][i & 3] + shift);
                psum[rg] = row_sum(rg);
            }
        }
        // P^T of k step a2, row group rg: key groups 2 a2 and 2 a2 + 1
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int rg = 0; rg < 2; ++rg) {
                const float *e0 = &e[rg][8 * a2];
                pk[a2][rg][0] = pack_bf16x2(e0[0], e0[1]);
                pk[a2][rg][1] = pack_bf16x2(e0[2], e0[3]);
                pk[a2][rg][2] = pack_bf16x2(e0[4], e0[5]);
                pk[a2][rg][3] = pack_bf16x2(e0[6], e0[7]);
            }
        l_run[0] += psum[0];
        l_run[1] += psum[1];
    };

    // ---- phases.  Even phase 2j: wait for this wave's copies, barrier, then
    // copy K of tile j+1 and V of tile j.  Odd phases: no barrier.
    // Phase barriers are bare s_barrier instructions (a memory clobber keeps the
    // compiler from moving LDS accesses across them): a workgroup fence would
    // also wait for copies that have two phases to land.  At even phases every
    // wave first waits for its own copies and LDS reads.
    auto sync_even = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    const int n_phases = 2 * n_tiles + 2;
    // Unrolled by 4 phases so every buffer choice is a compile-time constant;
    // tile 2m's K sits in k_lds0, tile 2m+1's in k_lds1, V likewise.
    auto run = [&](auto grp_tag) __attribute__((always_inline)) {
        constexpr int GRP = decltype(grp_tag)::value;
        for (int p = 0; p < n_phases; p += 4) {
            const int t0 = p >> 1;  // even tile index of this round
            sync_even();
            if constexpr (XA) xa_window(t0);
            if (GRP == 0) block_mfma(ic<1>{}, k_lds0, v_lds1, t0, k_lds1, v_lds0);
            else if (p > 0) block_valu(t0 - 1);
            if (p + 1 >= n_phases) break;
            if (GRP == 0) block_valu(t0);
            else block_mfma(ic<0>{}, k_lds0, v_lds1, t0, nullptr, nullptr);
            if (p + 2 >= n_phases) break;
            sync_even();
            if (GRP == 0) block_mfma(ic<1>{}, k_lds1, v_lds0, t0 + 1, k_lds0, v_lds1);
            else block_valu(t0);
            if (p + 3 >= n_phases) break;
            if (GRP == 0) block_valu(t0 + 1);
            else block_mfma(ic<0>{}, k_lds1, v_lds0, t0 + 1, nullptr, nullptr);
        }
    };
    // Use the scale once before the loop: its scalar load is then known to have
    // landed, so the LDS waits inside the loop count LDS reads only (a pending
    // scalar load forces a full lgkmcnt(0) wait before every MFMA block).
    asm volatile("" ::"s"(scale_log2));
    if (grp == 0) run(ic<0>{});
    else run(ic<1>{});
    // the last even phase issued copies nobody reads: let them land before the
    // workgroup (and its LDS) goes away
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if (!wave_active) return;
    // ---- epilogue: O = O^T / l, lse = (m + log2 l) ln 2, per row group
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
        const float l_tot = row4_sum(l_run[rg]);
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int t = pw0 + 16 * rg + c16;
        if (t < T) {
            const size_t row = (size_t)(start_q + t - q_off);
            uint16_t *orow = o + (row * hq + h) * D;
#pragma unroll
            for (int dg = 0; dg < D / 16; ++dg) {
                const f32x4 &a4 = oacc[dg][rg];
                u32x2 w = {pack_bf16x2(a4[0] * inv, a4[1] * inv),
                           pack_bf16x2(a4[2] * inv, a4[3] * inv)};
                *(u32x2 *)(orow + dg * 16 + 4 * g4) = w;
            }
            if (lse && g4 == 0) lse[row * hq + h] = (m_run[rg] + fast_log2(l_tot)) * kLn2;
        }
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
    const int32_t *__restrict__ cu_k, const uint8_t *__restrict__ route, int n_layers,
    int layer, int hq, int hkv, SparseRule rule, float scale_log2,
    const uint32_t *__restrict__ xa_mask, int xa_nqb, int xa_nw)
{
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    // query rows cu[b] .., keys cu_k[b] ..; query row r sits at position q_off + r
    const int start_q = cu[b];
    const int Tq = cu[b + 1] - start_q;
    const int start = cu_k[b];
    const int T = cu_k[b + 1] - start;
    const int q_off = T - Tq;
    const int r0 = blockIdx.x * 64;
    if (r0 >= Tq) return;
    if (q_off < 0) {  // more queries than keys: NaN rows, nothing read
        const int r = r0 + (int)threadIdx.x;
        if (r < Tq) {
            TE *orow = o + ((size_t)(start_q + r) * hq + h) * D;
            for (int c = 0; c < D; ++c) {
                if constexpr (sizeof(TE) == 2) ((uint16_t *)orow)[c] = 0x7fc0u;
                else ((float *)orow)[c] = __builtin_nanf("");
            }
            if (lse) lse[(size_t)(start_q + r) * hq + h] = __builtin_nanf("");
        }
        return;
    }
    const int p0 = q_off + r0;
    const int p1 = min(p0 + 64, T);
    const int t = min(p0 + (int)threadIdx.x, T - 1);
    const bool is_fa = MODE == kModeFA || MODE == kModeXA ? true
                       : MODE == kModeSA ? false
                                         : route[(size_t)b * n_layers + layer] != 0;
    const int G = hq / hkv;
    const int g = h / G;
    // XA: this row's kept-block words (query block t / B of head h)
    const uint32_t *xrow =
        MODE == kModeXA ? xa_mask + (((size_t)b * hq + h) * xa_nqb + (t >> rule.bk_log2)) * xa_nw
                        : nullptr;

    float qv[D], acc[D];
    const TE *qr = q + ((size_t)(start_q + t - q_off) * hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qv[c] = ld_elem<TE, D>(qr, c) * scale_log2;
        acc[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    // Triangle attention: rows at or past tail0 keep every key
    const int tail0 = is_fa ? 0 : dense_tail_start(T, rule);
    int a_end, b_begin;
    kept_ranges(p0, p1, is_fa || p1 - 1 >= tail0, rule, a_end, b_begin);
    for (int pass = 0; pass < 2; ++pass) {
        int s0 = pass == 0 ? 0 : b_begin;
        int s1 = pass == 0 ? a_end : p1;
        for (int s = s0; s < s1; ++s) {
            if (!visible(t, s, is_fa || t >= tail0, rule)) continue;
            if constexpr (MODE == kModeXA) {
                const int blk = s >> rule.bk_log2;
                if (((xrow[blk >> 5] >> (blk & 31)) & 1u) == 0) continue;
            }
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
    const size_t row = (size_t)(start_q + t - q_off);
    TE *orow = o + (row * hq + h) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        if constexpr (sizeof(TE) == 2)
            ((uint16_t *)orow)[c] = to_bf16(acc[c] * inv);
        else
            ((float *)orow)[c] = acc[c] * inv;
    }
    if (lse) lse[row * hq + h] = (m + fast_log2(l)) * kLn2;
}

template <typename TE, int D, int MODE>
hipError_t launch_generic(const PrefillArgs &a, hipStream_t stream, const SparseRule &r,
                          float scale_log2)
{
    dim3 grid((a.max_seqlen + 63) / 64, a.hq, a.batch);
    prefill_generic_kernel<TE, D, MODE><<<grid, 64, 0, stream>>>(
        (const TE *)a.q, (const TE *)a.k, (const TE *)a.v, (TE *)a.o, a.lse, a.cu_seqlens,
        a.cu_seqlens_k, a.route, a.n_layers, a.layer, a.hq, a.hkv, r, scale_log2, a.xa_mask,
        a.xa_nqb, a.xa_nw);
    return hipGetLastError();
}

// Query heads per workgroup: 4 (each K/V tile then serves 4 heads) unless the
// model has fewer per KV head.  Mode XA needs the workgroup's 256 / hpw
// positions inside one block, and walks the union of its heads' kept blocks:
// it takes the fewest heads that fit (2 at block 128), so that union is over
// fewer heads; 0 when none fits.
int mfma_hpw(int G, int mode, int block)
{
    const int h = G >= 4 ? 4 : G;
    if (mode != kModeXA) return h;
    const int need = block >= 256 ? 1 : 256 / block;
    return need <= h ? need : 0;
}

template <int D, int MODE>
hipError_t launch_mfma(const PrefillArgs &a, hipStream_t stream, const SparseRule &r,
                       float scale_log2)
{
    const int G = a.hq / a.hkv;
    const int hpw = mfma_hpw(G, MODE, 1 << a.bk_log2);
    const int n_hgroups = G / hpw;
    const int bm_pos = 2 * 32 * (4 / hpw);  // two groups of 4 waves x 32 rows
    const int n_ptiles = (a.max_seqlen + bm_pos - 1) / bm_pos;
    const int n_units = a.batch * a.hkv;
    const long long n_wg = (long long)n_ptiles * n_hgroups * n_units;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    prefill_bf16_kernel<D, MODE><<<(unsigned)n_wg, kThreads, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v, (uint16_t *)a.o,
        a.lse, a.cu_seqlens, a.cu_seqlens_k, a.route, a.n_layers, a.layer, a.hq, a.hkv, G, hpw,
        n_hgroups, n_units, n_ptiles, r, scale_log2, a.xa_mask, a.xa_nqb, a.xa_nw);
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
    const bool fits = mfma_hpw(G, MODE, 1 << a.bk_log2) != 0;
    if (a.bf16 && prefill_mfma_supported(a.d, G) && fits) {
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
    SparseRule r{a.ns, a.nw, a.bk_log2, a.nl};
    const float scale_log2 = a.sm_scale * kLog2e;
    switch (a.mode) {
    case kModeFA: return launch_mode<kModeFA>(a, stream, r, scale_log2);
    case kModeSA: return launch_mode<kModeSA>(a, stream, r, scale_log2);
    case kModeXA: return launch_mode<kModeXA>(a, stream, r, scale_log2);
    default: return launch_mode<kModeMixed>(a, stream, r, scale_log2);
    }
}

}  // namespace fa
