// xattn.hip -- the XAttention sparse branch (gfx950): antidiagonal block scores
// and threshold block selection.  The block-masked attention that follows runs
// in prefill.hip (mode XA).
//
// The pages name XAttention ("Block Sparse Attention with Antidiagonal
// Scoring", mlsanity reference list) as a block-level sparse operator with a
// block selection score for prefill [thelatestinai paper page, Table 3 and
// Table 12]; its steps are the published method's, read as:
//   reshaped rows: query row a stands for positions a*S + (S-1-s), key row b for
//   positions b*S + s (s = 0..S-1, positions past the sequence are zero);
//   A[a][b] = (sm_scale / S) sum_s <q[a*S+S-1-s], k[b*S+s]> -- the mean of the
//   S x S sub-block's antidiagonal -- for b <= a;  P = softmax_b(A[a][.]);
//   score[i][j] = sum of P over the 16 reshaped rows of query block i and the
//   16 reshaped columns of key block j (block size B = 16 S);
//   selection: block 0 and block i always, then blocks by decreasing score
//   (ties: smaller j) while the kept sum is below tau * sum_j score[i][j], with
//   every sum in fp32 in that order.
//
// Score kernel: one workgroup of 8 waves per (pair of query blocks 2m, 2m+1,
// 4 query heads of one KV head); wave w handles query block 2m + w/4 and head
// w%4.  Each wave keeps its head's 16 reshaped query rows in registers as the B
// operand of v_mfma_f32_16x16x32_bf16 (S*d / 32 k-steps); the key block --
// whose B rows are exactly the 16 reshaped key columns, S rows each -- is copied
// straight from global memory into LDS (buffer loads with an LDS destination,
// three buffers, two tiles ahead) once for all 8 waves and read as the A
// operand, 8 reads in flight ahead of the matrix core.  Two passes over the key
// blocks would redo every product; instead one pass keeps each reshaped row's
// running max and sum and stores the row's sum over every key block with the
// max it is relative to (a workspace of 8 bytes per row and cell), and a small
// kernel rescales those to the row's log-sum-exp and adds the 16 rows of each
// block.  Fixed reduction orders throughout.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kXaRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kXaLook = 8;                // LDS operand reads in flight
constexpr int kXaWaves = 8;


__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


template <int V>
using ic = std::integral_constant<int, V>;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// One 1 KiB copy from global memory into LDS: lane l moves the 16 bytes at
// byte offset voff of the buffer described by rsrc to LDS address lds + 16 l
// (a buffer load with an LDS destination, whose base sits in m0; reads past
// the buffer's range return zeros).  Written as inline assembly so the
// compiler places no waits for it: the kernel waits for its copies itself,
// with explicit vmcnt waits.  m0 has no other user in these kernels; the copy
// reads m0 one wait state after it is written (s_nop 0), as the hardware needs.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy_1k(uint32_t lds, uint32_t voff, i32x4 rsrc)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// raw buffer descriptor: base address, stride 0, num_records bytes
__device__ __forceinline__ i32x4 raw_rsrc(const void *base, int num_records)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
    r.z = num_records;
    r.w = kXaRsrcWord3;
    return r;
}

// s_waitcnt vmcnt(N) then s_barrier, through the builtins so the compiler's
// own wait placement knows which copies are done; the empty asm statements keep
// memory accesses from moving across.
template <int N>
__device__ __forceinline__ void vm_wait_barrier(ic<N>)
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 encoding: vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14; expcnt
    // (bits 6:4) and lgkmcnt (bits 11:8) at their no-wait maxima
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(imm);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D, int S>
__global__ __launch_bounds__(kXaWaves * 64) void xa_score_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const int32_t *__restrict__ cu,
    int hq, int hkv, int G, int hpw, int n_hgroups, int n_units, int npairs, int nqb,
    float scale_log2, float2 *__restrict__ part, float2 *__restrict__ rowstat)
{
    constexpr int B = kXaRows * S;   // positions per block
    constexpr int NK = S * D / 32;   // k-steps of one reshaped row
    constexpr int CH = D / 8;        // 16-byte chunks per key row
    constexpr int TILE = B * D * 2;  // bytes of one key block
    constexpr int NI = TILE / (1024 * kXaWaves);  // 1 KiB copies per wave per tile
    constexpr int NQ = D / 32;       // k-steps per key row
    constexpr int LK = NK > 2 * kXaLook ? kXaLook : NK / 2;  // reads in flight
    static_assert(NI >= 1 && NI * 1024 * kXaWaves == TILE, "tile split over the waves");
    __shared__ __attribute__((aligned(1024))) char lds0[TILE];
    __shared__ __attribute__((aligned(1024))) char lds1[TILE];
    __shared__ __attribute__((aligned(1024))) char lds2[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, wq = wave & 3;
    // unit (sequence, kv head), head group, block pair: as in the prefill
    // kernels, XCD x (blockIdx mod 8) walks the units 8u + x one at a time when
    // the unit count is a multiple of 8, so its CUs share one key stream in L2;
    // the heavy block pairs start first
    int unit, hg, pm;
    if (n_units % 8 == 0) {  // uniform
        const int m = blockIdx.x >> 3;
        const int per_unit = n_hgroups * npairs;
        const int u = m / per_unit, rem = m - u * per_unit;
        unit = 8 * u + (blockIdx.x & 7);
        hg = rem % n_hgroups;
        pm = npairs - 1 - rem / n_hgroups;
    } else {
        int bid = blockIdx.x;
        unit = bid % n_units;
        bid /= n_units;
        hg = bid % n_hgroups;
        pm = npairs - 1 - bid / n_hgroups;
    }
    const int b = unit / hkv, kvh = unit % hkv;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    // blocks at or past nqb (a sequence longer than the layout holds) are not computed
    const int nb = min((T + B - 1) / B, nqb);
    if (2 * pm >= nb) return;                 // uniform
    const int i = 2 * pm + grp;               // this wave's query block
    const int j_last = min(2 * pm + 1, nb - 1);  // last key block of the workgroup
    const int Tr = (T + S - 1) / S;           // reshaped rows of the sequence
    const bool active = wq < hpw && i < nb;
    const int h = kvh * G + hg * hpw + (wq < hpw ? wq : 0);
    const size_t row_stride = (size_t)hkv * D;
    const uint16_t *kb = k + ((size_t)start * hkv + kvh) * D;

    // Key block copies: LDS chunk p (16 bytes) of a tile holds key row r = p / CH,
    // logical chunk (p % CH) ^ ((r / S) mod CH), so that the 16 lanes of one
    // A-operand read (16 reshaped columns, key rows S apart) hit distinct banks.
    // Wave w copies LDS chunks (w NI + n) 64 + lane, n < NI.
    uint32_t goff[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int p = (wave * NI + n) * 64 + lane;
        const int r = p / CH;
        const int c = (p % CH) ^ ((r / S) & (CH - 1));
        goff[n] = (uint32_t)(r * row_stride * 2) + (uint32_t)(c << 4);
    }
    // Rows at or past the sequence end read as zero (buffer range check); a
    // tile past the workgroup's last key block is issued with an empty range, so
    // the copies are unconditional and every wave has NI of them per tile.
    auto issue_tile = [&](int jt, char *dst) __attribute__((always_inline)) {
        const long long bytes =
            jt <= j_last ? (long long)max(T - jt * B, 0) * (long long)row_stride * 2 : 0LL;
        const i32x4 rs =
            raw_rsrc(kb + (size_t)jt * B * row_stride, (int)min(bytes, 0x7fffffffLL));
        const uint32_t lds = (uint32_t)(uintptr_t)(lds_void *)dst + wave * NI * 1024;
#pragma unroll
        for (int n = 0; n < NI; ++n) lds_copy_1k(lds + n * 1024, goff[n], rs);
    };
    // Tile jt ready: this wave's copies of it are done (the NI copies of the next
    // tile, issued later, may still run; memory operations complete in order),
    // then every wave's.  The last block of a sequence may end inside the tile:
    // its rows past the end are cleared so they never hold an earlier tile's keys.
    auto tile_ready = [&](int jt, char *dst) __attribute__((always_inline)) {
        vm_wait_barrier(ic<NI>{});
        const int rows = T - jt * B;
        if (jt <= j_last && rows < B) {  // uniform
            for (int p = tid; p < TILE / 16; p += kXaWaves * 64)
                if (p / CH >= rows) *(u32x4 *)(dst + 16 * p) = u32x4{0u, 0u, 0u, 0u};
            __syncthreads();
        }
    };

    // B operand: lane l holds reshaped query row a = 16 i + l%16 at reshaped
    // k index kk*32 + 8*(l/16) .. +7, i.e. position a S + S-1-s, elements e .. e+7
    // with s = k / D, e = k % D.
    const int a_loc = lane & 15, kq = lane >> 4;
    const int a = i * kXaRows + a_loc;
    bf16x8 qr[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        const int kidx = kk * 32 + 8 * kq;
        const int s = kidx / D, e = kidx % D;
        const int pos = a * S + (S - 1 - s);
        u32x4 w = {0u, 0u, 0u, 0u};
        if (active && pos < T) w = *(const u32x4 *)(q + ((size_t)(start + pos) * hq + h) * D + e);
        qr[kk] = __builtin_bit_cast(bf16x8, w);
    }
    // consume the query loads here, before any tile copy is in flight, so the
    // waits the compiler places for them never cover a copy
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) asm volatile("" ::"v"(qr[kk]));

    // A operand: lane l holds reshaped key column cc = l%16 at k index
    // kk*32 + 8*(l/16): key row cc S + s, logical chunk e / 8 with s = kk*32 / D
    // and e / 8 = 4 (kk mod NQ) + l/16.  The swizzle depends on cc only, so the
    // per-lane offset takes NQ values and s adds a constant.
    uint32_t aoff[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m)
        aoff[m] = (uint32_t)(a_loc * S * D * 2) + (uint32_t)(((4 * m + kq) ^ (a_loc & (CH - 1))) << 4);
    auto block_product = [&](const char *t) __attribute__((always_inline)) {
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 ab[LK];
        auto rd = [&](int kk) __attribute__((always_inline)) {
            return __builtin_bit_cast(
                bf16x8, *(const u32x4 *)(t + aoff[kk % NQ] + (kk * 32 / D) * (D * 2)));
        };
        // reads issued in k order (LDS reads complete in issue order, so the
        // first MFMA waits for the first read only)
#pragma unroll
        for (int kk = 0; kk < LK; ++kk) {
            ab[kk] = rd(kk);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            acc[kk & 3] = mfma16(ab[kk % LK], qr[kk], acc[kk & 3]);
            if (kk + LK < NK) ab[kk % LK] = rd(kk + LK);
            __builtin_amdgcn_sched_barrier(0);
        }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    };

    // One pass.  Per reshaped row (held by lanes l, l^16, l^32, l^48): the
    // running max m and the sum l of 2^(A - m) over the blocks so far; after
    // block j the row's sum over that block, relative to the running max then,
    // goes to the workspace with that max.  The finishing kernel rescales to the
    // row's log-sum-exp and adds the 16 rows of each block.  A row's results of
    // block j are stored before the next tile copies are issued.
    float m_row = -INFINITY, l_row = 0.0f;
    float e_out = 0.0f, m_out = -INFINITY;  // the pending store
    int j_out = -1;
    const size_t ncell = (size_t)nqb * (nqb + 1) / 2;  // cells j <= i of one (b, h)
    float2 *pbase = part + (((size_t)b * hq + h) * ncell + (size_t)i * (i + 1) / 2) * kXaRows;
    auto flush = [&]() __attribute__((always_inline)) {
        if (j_out >= 0 && active && kq == 0)  // uniform but for kq: lanes 0..15, one row each
            pbase[(size_t)j_out * kXaRows + a_loc] = make_float2(e_out, m_out);
        j_out = -1;
    };
    // softmax update with key block j's products c; C lane layout: query row
    // a = 16 i + l%16, key columns 16 j + 4 (l/16) + jj
    auto soft = [&](int j, const f32x4 &c) __attribute__((always_inline)) {
        float v[4];
        bool ok[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int cb = j * kXaRows + 4 * kq + jj;
            ok[jj] = cb <= a && a < Tr;
            v[jj] = c[jj] * scale_log2;
        }
        float mb = fmaxf(fmaxf(ok[0] ? v[0] : -INFINITY, ok[1] ? v[1] : -INFINITY),
                         fmaxf(ok[2] ? v[2] : -INFINITY, ok[3] ? v[3] : -INFINITY));
        mb = row4_max(mb);
        const float m_new = fmaxf(m_row, mb);
        const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
        float e = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) e += ok[jj] ? fast_exp2(v[jj] - m_sub) : 0.0f;
        e = row4_sum(e);
        l_row = l_row * fast_exp2(m_row - m_sub) + e;
        m_row = m_new;
        e_out = e;
        m_out = m_new;
        j_out = j;
    };
    // one key block (tile in t)
    auto step = [&](int j, const char *t) __attribute__((always_inline)) {
        if (j <= i) soft(j, block_product(t));  // uniform: up to the causal edge
    };

    // resolve every scalar kernel argument the kernel still needs now, those
    // used after the loop too: a scalar load still in flight at the loop
    // header would turn the first LDS wait of every block into lgkmcnt(0)
    asm volatile("" ::"s"(pbase), "s"(scale_log2), "s"(rowstat));
    issue_tile(0, lds0);
    issue_tile(1, lds1);
    tile_ready(0, lds0);
    for (int j = 0; j <= j_last; j += 3) {
        flush();
        issue_tile(j + 2, lds2);
        step(j, lds0);
        tile_ready(j + 1, lds1);
        if (j + 1 > j_last) break;
        flush();
        issue_tile(j + 3, lds0);
        step(j + 1, lds1);
        tile_ready(j + 2, lds2);
        if (j + 2 > j_last) break;
        flush();
        issue_tile(j + 4, lds1);
        step(j + 2, lds2);
        tile_ready(j + 3, lds0);
    }
    flush();
    // the row's max and sum (2^lse = l 2^m); rows past the sequence end have l = 0
    if (active && kq == 0)
        rowstat[(((size_t)b * hq + h) * nqb + i) * kXaRows + a_loc] = make_float2(m_row, l_row);
    // drain the copies of tiles past the end before the workgroup leaves
    vm_wait_barrier(ic<0>{});
}

// fp32 inputs: the same partials from a plain VALU kernel.  One workgroup per
// (query block i, head, sequence); thread (r, c) = (tid / 16, tid % 16) forms
// A[16 i + r][16 j + c] for every key block j <= i as one fp32 dot product over
// the S*d reshaped k-values (k index s*d + e), its query row staged in LDS.  The
// 16 threads of a row then take the same online update as the MFMA kernel
// (sum and max over the row's 16 columns in a fixed DPP order) and store the
// row's (sum, max) of block j; the finishing kernel is shared.
template <int D, int S>
__global__ __launch_bounds__(256) void xa_score_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const int32_t *__restrict__ cu,
    int hq, int hkv, int nqb, float scale_log2, float2 *__restrict__ part,
    float2 *__restrict__ rowstat)
{
    constexpr int RK = S * D;  // reshaped k-values per row
    __shared__ __attribute__((aligned(16))) float qs[kXaRows][RK];
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int r = tid >> 4, c = tid & 15;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    const int nb = T > 0 ? min((T + kXaRows * S - 1) / (kXaRows * S), nqb) : 0;
    if (i >= nb) return;  // uniform
    const int Tr = (T + S - 1) / S;
    const int kvh = h / (hq / hkv);
    // query rows of block i: reshaped row a = 16 i + rr, k index s*D + e holds
    // position a*S + S-1-s (zero past the sequence)
    for (int idx = tid; idx < kXaRows * RK / 4; idx += 256) {
        const int rr = idx / (RK / 4), kk = (idx % (RK / 4)) * 4;
        const int s = kk / D, e = kk % D;
        const int pos = (i * kXaRows + rr) * S + (S - 1 - s);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (pos < T) v = *(const float4 *)(q + ((size_t)(start + pos) * hq + h) * D + e);
        *(float4 *)&qs[rr][kk] = v;
    }
    __syncthreads();
    const int a = i * kXaRows + r;
    const size_t ncell = (size_t)nqb * (nqb + 1) / 2;
    float2 *pbase = part + (((size_t)b * hq + h) * ncell + (size_t)i * (i + 1) / 2) * kXaRows;
    float m_row = -INFINITY, l_row = 0.0f;
    for (int j = 0; j <= i; ++j) {  // uniform
        const int bc = j * kXaRows + c;  // this thread's reshaped key column
        float acc = 0.0f;
        for (int s = 0; s < S; ++s) {
            const int pos = bc * S + s;
            if (pos >= T) break;  // zero rows past the sequence
            const float *kr = k + ((size_t)(start + pos) * hkv + kvh) * D;
#pragma unroll 4
            for (int e = 0; e < D; e += 4) {
                const float4 kv = *(const float4 *)(kr + e);
                const float4 qv = *(const float4 *)&qs[r][s * D + e];
                acc = __builtin_fmaf(qv.x, kv.x, acc);
                acc = __builtin_fmaf(qv.y, kv.y, acc);
                acc = __builtin_fmaf(qv.z, kv.z, acc);
                acc = __builtin_fmaf(qv.w, kv.w, acc);
            }
        }
        const bool ok = bc <= a && a < Tr;
        const float v = acc * scale_log2;
        const float mb = group_max<16>(ok ? v : -INFINITY);
        const float m_new = fmaxf(m_row, mb);
        const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
        const float e = group_sum<16>(ok ? fast_exp2(v - m_sub) : 0.0f);
        l_row = l_row * fast_exp2(m_row - m_sub) + e;
        m_row = m_new;
        if (c == 0) pbase[(size_t)j * kXaRows + r] = make_float2(e, m_new);
    }
    if (c == 0)
        rowstat[(((size_t)b * hq + h) * nqb + i) * kXaRows + r] = make_float2(m_row, l_row);
}

// Block scores from the row partials: score[i][j] = sum over the 16 rows r of
// block i of e_rj 2^(m_rj - M_r) / l_r, rows with l_r = 0 (past the sequence
// end) left out.  One workgroup per (query block i, head, sequence); 8 lanes
// per cell j, lane q reading rows 2q and 2q+1 (16 bytes, so a wave reads 1 KiB
// in one coalesced load), summed over the 8 lanes in a fixed DPP order.
__global__ __launch_bounds__(256) void xa_score_finish_kernel(
    const float2 *__restrict__ part, const float2 *__restrict__ rowstat,
    const int32_t *__restrict__ cu, int hq, int nqb, int block, float *__restrict__ scores)
{
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int T = cu[b + 1] - cu[b];
    const int nb = T > 0 ? min((T + block - 1) / block, nqb) : 0;
    if (i >= nb) return;
    __shared__ float2 st[kXaRows];  // (M_r, 1 / l_r), 1 / l_r = 0 marking an empty row
    if (tid < kXaRows) {
        const float2 ml = rowstat[(((size_t)b * hq + h) * nqb + i) * kXaRows + tid];
        st[tid] = make_float2(ml.x, ml.y > 0.0f ? 1.0f / ml.y : 0.0f);
    }
    __syncthreads();
    const int q = tid & 7;
    const float2 s0 = st[2 * q], s1 = st[2 * q + 1];
    const size_t ncell = (size_t)nqb * (nqb + 1) / 2;
    const float4 *pb = (const float4 *)(part + (((size_t)b * hq + h) * ncell +
                                                (size_t)i * (i + 1) / 2) * kXaRows);
    float *srow = scores + (((size_t)b * hq + h) * nqb + i) * nqb;
    for (int j0 = 0; j0 <= i; j0 += 32) {  // uniform: every lane joins the DPP sum
        const int j = j0 + (tid >> 3);
        float t = 0.0f;
        if (j <= i) {
            const float4 em = pb[(size_t)j * (kXaRows / 2) + q];
            const float t0 = s0.y > 0.0f ? em.x * fast_exp2(em.y - s0.x) * s0.y : 0.0f;
            const float t1 = s1.y > 0.0f ? em.z * fast_exp2(em.w - s1.x) * s1.y : 0.0f;
            t = t0 + t1;
        }
        t = group_sum<8>(t);
        if (q == 0 && j <= i) srow[j] = t;
    }
}

// One workgroup per (query block i, head h, sequence b): the kept-block bits.
// LDS of the selection kernel, sized per launch for Pm = max(16, the power of
// two >= n_qblocks) so that more workgroups share a CU when rows are short:
// key_s [Pm + 16] and row_s [Pm + 16] floats (16 entries of padding: the
// decision loads 16 values at a time), key_j [Pm], bits [nw], the cut.
__host__ __device__ inline size_t xa_select_lds_bytes(int pm, int nw)
{
    return (size_t)4 * (2 * (pm + 16) + pm + nw + 1);
}

__global__ __launch_bounds__(256) void xa_select_kernel(const float *__restrict__ scores,
                                                        const int32_t *__restrict__ cu, int hq,
                                                        int nqb, int nw, int pm, int block,
                                                        float tau, uint32_t *__restrict__ mask)
{
    extern __shared__ __attribute__((aligned(16))) float xa_sel_lds[];
    float *key_s = xa_sel_lds;
    float *row_s = key_s + pm + 16;  // 16-byte aligned: pm is a multiple of 16
    int *key_j = (int *)(row_s + pm + 16);
    uint32_t *bits = (uint32_t *)(key_j + pm);
    int &s_cut = *(int *)(bits + nw);
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int T = cu[b + 1] - cu[b];
    const int nb = T > 0 ? min((T + block - 1) / block, nqb) : 0;
    uint32_t *mrow = mask + (((size_t)b * hq + h) * nqb + i) * nw;
    for (int w = tid; w < nw; w += 256) bits[w] = 0u;
    if (i >= nb) {
        for (int w = tid; w < nw; w += 256) mrow[w] = 0u;
        return;
    }
    const float *row = scores + (((size_t)b * hq + h) * nqb + i) * nqb;
    // candidates 1 .. i-1, padded to a power of two with entries that sort last
    const int n = i > 1 ? i - 1 : 0;
    int P = 1;
    while (P < n) P <<= 1;
    for (int j = tid; j <= i; j += 256) row_s[j] = row[j];
    for (int t = tid; t < P; t += 256) {
        key_s[t] = t < n ? row[t + 1] : -INFINITY;
        key_j[t] = t < n ? t + 1 : 0x7fffffff;
    }
    __syncthreads();
    // bitonic sort into the order (score descending, block ascending)
    for (int kk = 2; kk <= P; kk <<= 1)
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int t = tid; t < P; t += 256) {
                const int u = t ^ jj;
                if (u > t) {
                    const float st = key_s[t], su = key_s[u];
                    const int jt = key_j[t], ju = key_j[u];
                    const bool t_first = st > su || (st == su && jt < ju);
                    const bool want_t_first = (t & kk) == 0;
                    if (t_first != want_t_first) {
                        key_s[t] = su;
                        key_s[u] = st;
                        key_j[t] = ju;
                        key_j[u] = jt;
                    }
                }
            }
            __syncthreads();
        }
    // The decision, on one lane: every sum is fp32, one add at a time in the
    // stated order; the LDS loads fetch 16 values (4 x 16 bytes) ahead of the
    // adds.  A chunk starts at a multiple of 16 below Pm (t0 <= i < n_qblocks,
    // t0 < n <= Pm), so it stays in the padded arrays; values past the row are
    // loaded but never added.
    if (tid == 0) {
        auto chunk = [&](const float *a, int t0, float (&x)[16]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 v = *(const float4 *)(a + t0 + 4 * u);
                x[4 * u] = v.x;
                x[4 * u + 1] = v.y;
                x[4 * u + 2] = v.z;
                x[4 * u + 3] = v.w;
            }
        };
        float x[16];
        float total = 0.0f;
        for (int t0 = 0; t0 <= i; t0 += 16) {
            chunk(row_s, t0, x);
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (t0 + u <= i) total = total + x[u];
        }
        const float goal = tau * total;
        float kept = row_s[0];
        if (i > 0) kept = kept + row_s[i];
        // candidates in sorted order join while the kept sum is below the goal
        int cut = 0;
        bool stop = false;
        for (int t0 = 0; t0 < n && !stop; t0 += 16) {
            chunk(key_s, t0, x);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (stop || t0 + u >= n) break;
                if (!(kept < goal)) {
                    stop = true;
                    break;
                }
                kept = kept + x[u];
                cut = t0 + u + 1;
            }
        }
        s_cut = cut;
        bits[0] |= 1u;
        bits[i >> 5] |= 1u << (i & 31);
    }
    __syncthreads();
    const int cut = s_cut;
    for (int t = tid; t < cut; t += 256) {
        const int j = key_j[t];
        atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    for (int w = tid; w < nw; w += 256) mrow[w] = bits[w];
}

template <int D, int S>
hipError_t launch_scores_t(const XaScoreArgs &a, hipStream_t stream)
{
    const int G = a.hq / a.hkv;
    const int hpw = G >= 4 ? 4 : G;
    const int n_hgroups = G / hpw;
    const int n_units = a.batch * a.hkv;
    const int npairs = (a.nqb + 1) / 2;
    const long long n_wg = (long long)npairs * n_hgroups * n_units;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    float2 *part = (float2 *)a.workspace;
    float2 *rowstat = part + xa_part_entries(a.batch, a.hq, a.nqb);
    xa_score_kernel<D, S><<<(unsigned)n_wg, kXaWaves * 64, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, a.cu_seqlens, a.hq, a.hkv, G, hpw,
        n_hgroups, n_units, npairs, a.nqb, a.sm_scale / S * kLog2e, part, rowstat);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(a.nqb, a.hq, a.batch);
    xa_score_finish_kernel<<<grid, 256, 0, stream>>>(part, rowstat, a.cu_seqlens, a.hq, a.nqb,
                                                     kXaRows * S, a.scores);
    return hipGetLastError();
}

template <int D, int S>
hipError_t launch_scores_f32_t(const XaScoreArgs &a, hipStream_t stream)
{
    float2 *part = (float2 *)a.workspace;
    float2 *rowstat = part + xa_part_entries(a.batch, a.hq, a.nqb);
    dim3 grid(a.nqb, a.hq, a.batch);
    xa_score_f32_kernel<D, S><<<grid, 256, 0, stream>>>(
        (const float *)a.q, (const float *)a.k, a.cu_seqlens, a.hq, a.hkv, a.nqb,
        a.sm_scale / S * kLog2e, part, rowstat);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    xa_score_finish_kernel<<<grid, 256, 0, stream>>>(part, rowstat, a.cu_seqlens, a.hq, a.nqb,
                                                     kXaRows * S, a.scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_xa_scores(const XaScoreArgs &a, hipStream_t stream)
{
    if (!a.bf16) {
        if (a.d == 128) return a.stride == 8 ? launch_scores_f32_t<128, 8>(a, stream)
                                             : launch_scores_f32_t<128, 4>(a, stream);
        return a.stride == 8 ? launch_scores_f32_t<64, 8>(a, stream)
                             : launch_scores_f32_t<64, 4>(a, stream);
    }
    if (a.d == 128) return a.stride == 8 ? launch_scores_t<128, 8>(a, stream)
                                         : launch_scores_t<128, 4>(a, stream);
    return a.stride == 8 ? launch_scores_t<64, 8>(a, stream) : launch_scores_t<64, 4>(a, stream);
}

hipError_t launch_xa_select(const XaSelectArgs &a, hipStream_t stream)
{
    dim3 grid(a.nqb, a.hq, a.batch);
    int pm = 16;
    while (pm < a.nqb) pm <<= 1;
    xa_select_kernel<<<grid, 256, xa_select_lds_bytes(pm, a.nw), stream>>>(
        a.scores, a.cu_seqlens, a.hq, a.nqb, a.nw, pm, a.block, a.threshold, a.mask);
    return hipGetLastError();
}

}  // namespace fa
