// xattn.hip -- the XAttention sparse branch (gfx950): antidiagonal block scores
// and threshold block selection.  The block-masked attention that follows runs
// in prefill.hip (mode XA).
//
// The pages name XAttention ("Block Sparse Attention with Antidiagonal
// Scoring", mlsanity reference list) as a block-level sparse operator with a
// block selection score for prefill [thelatestinai paper page, Table 4 and
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
// Score kernel: one workgroup per (query block, 4 query heads of one KV head).
// Each wave keeps its head's 16 reshaped query rows in registers as the B
// operand of v_mfma_f32_16x16x32_bf16 (S*d / 32 k-steps); the key block --
// whose B rows are exactly the 16 reshaped key columns, S rows each -- is staged
// in LDS once for the 4 heads and read as the A operand.  Two passes over the
// key blocks: the first finds every reshaped row's log-sum-exp, the second
// sums 2^(A - lse) per key block.  No workspace; fixed reduction orders.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kXaRows = 16;  // reshaped rows (and columns) per block: B = 16 S
constexpr int kXaMaxBlocks = 4096;

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// reductions over the 4 lanes l, l^16, l^32, l^48 that hold one reshaped row
__device__ __forceinline__ float row4_sum(float x)
{
    x += xor16(x);
    return sum_xor32(x);
}
__device__ __forceinline__ float row4_max(float x)
{
    x = fmaxf(x, xor16(x));
    return max_xor32(x);
}

template <int D, int S>
__global__ __launch_bounds__(256) void xa_score_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const int32_t *__restrict__ cu,
    int hq, int hkv, int G, int hpw, int n_hgroups, int n_units, int nqb, float scale_log2,
    float *__restrict__ scores)
{
    constexpr int B = kXaRows * S;   // positions per block
    constexpr int NK = S * D / 32;   // k-steps of one reshaped row
    constexpr int CH = D / 8;        // 16-byte chunks per key row
    constexpr int TILE = B * D * 2;  // bytes of one key block
    constexpr int NCH = B * CH / 256;
    static_assert(NCH * 256 == B * CH, "tile split over 256 threads");
    __shared__ __attribute__((aligned(1024))) char lds[2][TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = blockIdx.x;
    const int unit = bid % n_units;
    bid /= n_units;
    const int hg = bid % n_hgroups;
    const int i = nqb - 1 - bid / n_hgroups;  // query block; the heavy ones start first
    const int b = unit / hkv, kvh = unit % hkv;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    const int nb = (T + B - 1) / B;
    if (i >= nb) return;                      // uniform
    const int Tr = (T + S - 1) / S;           // reshaped rows of the sequence
    const bool active = wave < hpw;
    const int h = kvh * G + hg * hpw + (active ? wave : 0);
    const size_t row_stride = (size_t)hkv * D;
    const uint16_t *kb = k + ((size_t)start * hkv + kvh) * D;

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

    // Key block j into LDS: chunk p = tid + 256 n is row r = p / CH, chunk c = p % CH
    // of the block, stored at chunk c ^ ((r / S) mod CH) so the 16 lanes of an
    // A-operand read (16 reshaped columns, rows S apart) hit distinct banks.
    u32x4 stage[NCH];
    auto load_tile = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NCH; ++n) {
            const int p = tid + 256 * n;
            const int r = p / CH, c = p % CH;
            const int pos = j * B + r;
            stage[n] = pos < T ? *(const u32x4 *)(kb + (size_t)pos * row_stride + c * 8)
                               : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NCH; ++n) {
            const int p = tid + 256 * n;
            const int r = p / CH, c = p % CH;
            *(u32x4 *)(lds[buf] + r * (D * 2) + ((c ^ ((r / S) & (CH - 1))) << 4)) = stage[n];
        }
    };
    // A operand: lane l holds reshaped key column cc = l%16 at k index
    // kk*32 + 8*(l/16): key row cc S + s, chunk e / 8 (s = k / D, e = k % D)
    auto block_product = [&](const char *t) __attribute__((always_inline)) {
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const int kidx = kk * 32 + 8 * kq;
            const int s = kidx / D, e = kidx % D;
            const int r = a_loc * S + s;
            const bf16x8 av = __builtin_bit_cast(
                bf16x8, *(const u32x4 *)(t + r * (D * 2) + (((e >> 3) ^ (a_loc & (CH - 1))) << 4)));
            acc[kk & 3] = mfma16(av, qr[kk], acc[kk & 3]);
        }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    };

    // pass 0: per-lane running max / sum (log2 domain) over the lane's values;
    // pass 1: per key block, sum of 2^(A - lse) over the 16 x 16 tile
    float m_l = -INFINITY, l_l = 0.0f, lse_row = 0.0f;
    float *srow = scores + (((size_t)b * hq + h) * nqb + i) * nqb;
    for (int pass = 0; pass < 2; ++pass) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int j = 0; j <= i; ++j) {
            if (j < i) load_tile(j + 1);
            const f32x4 c = block_product(lds[j & 1]);
            // C lane layout: query row a = 16 i + l%16, key columns 16 j + 4 (l/16) + jj
            float e_sum = 0.0f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int cb = j * kXaRows + 4 * kq + jj;
                const bool ok = cb <= a && a < Tr;
                const float v = c[jj] * scale_log2;
                if (pass == 0) {
                    if (ok) {
                        const float m_new = fmaxf(m_l, v);
                        l_l = l_l * fast_exp2(m_l - m_new) + fast_exp2(v - m_new);
                        m_l = m_new;
                    }
                } else if (ok) {
                    e_sum += fast_exp2(v - lse_row);
                }
            }
            if (pass == 1) {
                e_sum = group_sum<32>(e_sum);
                e_sum = sum_xor32(e_sum);
                if (active && lane == 0) srow[j] = e_sum;
            }
            if (j < i) store_tile((j + 1) & 1);
            __syncthreads();
        }
        if (pass == 0) {
            const float M = row4_max(m_l);
            const float L = row4_sum(m_l == -INFINITY ? 0.0f : l_l * fast_exp2(m_l - M));
            lse_row = M + fast_log2(L);
        }
    }
}

// One workgroup per (query block i, head h, sequence b): the kept-block bits.
__global__ __launch_bounds__(256) void xa_select_kernel(const float *__restrict__ scores,
                                                        const int32_t *__restrict__ cu, int hq,
                                                        int nqb, int nw, int block, float tau,
                                                        uint32_t *__restrict__ mask)
{
    __shared__ float key_s[kXaMaxBlocks];
    __shared__ int key_j[kXaMaxBlocks];
    __shared__ float row_s[kXaMaxBlocks];
    __shared__ uint32_t bits[kXaMaxBlocks / 32];
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int T = cu[b + 1] - cu[b];
    const int nb = T > 0 ? (T + block - 1) / block : 0;
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
    if (tid == 0) {
        float total = 0.0f;
        for (int j = 0; j <= i; ++j) total = total + row_s[j];
        const float goal = tau * total;
        bits[0] |= 1u;
        bits[i >> 5] |= 1u << (i & 31);
        float kept = row_s[0];
        if (i > 0) kept = kept + row_s[i];
        for (int t = 0; t < n; ++t) {
            if (!(kept < goal)) break;
            const int j = key_j[t];
            bits[j >> 5] |= 1u << (j & 31);
            kept = kept + key_s[t];
        }
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
    const long long n_wg = (long long)a.nqb * n_hgroups * n_units;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    xa_score_kernel<D, S><<<(unsigned)n_wg, 256, 0, stream>>>(
        (const uint16_t *)a.q, (const uint16_t *)a.k, a.cu_seqlens, a.hq, a.hkv, G, hpw,
        n_hgroups, n_units, a.nqb, a.sm_scale / S * kLog2e, a.scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_xa_scores(const XaScoreArgs &a, hipStream_t stream)
{
    if (a.d == 128) return a.stride == 8 ? launch_scores_t<128, 8>(a, stream)
                                         : launch_scores_t<128, 4>(a, stream);
    return a.stride == 8 ? launch_scores_t<64, 8>(a, stream) : launch_scores_t<64, 4>(a, stream);
}

hipError_t launch_xa_select(const XaSelectArgs &a, hipStream_t stream)
{
    dim3 grid(a.nqb, a.hq, a.batch);
    xa_select_kernel<<<grid, 256, 0, stream>>>(a.scores, a.cu_seqlens, a.hq, a.nqb, a.nw,
                                               a.block, a.threshold, a.mask);
    return hipGetLastError();
}

}  // namespace fa
