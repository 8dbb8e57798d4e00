// router.hip -- Layer Router and streaming block plan kernels (gfx950).
//
// Layer Router [HF model card, summary paragraph; thelatestinai paper page,
// Figure 2]: the query hidden states x_Q of each sequence are mean-pooled over
// the sequence suffix (the pooling budget of [thelatestinai paper page,
// Figure 8]), passed through a two-layer fp32 MLP and thresholded at zero into
// one FA (1) / SA (0) bit per layer; decode reuses the bits [thelatestinai
// paper page, Table 3].
//
// Three launches, all with fixed reduction orders (no atomics), so the route
// bits are reproducible bit for bit:
//   1. pool:  one thread per hidden column, ascending-t fp32 sum / P;
//   2. gemv1: one wavefront per router-hidden row, all sequences; float4
//             strided partial sums then a fixed DPP/swizzle/permlane tree;
//   3. gemv2: one wavefront per (sequence, layer), same tree, then the
//             threshold.
// The router is latency-bound (W1 is 4 MiB at hidden 4096), so the work is
// spread over router_hidden wavefronts to read W1 with the whole chip.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

__device__ __forceinline__ float wave_sum(float x)
{
    x = group_sum<32>(x);
    return sum_xor32(x);
}

template <bool BF16>
__global__ __launch_bounds__(256) void router_pool_kernel(const void *__restrict__ x,
                                                          const int32_t *__restrict__ cu,
                                                          int hidden, int pool_tokens,
                                                          float *__restrict__ p)
{
    const int b = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= hidden) return;
    const int start = cu[b];
    const int T = cu[b + 1] - start;
    if (T <= 0) {
        p[(size_t)b * hidden + j] = __builtin_nanf("");
        return;
    }
    const int P = min(pool_tokens, T);
    float s = 0.0f;
    for (int t = T - P; t < T; ++t) {
        size_t idx = (size_t)(start + t) * hidden + j;
        float v;
        if constexpr (BF16)
            v = __uint_as_float((uint32_t)((const uint16_t *)x)[idx] << 16);
        else
            v = ((const float *)x)[idx];
        s += v;
    }
    p[(size_t)b * hidden + j] = s / (float)P;
}

// h[b][i] = ReLU(sum_j W1[i][j] p[b][j] + b1[i]); one wavefront per i.
__global__ __launch_bounds__(256) void router_gemv1_kernel(const float *__restrict__ w1,
                                                           const float *__restrict__ b1,
                                                           const float *__restrict__ p, int batch,
                                                           int hidden, int router_hidden,
                                                           float *__restrict__ h)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= router_hidden) return;
    const float *wr = w1 + (size_t)i * hidden;
    const bool vec = (hidden & 3) == 0;
    for (int b = 0; b < batch; ++b) {
        const float *pb = p + (size_t)b * hidden;
        float acc = 0.0f;
        if (vec) {
            for (int j = lane * 4; j < hidden; j += 256) {
                f32x4 w = *(const f32x4 *)(wr + j);
                f32x4 x = *(const f32x4 *)(pb + j);
                acc += w[0] * x[0];
                acc += w[1] * x[1];
                acc += w[2] * x[2];
                acc += w[3] * x[3];
            }
        } else {
            for (int j = lane; j < hidden; j += 64) acc += wr[j] * pb[j];
        }
        acc = wave_sum(acc) + b1[i];
        if (lane == 0) h[(size_t)b * router_hidden + i] = acc > 0.0f ? acc : 0.0f;
    }
}

// logit[b][l] = sum_i W2[l][i] h[b][i] + b2[l]; route = logit > 0.
// An empty sequence has no pooled vector: its logits are NaN and its bits SA.
__global__ __launch_bounds__(256) void router_gemv2_kernel(const float *__restrict__ w2,
                                                           const float *__restrict__ b2,
                                                           const float *__restrict__ h,
                                                           const int32_t *__restrict__ cu,
                                                           int batch, int router_hidden,
                                                           int n_layers,
                                                           uint8_t *__restrict__ route,
                                                           float *__restrict__ logits)
{
    const int lane = threadIdx.x & 63;
    const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= batch * n_layers) return;
    const int b = unit / n_layers, l = unit % n_layers;
    const float *wr = w2 + (size_t)l * router_hidden;
    const float *hb = h + (size_t)b * router_hidden;
    float acc = 0.0f;
    for (int i = lane; i < router_hidden; i += 64) acc += wr[i] * hb[i];
    acc = wave_sum(acc) + b2[l];
    if (cu[b + 1] - cu[b] <= 0) acc = __builtin_nanf("");
    if (lane == 0) {
        route[unit] = acc > 0.0f ? 1 : 0;  // NaN compares false -> SA
        if (logits) logits[unit] = acc;
    }
}

// plan[b][i] = (0, sink_end, win_begin, i + 1), or zeros past the sequence.
__global__ __launch_bounds__(256) void block_plan_kernel(const int32_t *__restrict__ cu, int batch,
                                                         int max_qblocks,
                                                         const uint8_t *__restrict__ route,
                                                         int n_layers, int layer, SparseRule r,
                                                         int32_t *__restrict__ plan)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int b = blockIdx.y;
    if (i >= max_qblocks) return;
    const int T = cu[b + 1] - cu[b];
    const int nqb = T > 0 ? ((T - 1) >> r.bk_log2) + 1 : 0;
    int4 e = make_int4(0, 0, 0, 0);
    if (i < nqb) {
        const bool is_fa = route[(size_t)b * n_layers + layer] != 0;
        int sink_end = i + 1, win_begin = i + 1;
        if (!is_fa) {
            sink_end = min(r.ns, i + 1);
            win_begin = max(sink_end, i - r.nw + 1);
        }
        e = make_int4(0, sink_end, win_begin, i + 1);
    }
    *(int4 *)(plan + ((size_t)b * max_qblocks + i) * 4) = e;
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, hipStream_t stream)
{
    dim3 g1((a.hidden + 255) / 256, a.batch);
    if (a.x_bf16)
        router_pool_kernel<true><<<g1, 256, 0, stream>>>(a.x_q, a.cu_seqlens, a.hidden,
                                                         a.pool_tokens, a.ws_pool);
    else
        router_pool_kernel<false><<<g1, 256, 0, stream>>>(a.x_q, a.cu_seqlens, a.hidden,
                                                          a.pool_tokens, a.ws_pool);
    router_gemv1_kernel<<<(a.router_hidden + 3) / 4, 256, 0, stream>>>(
        a.w1, a.b1, a.ws_pool, a.batch, a.hidden, a.router_hidden, a.ws_hidden);
    router_gemv2_kernel<<<(a.batch * a.n_layers + 3) / 4, 256, 0, stream>>>(
        a.w2, a.b2, a.ws_hidden, a.cu_seqlens, a.batch, a.router_hidden, a.n_layers, a.route,
        a.logits);
    return hipGetLastError();
}

hipError_t launch_block_plan(const PlanArgs &a, hipStream_t stream)
{
    SparseRule r{a.ns, a.nw, a.bk_log2, 0};
    dim3 g((a.max_qblocks + 255) / 256, a.batch);
    block_plan_kernel<<<g, 256, 0, stream>>>(a.cu_seqlens, a.batch, a.max_qblocks, a.route,
                                             a.n_layers, a.layer, r, a.plan);
    return hipGetLastError();
}

}  // namespace fa
