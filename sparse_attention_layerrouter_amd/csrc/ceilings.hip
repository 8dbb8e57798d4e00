// Ceiling kernels: what plain instruction streams reach on this board, as the
// measured context of the attention kernels' roofline fractions.
//
// These are measuring instruments, not part of the attention path: they are
// built into their own library (libfa_ceilings.so) and only the benchmark and
// its tests call them.
//
//  * fa_ceiling_read streams a device buffer: each 256-thread workgroup reads
//    one contiguous chunk with 16-byte non-temporal loads, eight in flight per
//    lane (the access pattern of the decode kernels' K/V reads).  Its rate is
//    what a plain read of that many bytes reaches, against the 8 TB/s HBM peak.
//  * fa_ceiling_mix issues 32x32x16 (or 16x16x32) bf16 matrix products from 8
//    waves per CU (two per SIMD, one workgroup per CU, like the prefill and
//    XAttention score kernels), with a
//    chosen number of 1 KiB LDS operand reads per product and, optionally, an
//    online-softmax-like VALU mix per product: one exponential, one FMA, one
//    add and half of a bf16 pair pack with its consumer.  The board runs such
//    work at a power-limited clock, so the matrix cores' rate depends on what
//    else the CU issues; this stream has no dependences between the three
//    kinds of work, no barriers and no global traffic, so it is the rate that
//    a kernel with the same mix can reach at best.
//  * fa_ceiling_valu times VALU issue alone: each lane runs 8 independent
//    chains of FMAs, of exponentials (v_exp_f32), or of both interleaved, and
//    each wave writes its loop's shader-clock ticks (s_memtime) and realtime
//    ticks (s_memrealtime, 100 MHz): with the workgroup size and count chosen
//    for 1, 2 or 8 waves per SIMD, the ticks per wave instruction on a SIMD and
//    the clock the loop ran at.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <type_traits>

extern "C" {
const char *fa_ceiling_last_error(void);
int fa_ceiling_read(const void *buf, size_t bytes, size_t chunk, uint32_t *sink,
                    hipStream_t stream);
int fa_ceiling_mix(int reads_per_8, int softmax, int shape, int n_workgroups, int iterations,
                   const void *seed, float *out, hipStream_t stream);
int fa_ceiling_valu(int kind, int n_workgroups, int threads, int iterations, float *out,
                    unsigned long long *cycles, hipStream_t stream);
}

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

thread_local char g_err[256] = "";

int fail(int code, const char *msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return code;
}

constexpr int kReadThreads = 256;
constexpr int kReadInFlight = 8;
constexpr size_t kReadGranule = (size_t)16 * kReadThreads * kReadInFlight;  // 32 KiB

// One workgroup per chunk of chunk16 16-byte words; chunk16 is a multiple of
// kReadThreads * kReadInFlight, so every load is inside the workgroup's chunk.
// Each thread writes the XOR of the 32-bit words it read, so the loads are
// kept and the XOR of all sink words is the XOR of the whole buffer.
__global__ __launch_bounds__(kReadThreads) void ceiling_read_kernel(
    const u32x4 *__restrict__ p, size_t chunk16, uint32_t *__restrict__ sink) {
    const u32x4 *base = p + (size_t)blockIdx.x * chunk16 + threadIdx.x;
    uint32_t acc = 0;
    for (size_t i = 0; i < chunk16; i += (size_t)kReadThreads * kReadInFlight) {
        u32x4 v[kReadInFlight];
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u)
            v[u] = __builtin_nontemporal_load(base + i + (size_t)u * kReadThreads);
#pragma unroll
        for (int u = 0; u < kReadInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(size_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

constexpr int kMixThreads = 512;
constexpr int kSeedWords = 512;      // 16-byte words of the seed buffer (8 KiB)
constexpr int kLdsWords = 6144;      // 96 KiB: one workgroup per CU, as the prefill kernel
constexpr int kMixProducts = 8;      // independent accumulators per wave

// Per iteration each wave issues 8 products into 8 accumulators; the first RD of
// them take their A operand from a fresh 16-byte-per-lane LDS read (1 KiB per
// wave), the others from a register.  The read rows move with the iteration
// (16 sets), so operand values change and no read is loop-invariant.  With SM
// every product is paired with x = x * 0.5 - 0.25 (FMA), e = 2^x, s += e, and
// every second product with a bf16 pair conversion of two e's folded into a
// running XOR (for 16x16x32 products, every second product: the same VALU
// work per flop).
template <int RD, bool SM, bool SMALL>
__global__ __launch_bounds__(kMixThreads, 1) void ceiling_mix_kernel(
    const u32x4 *__restrict__ seed, float *__restrict__ out, int iterations) {
    __shared__ u32x4 lds[kLdsWords];
    for (int i = threadIdx.x; i < kLdsWords; i += kMixThreads) lds[i] = seed[i & (kSeedWords - 1)];
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bf16x8 b = __builtin_bit_cast(bf16x8, seed[(threadIdx.x + 7) & (kSeedWords - 1)]);
    const bf16x8 a_reg = __builtin_bit_cast(bf16x8, seed[(threadIdx.x + 3) & (kSeedWords - 1)]);
    typedef typename std::conditional<SMALL, f32x4, f32x16>::type acc_t;
    acc_t c[kMixProducts];
#pragma unroll
    for (int i = 0; i < kMixProducts; ++i) c[i] = acc_t{};
    float x[kMixProducts], s[kMixProducts];
#pragma unroll
    for (int i = 0; i < kMixProducts; ++i) {
        x[i] = 0.001f * (float)(threadIdx.x + i);
        s[i] = 0.0f;
    }
    uint32_t pk = 0;
    for (int it = 0; it < iterations; ++it) {
        // rows wave * 64 + lane + 64 (it mod 16) + 512 i: at most 511 + 960 + 3584 < kLdsWords
        const u32x4 *set = lds + wave * 64 + lane + 64 * (it & 15);
        bf16x8 a[kMixProducts];
#pragma unroll
        for (int i = 0; i < kMixProducts; ++i)
            a[i] = i < RD ? __builtin_bit_cast(bf16x8, set[512 * i]) : a_reg;
#pragma unroll
        for (int i = 0; i < kMixProducts; ++i) {
            if constexpr (SMALL)
                c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, c[i], 0, 0, 0);
            else
                c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, c[i], 0, 0, 0);
        }
        if constexpr (SM) {
            // the same VALU work per flop for both shapes: 8 elements per 8
            // 32x32x16 products, 4 per 8 16x16x32 products
            constexpr int NE = SMALL ? kMixProducts / 2 : kMixProducts;
            float e[NE];
#pragma unroll
            for (int i = 0; i < NE; ++i) {
                x[i] = x[i] * 0.5f - 0.25f;
                e[i] = __builtin_amdgcn_exp2f(x[i]);
                s[i] += e[i];
            }
#pragma unroll
            for (int i = 0; i < NE; i += 2) {
                const bf16x2 pair = {(__bf16)e[i], (__bf16)e[i + 1]};
                pk ^= __builtin_bit_cast(uint32_t, pair);
            }
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < kMixProducts; ++i)
#pragma unroll
        for (int j = 0; j < (SMALL ? 4 : 16); ++j) r += c[i][j];
#pragma unroll
    for (int i = 0; i < kMixProducts; ++i) r += s[i];
    r += (float)(pk & 1u);
    // one LDS word in the result keeps the 96 KiB allocation (one workgroup
    // per CU) also in the variants without operand reads
    r += (float)(lds[threadIdx.x].x & 1u);
    out[(size_t)blockIdx.x * kMixThreads + threadIdx.x] = r;
}

template <int RD, bool SMALL>
void launch_mix(bool sm, int n_wg, int iterations, const u32x4 *seed, float *out, hipStream_t st) {
    if (sm)
        ceiling_mix_kernel<RD, true, SMALL><<<n_wg, kMixThreads, 0, st>>>(seed, out, iterations);
    else
        ceiling_mix_kernel<RD, false, SMALL><<<n_wg, kMixThreads, 0, st>>>(seed, out, iterations);
}

template <int RD>
void launch_mix(bool sm, bool small, int n_wg, int iterations, const u32x4 *seed, float *out,
                hipStream_t st) {
    if (small) launch_mix<RD, true>(sm, n_wg, iterations, seed, out, st);
    else launch_mix<RD, false>(sm, n_wg, iterations, seed, out, st);
}

constexpr int kValuChains = 8;
constexpr int kValuUnroll = 8;

// KIND 0: x = x * a + b (FMA); 1: x = 2^(-x) (v_exp_f32 with a negated input,
// which converges to about 0.64); 2: both, one after the other, per chain.
// Every chain is independent, so the issue rate alone sets the pace.  Each
// wave writes (shader-clock ticks, realtime ticks) of its loop.
template <int KIND>
__global__ __launch_bounds__(1024) void ceiling_valu_kernel(
    float *__restrict__ out, unsigned long long *__restrict__ cycles, int iterations) {
    float x[kValuChains];
#pragma unroll
    for (int i = 0; i < kValuChains; ++i) x[i] = 0.25f + 0.001f * (float)(threadIdx.x + i);
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iterations; ++it) {
        // 8 steps of every chain per iteration, so the loop branch is amortised
#pragma unroll
        for (int u = 0; u < kValuUnroll; ++u)
#pragma unroll
            for (int i = 0; i < kValuChains; ++i) {
                if constexpr (KIND == 0 || KIND == 2) x[i] = __builtin_fmaf(x[i], 0.999f, 0.0001f);
                if constexpr (KIND == 1 || KIND == 2) x[i] = __builtin_amdgcn_exp2f(-x[i]);
            }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float r = 0.0f;
#pragma unroll
    for (int i = 0; i < kValuChains; ++i) r += x[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
    if ((threadIdx.x & 63) == 0) {
        const size_t w = (size_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
        cycles[2 * w] = t1 - t0;
        cycles[2 * w + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" const char *fa_ceiling_last_error(void) { return g_err; }

// kind: 0 FMA chains, 1 exponential chains, 2 both interleaved; n_workgroups
// of `threads` threads (a multiple of 64, at most 1024); iterations >= 1 (64
// chain steps per lane each: 8 chains x 8); out: device, n_workgroups * threads floats;
// cycles: device, 2 values per wave (n_workgroups * threads / 32): its loop's
// shader-clock ticks, then its realtime (100 MHz) ticks.
extern "C" int fa_ceiling_valu(int kind, int n_workgroups, int threads, int iterations,
                               float *out, unsigned long long *cycles, hipStream_t stream) {
    if (!out || !cycles) return fail(1, "fa_ceiling_valu: null pointer");
    if (kind < 0 || kind > 2) return fail(1, "fa_ceiling_valu: kind must be 0, 1 or 2");
    if (n_workgroups < 1) return fail(1, "fa_ceiling_valu: n_workgroups must be >= 1");
    if (threads < 64 || threads > 1024 || threads % 64 != 0)
        return fail(1, "fa_ceiling_valu: threads must be a multiple of 64 up to 1024");
    if (iterations < 1) return fail(1, "fa_ceiling_valu: iterations must be >= 1");
    (void)hipGetLastError();
    if (kind == 0)
        ceiling_valu_kernel<0><<<n_workgroups, threads, 0, stream>>>(out, cycles, iterations);
    else if (kind == 1)
        ceiling_valu_kernel<1><<<n_workgroups, threads, 0, stream>>>(out, cycles, iterations);
    else
        ceiling_valu_kernel<2><<<n_workgroups, threads, 0, stream>>>(out, cycles, iterations);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(4, hipGetErrorString(e));
    return 0;
}

// buf: device, bytes long, 16-byte aligned; chunk: bytes per workgroup, a
// multiple of 32 KiB dividing bytes; sink: device, (bytes / chunk) * 256
// uint32.  Returns 0, 1 for a bad argument, 4 for a HIP launch error.
extern "C" int fa_ceiling_read(const void *buf, size_t bytes, size_t chunk, uint32_t *sink,
                               hipStream_t stream) {
    if (!buf || !sink) return fail(1, "fa_ceiling_read: null pointer");
    if (((uintptr_t)buf & 15u) != 0) return fail(1, "fa_ceiling_read: buffer not 16-byte aligned");
    if (chunk == 0 || chunk % kReadGranule != 0)
        return fail(1, "fa_ceiling_read: chunk must be a positive multiple of 32 KiB");
    if (bytes == 0 || bytes % chunk != 0) return fail(1, "fa_ceiling_read: chunk must divide bytes");
    if (bytes / chunk > (size_t)INT_MAX) return fail(1, "fa_ceiling_read: too many chunks");
    (void)hipGetLastError();
    ceiling_read_kernel<<<(unsigned)(bytes / chunk), kReadThreads, 0, stream>>>(
        (const u32x4 *)buf, chunk / 16, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(4, hipGetErrorString(e));
    return 0;
}

// reads_per_8: 0, 2, 4, 6 or 8 LDS operand reads per 8 products; softmax: 0
// or 1; shape: 0 for 32x32x16 products (32768 flop each), 1 for 16x16x32
// (16384 flop each); n_workgroups >= 1; iterations >= 1 (8 products per wave
// each); seed: device, 8 KiB; out: device, n_workgroups * 512 floats.  Each
// launch performs n_workgroups * 8 waves * iterations * 8 products.
extern "C" int fa_ceiling_mix(int reads_per_8, int softmax, int shape, int n_workgroups,
                              int iterations, const void *seed, float *out, hipStream_t stream) {
    if (!seed || !out) return fail(1, "fa_ceiling_mix: null pointer");
    if (softmax != 0 && softmax != 1) return fail(1, "fa_ceiling_mix: softmax must be 0 or 1");
    if (shape != 0 && shape != 1) return fail(1, "fa_ceiling_mix: shape must be 0 or 1");
    if (n_workgroups < 1) return fail(1, "fa_ceiling_mix: n_workgroups must be >= 1");
    if (iterations < 1) return fail(1, "fa_ceiling_mix: iterations must be >= 1");
    const u32x4 *sd = (const u32x4 *)seed;
    const bool sm = softmax == 1, small = shape == 1;
    (void)hipGetLastError();
    switch (reads_per_8) {
        case 0: launch_mix<0>(sm, small, n_workgroups, iterations, sd, out, stream); break;
        case 2: launch_mix<2>(sm, small, n_workgroups, iterations, sd, out, stream); break;
        case 4: launch_mix<4>(sm, small, n_workgroups, iterations, sd, out, stream); break;
        case 6: launch_mix<6>(sm, small, n_workgroups, iterations, sd, out, stream); break;
        case 8: launch_mix<8>(sm, small, n_workgroups, iterations, sd, out, stream); break;
        default: return fail(1, "fa_ceiling_mix: reads_per_8 must be 0, 2, 4, 6 or 8");
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(4, hipGetErrorString(e));
    return 0;
}
