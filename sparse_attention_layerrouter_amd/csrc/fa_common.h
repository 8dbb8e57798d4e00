// fa_common.h -- device helpers shared by the gfx950 kernels of libfluxattn.
//
// Holds the wavefront primitives (DPP / swizzle / permlane reductions), bf16
// conversions and the streaming sink + local-window rule of the sparse (SA)
// layers.  The rule follows the streaming block-sparse layout of the Flux
// Attention pages [thelatestinai paper page, Table 6: block size, sink size;
// codewithpapers function list: generate_streaming_info_blocksparse_flash_attn]:
// with ns = sink / block and nw = window / block, query block i keeps key
// blocks j < ns and i - nw + 1 <= j <= i; inside a kept block the causal rule
// s <= t applies.  FA layers keep every j <= i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16x2 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float a)
{
    return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Cross-lane moves.  All patterns are fixed, so reductions are deterministic.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// quad_perm [1,0,3,2] = lane ^ 1; quad_perm [2,3,0,1] = lane ^ 2
__device__ __forceinline__ float xor1(float x) { return dpp<0xB1>(x); }
__device__ __forceinline__ float xor2(float x) { return dpp<0x4E>(x); }
// row_half_mirror: lane i -> 7 - i inside each group of 8
__device__ __forceinline__ float half_mirror(float x) { return dpp<0x141>(x); }
// row_mirror: lane i -> 15 - i inside each row of 16
__device__ __forceinline__ float row_mirror(float x) { return dpp<0x140>(x); }
// ds_swizzle bit mode: lane ^ 16 inside each group of 32
__device__ __forceinline__ float xor16(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
__device__ __forceinline__ float xor8(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x201F));
}
__device__ __forceinline__ float xor4(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x101F));
}

// Lanes l and l ^ 32 combined with max / sum; both halves get the result.
__device__ __forceinline__ float max_xor32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that hold one row in the
// 16x16 product layouts) combined with max / sum; the lane ^ 16 step is a VALU
// row swap: with both operands x, each lane receives x[l] and x[l ^ 16].
__device__ __forceinline__ float row4_sum(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return sum_xor32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}
__device__ __forceinline__ float row4_max(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max_xor32(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32); every lane of the
// group receives the same value.  Order: pairs, quads, 8s, 16s, 32s.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2) x += xor1(x);
    if constexpr (N >= 4) x += xor2(x);
    if constexpr (N >= 8) x += half_mirror(x);
    if constexpr (N >= 16) x += row_mirror(x);
    if constexpr (N >= 32) x += xor16(x);
    return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x)
{
    if constexpr (N >= 2) x = fmaxf(x, xor1(x));
    if constexpr (N >= 4) x = fmaxf(x, xor2(x));
    if constexpr (N >= 8) x = fmaxf(x, half_mirror(x));
    if constexpr (N >= 16) x = fmaxf(x, row_mirror(x));
    if constexpr (N >= 32) x = fmaxf(x, xor16(x));
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// Sparse rule
// ---------------------------------------------------------------------------

struct SparseRule {
    int ns;       // sink blocks
    int nw;       // window blocks (including the query's own block)
    int bk_log2;  // log2(block tokens)
    int nl;       // Triangle attention: the last nl query blocks of a sequence keep
                  // every key block; 0 for the streaming rule
};

// First position of the dense tail of a sequence of T tokens under the rule
// (T when the rule has none): rows at or past it keep every earlier key.
__device__ __forceinline__ int dense_tail_start(int T, const SparseRule &r)
{
    if (r.nl <= 0) return T;
    const int nb = (T + (1 << r.bk_log2) - 1) >> r.bk_log2;
    return max(0, nb - r.nl) << r.bk_log2;
}

// Key s visible from query t (positions inside one sequence).
__device__ __forceinline__ bool visible(int t, int s, bool fa, const SparseRule &r)
{
    if (s > t) return false;
    if (fa) return true;
    int j = s >> r.bk_log2, i = t >> r.bk_log2;
    return j < r.ns || j > i - r.nw;
}

// Union of the kept key-token ranges of query rows [p0, p1) (p0 < p1):
// [0, a_end) and [b_begin, p1).  For FA the first range is [0, p1) and the
// second empty; for SA a_end <= b_begin.
__device__ __forceinline__ void kept_ranges(int p0, int p1, bool fa, const SparseRule &r,
                                            int &a_end, int &b_begin)
{
    if (fa) {
        a_end = p1;
        b_begin = p1;
        return;
    }
    int sink_tok = r.ns << r.bk_log2;
    a_end = min(sink_tok, p1);
    int win = ((p0 >> r.bk_log2) - r.nw + 1) << r.bk_log2;
    b_begin = max(win, a_end);
    b_begin = min(b_begin, p1);
}

}  // namespace fa
