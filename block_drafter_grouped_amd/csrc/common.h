// Internal helpers shared by the gfx950 kernels of libdflash2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Candidate keys.  A 64-bit key orders candidates exactly as the method
// does: larger logit first, equal logits by smaller vocabulary id.  High word:
// the fp32 bits mapped to an unsigned order-preserving code (-0 folded onto
// +0); low word: ~id.  Keys of distinct ids are distinct, so a max over keys
// has a single winner.  Key 0 is below every finite or -inf logit and marks
// an empty slot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t make_key(float v, uint32_t id) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ float key_value(uint64_t k) {
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)k); }

// ---------------------------------------------------------------------------
// Wave-wide reductions.  Four DPP steps (quad swaps, then the half-row and
// row mirrors) make every lane of each 16-lane row hold the row's result;
// v_readlane then brings the four row results to scalar registers.  DPP moves
// are VALU operations with a few cycles of latency, where an LDS-routed
// shuffle costs a full LDS round trip per step.  All 64 lanes must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(x >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)x);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
}
__device__ __forceinline__ float readlane_f32(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = umax64(x, dpp_u64<kDppQuadXor1>(x));
    x = umax64(x, dpp_u64<kDppQuadXor2>(x));
    x = umax64(x, dpp_u64<kDppHalfMirror>(x));
    x = umax64(x, dpp_u64<kDppMirror>(x));
    return umax64(umax64(readlane_u64(x, 0), readlane_u64(x, 16)), umax64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

__device__ __forceinline__ float wave_max_f32(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppMirror>(x));
    return fmaxf(fmaxf(readlane_f32(x, 0), readlane_f32(x, 16)), fmaxf(readlane_f32(x, 32), readlane_f32(x, 48)));
}

// Sum in a fixed order (the same result on every run).
__device__ __forceinline__ float wave_sum_f32(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppHalfMirror>(x);
    x += dpp_f32<kDppMirror>(x);
    return (readlane_f32(x, 0) + readlane_f32(x, 16)) + (readlane_f32(x, 32) + readlane_f32(x, 48));
}

// Online (max, sum of exp) pair: value set {x} is represented by
// m = max x and s = sum exp(x - m).  m = -inf, s = 0 is the empty set.
struct MaxSum {
    float m, s;
};

__device__ __forceinline__ MaxSum ms_combine(MaxSum a, MaxSum b) {
    if (a.m == -INFINITY) return b;
    if (b.m == -INFINITY) return a;
    float m = fmaxf(a.m, b.m);
    return MaxSum{m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
}

template <int CTRL>
__device__ __forceinline__ MaxSum ms_dpp_step(MaxSum a) {
    return ms_combine(a, MaxSum{dpp_f32<CTRL>(a.m), dpp_f32<CTRL>(a.s)});
}

// Fixed combination order: identical results from run to run.
__device__ __forceinline__ MaxSum wave_ms_reduce(MaxSum a) {
    a = ms_dpp_step<kDppQuadXor1>(a);
    a = ms_dpp_step<kDppQuadXor2>(a);
    a = ms_dpp_step<kDppHalfMirror>(a);
    a = ms_dpp_step<kDppMirror>(a);
    MaxSum r = MaxSum{readlane_f32(a.m, 0), readlane_f32(a.s, 0)};
    r = ms_combine(r, MaxSum{readlane_f32(a.m, 16), readlane_f32(a.s, 16)});
    r = ms_combine(r, MaxSum{readlane_f32(a.m, 32), readlane_f32(a.s, 32)});
    r = ms_combine(r, MaxSum{readlane_f32(a.m, 48), readlane_f32(a.s, 48)});
    return r;
}

// ---------------------------------------------------------------------------
// Merging sorted key lists across lanes.  Each lane holds N keys sorted
// descending.  One level takes a partner lane's list (a DPP move), keeps the
// element-wise max of the own list and the partner's list reversed -- which
// holds exactly the N largest of the union, as a bitonic sequence -- and sorts
// that with a bitonic half-cleaner cascade.  Six levels (quad swaps, the two
// mirrors, then the row broadcasts into rows 1/3 and row 3) leave in lane 63
// the N largest keys of all 64 lanes.  All lanes must be active.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64m(uint64_t x) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x >> 32), CTRL, ROW_MASK, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

template <int N>
__device__ __forceinline__ void bitonic_clean_desc(uint64_t (&c)[N]) {
#pragma unroll
    for (int st = N / 2; st >= 1; st >>= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if ((i & st) == 0) {
                const uint64_t x = c[i], y = c[i + st];
                const bool gt = x > y;
                c[i] = gt ? x : y;
                c[i + st] = gt ? y : x;
            }
        }
    }
}

// a <- the N largest keys of a and b (both sorted descending), sorted.
template <int N>
__device__ __forceinline__ void merge_top(uint64_t (&a)[N], const uint64_t (&b)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = umax64(a[i], b[N - 1 - i]);
    bitonic_clean_desc<N>(a);
}

template <int CTRL, int ROW_MASK, int N>
__device__ __forceinline__ void merge_top_dpp(uint64_t (&a)[N]) {
    uint64_t b[N];
#pragma unroll
    for (int i = 0; i < N; ++i) b[i] = dpp_u64m<CTRL, ROW_MASK>(a[i]);
    merge_top<N>(a, b);
}

template <int N>
__device__ __forceinline__ void wave_merge_top(uint64_t (&a)[N]) {
    merge_top_dpp<kDppQuadXor1, 0xF>(a);
    merge_top_dpp<kDppQuadXor2, 0xF>(a);
    merge_top_dpp<kDppHalfMirror, 0xF>(a);
    merge_top_dpp<kDppMirror, 0xF>(a);
    merge_top_dpp<kDppRowBcast15, 0xA>(a);
    merge_top_dpp<kDppRowBcast31, 0x8>(a);
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

constexpr int kCandCap = 256;

// Sorted (descending) register list of KL keys; inserts x, dropping the
// smallest.  Straight-line code so the list stays in registers.
template <int KL>
__device__ __forceinline__ void list_insert(uint64_t (&lst)[KL], uint64_t x) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
        uint64_t hi = lst[i] > x ? lst[i] : x;
        x = lst[i] > x ? x : lst[i];
        lst[i] = hi;
    }
}

// One wavefront merges up to 64 sorted (descending) lists held in LDS into
// the top K keys.  List `src` starts at lists[src * stride] and has `len`
// entries.  Lane 0 receives the result in out[0..K) (global or LDS).  Every
// round takes the largest head; keys are distinct, so exactly one lane
// advances.  Empty heads read as 0.
__device__ __forceinline__ void wave_tournament(const uint64_t* lists, int nsrc, int stride, int len,
                                                int K, uint64_t* out, int out_stride = 1) {
    const int lane = threadIdx.x & (kWave - 1);
    int head = 0;
    for (int round = 0; round < K; ++round) {
        uint64_t key = (lane < nsrc && head < len) ? lists[lane * stride + head] : 0ull;
        uint64_t mx = wave_max_u64(key);
        if (key == mx && mx != 0ull) ++head;
        if (lane == 0) out[(size_t)round * out_stride] = mx;
    }
}

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dfs
