// Internal helpers shared by the gfx950 kernels of libdflash2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    lo = (uint32_t)__shfl_xor((int)lo, m, kWave);
    hi = (uint32_t)__shfl_xor((int)hi, m, kWave);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t y = shfl_xor_u64(x, m);
        x = y > x ? y : x;
    }
    return x;
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

// Fixed butterfly order: identical results from run to run.
__device__ __forceinline__ MaxSum wave_ms_reduce(MaxSum a) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        MaxSum b{__shfl_xor(a.m, m, kWave), __shfl_xor(a.s, m, kWave)};
        a = ms_combine(a, b);
    }
    return a;
}

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
                                                int K, uint64_t* out) {
    const int lane = threadIdx.x & (kWave - 1);
    int head = 0;
    for (int round = 0; round < K; ++round) {
        uint64_t key = (lane < nsrc && head < len) ? lists[lane * stride + head] : 0ull;
        uint64_t mx = wave_max_u64(key);
        if (key == mx && mx != 0ull) ++head;
        if (lane == 0) out[round] = mx;
    }
}

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dfs
