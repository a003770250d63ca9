// Step 3 of the draft-block path on written logits (vLLM release-note
// article on DFlash2, section "two additions": the top-K of each slot's
// log-softmax over the full vocabulary): per-slice top-K keys and
// (max, sum of exp) partials, merged per row by the kernels in head.hip.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

// Top-K keys and (max, sum of exp) of one slice of one row of fp32 logits;
// one workgroup of 512 threads per (slice, row), K <= 64, four workgroups
// per CU so that some load while others rank (the launch bound caps the
// registers at 64; the few values that spill cost less than the lost
// occupancy: 14 % on 256 rows of the page vocabulary).
//  - Thread t holds 16 values of the slice in registers: with 16-B aligned
//    rows (V % 4 == 0) the 4-value units t, t + 512, ..., else the values
//    t, t + 512, ...  Consecutive threads read consecutive addresses.
//  - Every 8-lane group takes the largest key of its values: 64 group
//    maxima, distinct keys unless 0 (an empty group).  Their K-th largest,
//    theta, has at least K keys >= theta in the slice, so every key of the
//    slice's top K is >= theta; for ordinary data a few dozen keys pass.
//    The maxima are ranked by counting, wave w counting maxima 8w .. 8w + 7.
//    The tests run on the float value and id of a key, not on 64-bit keys.
//  - The passing keys are gathered in LDS and each is placed by its rank
//    among them.
//  - If more than kSliceCap keys pass (massively tied logits), theta is
//    raised to the exact K-th largest key by bisection over the 64-bit key
//    range, counting keys >= the midpoint; exactly K keys then pass.
// The slice's (max, sum of exp) comes from the same registers.
constexpr int kSliceThreads = 512;
constexpr int kSliceQ = 16;                                // values per thread
constexpr int kSliceLen = kSliceQ * kSliceThreads;         // longest slice
constexpr int kSliceCap = 1024;                            // gathered keys

template <bool VEC>
__device__ __forceinline__ int slice_id(int v0, int t, int q) {
    return VEC ? v0 + 4 * (t + kSliceThreads * (q / 4)) + (q & 3) : v0 + t + kSliceThreads * q;
}

// make_key(x, id) >= the key of (tv, tid), for a key made from a value
// (not 0, and not a midpoint between keys: its value must be one a key
// decodes to).  -0 and +0 compare equal, as the keys fold them.
__device__ __forceinline__ bool key_ge(float x, uint32_t id, float tv, uint32_t tid) {
    return x > tv || (x == tv && id <= tid);
}

template <bool VEC>
__global__ __launch_bounds__(kSliceThreads, 8) void slice_topk_kernel(const float* __restrict__ logits, int V,
                                                                      int nsl, int K, uint64_t* __restrict__ part_keys,
                                                                      float2* __restrict__ part_ms) {
    constexpr int NWV = kSliceThreads / kWave;
    __shared__ uint64_t gmax[64];
    __shared__ int gabove[NWV][64];
    __shared__ uint64_t cand[kSliceCap];
    __shared__ float wsum[NWV];
    __shared__ int wcnt[NWV];
    __shared__ int cnt;
    __shared__ uint64_t theta_sh, top_sh;
    const int sl = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
    const int lane = t & (kWave - 1), wave = t / kWave;
    int v0, v1;
    if (VEC) {
        const int64_t n4 = V / 4;
        v0 = 4 * (int)(n4 * sl / nsl);
        v1 = 4 * (int)(n4 * (sl + 1) / nsl);
    } else {
        v0 = (int)((int64_t)V * sl / nsl);
        v1 = (int)((int64_t)V * (sl + 1) / nsl);
    }
    const float* src = logits + (size_t)row * V;
    float x[kSliceQ];
    if (VEC) {
#pragma unroll
        for (int q4 = 0; q4 < kSliceQ / 4; ++q4) {
            const int v = slice_id<true>(v0, t, 4 * q4);
            const f32x4 u = v < v1 ? *(const f32x4*)(src + v) : f32x4{NAN, NAN, NAN, NAN};
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * q4 + e] = u[e];
        }
    } else {
#pragma unroll
        for (int q = 0; q < kSliceQ; ++q) {
            const int v = slice_id<false>(v0, t, q);
            x[q] = v < v1 ? src[v] : NAN;
        }
    }
    // Positions outside the slice hold NaN, which fails every comparison.
    // The thread's largest key: largest value, first (lowest) id among equals.
    float mv = NAN;
    int mid = -1;
#pragma unroll
    for (int q = 0; q < kSliceQ; ++q) {
        if (x[q] > mv || (mid < 0 && x[q] == x[q])) {
            mv = x[q];
            mid = slice_id<VEC>(v0, t, q);
        }
    }
    uint64_t mk = mid >= 0 ? make_key(mv, (uint32_t)mid) : 0ull;
    mk = umax64(mk, dpp_u64<kDppQuadXor1>(mk));
    mk = umax64(mk, dpp_u64<kDppQuadXor2>(mk));
    mk = umax64(mk, dpp_u64<kDppHalfMirror>(mk));
    if ((lane & 7) == 0) gmax[wave * 8 + lane / 8] = mk;
    if (t == 0) {
        cnt = 0;
        theta_sh = 0ull;
    }
    __syncthreads();
    {  // thread (w, i) counts the maxima 8w .. 8w + 7 above group maximum i
        const uint64_t g = gmax[lane];
        int c = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) c += gmax[8 * wave + j] > g ? 1 : 0;
        gabove[wave][lane] = c;
    }
    __syncthreads();
    if (wave == 0) {  // lane i: the rank of group maximum i
        const uint64_t g = gmax[lane];
        int rank = 0;
#pragma unroll
        for (int w = 0; w < NWV; ++w) rank += gabove[w][lane];
        if (rank == K - 1 && g != 0ull) theta_sh = g;  // fewer than K non-empty groups: theta stays 0
        if (rank == 0) top_sh = g;                      // unique when g != 0; all-empty slices write 0
    }
    __syncthreads();
    const uint64_t top = top_sh;
    const float m = top ? key_value(top) : -INFINITY;
    float se = 0.f;
    if (top) {
#pragma unroll
        for (int q = 0; q < kSliceQ; ++q)
            if (x[q] == x[q]) se += __expf(x[q] - m);
    }
    se = wave_sum_f32(se);
    if (lane == 0) wsum[wave] = se;

    uint64_t theta = theta_sh;
    int n = 0;
    for (int attempt = 0; attempt < 2; ++attempt) {
        // gather the keys >= theta (theta 0: every key of the slice; NaN,
        // outside the slice, never passes)
        const float tv = theta ? key_value(theta) : -INFINITY;
        const uint32_t tid = theta ? (uint32_t)key_id(theta) : 0xFFFFFFFFu;
        int mine = 0;
#pragma unroll
        for (int q = 0; q < kSliceQ; ++q) mine += key_ge(x[q], (uint32_t)slice_id<VEC>(v0, t, q), tv, tid) ? 1 : 0;
        int p = 0;
        if (mine) p = atomicAdd(&cnt, mine);
        __syncthreads();
        n = cnt;
        if (n <= kSliceCap) {
            if (mine) {
#pragma unroll
                for (int q = 0; q < kSliceQ; ++q) {
                    const uint32_t v = (uint32_t)slice_id<VEC>(v0, t, q);
                    if (key_ge(x[q], v, tv, tid)) cand[p++] = make_key(x[q], v);
                }
            }
            break;
        }
        // Too many: the exact K-th largest key by bisection (more than
        // kSliceCap >= K keys are >= theta, so it lies in [theta, top]).
        uint64_t lo = theta, hi = top;
        while (lo < hi) {
            const uint64_t mk2 = lo + (hi - lo) / 2 + 1;  // any 64-bit value: compare whole keys
            int c = 0;
#pragma unroll
            for (int q = 0; q < kSliceQ; ++q)
                c += (x[q] == x[q] && make_key(x[q], (uint32_t)slice_id<VEC>(v0, t, q)) >= mk2) ? 1 : 0;
            c = (int)wave_sum_f32((float)c);  // exact: counts stay far below 2^24
            if (lane == 0) wcnt[wave] = c;
            __syncthreads();
            int all = 0;
            for (int w = 0; w < NWV; ++w) all += wcnt[w];
            __syncthreads();
            if (all >= K) lo = mk2;
            else hi = mk2 - 1;
        }
        theta = lo;
        __syncthreads();  // every thread has read cnt
        if (t == 0) cnt = 0;
        __syncthreads();
    }
    if (n > kSliceCap) n = 0;  // unreachable: exactly K <= kSliceCap keys pass the exact threshold
    __syncthreads();
    uint64_t* out = part_keys + (size_t)row * K * nsl + sl;
    for (int i = t; i < n; i += kSliceThreads) {
        const uint64_t key = cand[i];
        int rank = 0;
#pragma unroll 8
        for (int j = 0; j < n; ++j) rank += cand[j] > key ? 1 : 0;
        if (rank < K) out[(size_t)rank * nsl] = key;
    }
    for (int i = n + t; i < K; i += kSliceThreads) out[(size_t)i * nsl] = 0ull;
    if (t == 0) {
        float sum = 0.f;
        for (int w = 0; w < NWV; ++w) sum += wsum[w];
        part_ms[(size_t)row * nsl + sl] = make_float2(m, top ? sum : 0.f);
    }
}

}  // namespace

// Slices of the logits ranked per row: at most kSliceLen values each, at
// most 256 (the partial buffer's chunk count), and enough (slice, row)
// workgroups to fill the chip when there are few rows -- but no shorter than
// kSliceMin values, so that every lane group holds values: a slice with
// fewer occupied groups than K has no threshold and ranks all its values.
constexpr int kSliceMin = 8 * kSliceThreads;

int logits_slices(const Dims& d) {
    const int64_t need = ((int64_t)d.V + kSliceLen - 1) / kSliceLen;
    const int64_t fill = (2048 + d.rows() - 1) / d.rows();
    const int64_t most = std::min<int64_t>(256, std::max<int64_t>(1, (int64_t)d.V / kSliceMin));
    return (int)std::max<int64_t>(need, std::min<int64_t>(fill, most));
}

hipError_t launch_logits_partials(const Dims& d, const float* logits, int nsl, uint64_t* keys, float2* ms,
                                  hipStream_t s) {
    const dim3 grid(nsl, d.rows());
    if (d.V % 4 == 0)
        slice_topk_kernel<true><<<grid, kSliceThreads, 0, s>>>(logits, d.V, nsl, d.K, keys, ms);
    else
        slice_topk_kernel<false><<<grid, kSliceThreads, 0, s>>>(logits, d.V, nsl, d.K, keys, ms);
    return hipGetLastError();
}

}  // namespace dfs
