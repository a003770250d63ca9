// Steps 2-3 of the draft-block path: the vocabulary head (the target's
// shared lm_head), log-softmax and the per-slot top-K candidates (vLLM
// release-note article on DFlash2, section "two additions": at each slot the
// selector works on the K tokens the target head ranks highest).  Up to 8
// rows with K <= 16 (the batch-1 case) the logits are never written to HBM:
// the streaming head keeps, per vocabulary chunk, each row's top-K keys and
// its (max, sum of exp) pair.  More rows
// with K <= 16: the GEMM head writes the logits and per-segment partials,
// and its segment merge ranks them (gemm_head.hip).  Otherwise a head that
// writes the logits is followed by the slice top-K (slice_topk.hip).  The
// merge kernels here combine chunk or slice partials.
//
// bf16 streaming head (up to 8 rows): the work is a stream of the [V, D]
// weight (2.5 GB at D 5120, V 248 320) against a tiny [rows, D] operand, so
// it is bound by HBM.  One persistent workgroup per CU owns every nch-th
// vocabulary tile (tiles c, c + nch, ...: at any time the workgroups stream
// neighbouring tiles, which measured 2 % faster at the page shape than
// contiguous ranges per workgroup); the hidden rows sit in LDS for the whole kernel,
// pre-swizzled into MFMA B-operand order, and every wave streams its tiles
// with v_mfma_f32_16x16x32_bf16 while U k-steps of weight loads are in
// flight.  The MFMA's 16 output columns hold the (<= 8) rows, so part of each
// MFMA is padding -- harmless, the kernel waits on HBM.  The lanes that own
// results keep a sorted register list of their best keys plus an online
// (max, sum of exp).  head_pair_kernel (below) serves D % 64 == 0, the page
// shapes; head_bf16_kernel, with 16-row tiles of 64-B row pieces, serves the
// other D.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

constexpr size_t kMinHeadLds = 82 * 1024;  // > 80 KB: one workgroup per CU

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

template <int NW, int U, int KL>
__global__ __launch_bounds__(NW * kWave) void head_bf16_kernel(
    const uint16_t* __restrict__ y, int rows_total, int D, const uint16_t* __restrict__ W, int V, int nch, int K,
    uint64_t* __restrict__ part_keys, float2* __restrict__ part_ms, float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NSRC = NW * 4;
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * kRowsPass;
    const int rows = min(kRowsPass, rows_total - row_base);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int S = D / 32;

    // Hidden rows -> LDS.  16-B unit (s, q, j) holds channels 32s+8q..+7 of
    // row j; a wave's B operand for k-step s is then one contiguous 512-B
    // read (lanes with the same j%8 read the same unit).
    {
        uint4* ys = (uint4*)smem;
        const int per_row = S * 4;
        for (int u = threadIdx.x; u < per_row * kRowsPass; u += NW * kWave) {
            const int j = u / per_row, ch = u % per_row;
            uint4 v = {0u, 0u, 0u, 0u};
            if (j < rows) v = *(const uint4*)(y + (size_t)(row_base + j) * D + 8 * ch);
            ys[ch * kRowsPass + j] = v;
        }
    }
    __syncthreads();

    // Chunk c owns tiles c, c + nch, ... (as in head_pair_kernel, below).
    const int64_t T = ((int64_t)V + 15) / 16;
    const int cnt_c = (int)((T - c + nch - 1) / nch);
    const int my_n = max(0, (cnt_c - wave + NW - 1) / NW);
    const int i16 = lane & 15, q = lane >> 4, jrow = lane & 15;
    const int GPT = S / U;  // k-step groups per tile
    const int total = my_n * GPT;
    const uint4* ysb = (const uint4*)smem + q * kRowsPass + (lane & 7);

    auto tile_ptr = [&](int i) -> const uint16_t* {
        const int tt = c + nch * (wave + i * NW);
        const int v = min(tt * 16 + i16, V - 1);
        return W + (size_t)v * D + 8 * q;
    };

    uint64_t lst[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) lst[i] = 0ull;
    MaxSum ms{-INFINITY, 0.f};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    bf16x8 a[U];

    const uint16_t* cur = tile_ptr(0);
    if (total > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = *(const bf16x8*)(cur + 32 * u);
    }
    int ti = 0, gi = 0;
    for (int g = 0; g < total; ++g) {
        int nti = ti, ngi = gi + 1;
        if (ngi == GPT) {
            ngi = 0;
            nti = ti + 1;
        }
        const uint16_t* nxt = (g + 1 < total) ? (ngi == 0 ? tile_ptr(nti) : cur + 32 * U) : cur;
        const int s0 = gi * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bf16x8 b = *(const bf16x8*)(ysb + (size_t)(s0 + u) * 4 * kRowsPass);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc, 0, 0, 0);
            a[u] = *(const bf16x8*)(nxt + 32 * u);
        }
        if (ngi == 0) {
            // Tile done: lane holds logit[v0 + 4q + r][row jrow] in acc[r].
            const int v0 = (c + nch * (wave + ti * NW)) * 16 + 4 * q;
            if (jrow < rows) {
                float mnew = ms.m;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (v0 + r < V) mnew = fmaxf(mnew, acc[r]);
                float s = (ms.m == -INFINITY) ? 0.f : ms.s * __expf(ms.m - mnew);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (v0 + r < V) {
                        s += __expf(acc[r] - mnew);
                        const uint64_t key = make_key(acc[r], (uint32_t)(v0 + r));
                        if (key > lst[KL - 1]) list_insert<KL>(lst, key);
                        if (logits) logits[(size_t)(row_base + jrow) * V + v0 + r] = acc[r];
                    }
                }
                ms = MaxSum{mnew, s};
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        cur = nxt;
        ti = nti;
        gi = ngi;
    }
    __syncthreads();  // LDS switches from hidden rows to the merge lists

    uint64_t* L = (uint64_t*)smem;                                     // [kRowsPass][NSRC][K]
    float2* M = (float2*)(smem + (size_t)kRowsPass * NSRC * K * 8);  // [kRowsPass][NSRC]
    if (jrow < rows) {
        const int src = wave * 4 + q;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (i < K) L[((size_t)jrow * NSRC + src) * K + i] = lst[i];
        M[jrow * NSRC + src] = make_float2(ms.m, ms.s);
    }
    __syncthreads();
    for (int jr = wave; jr < rows; jr += NW) {
        wave_tournament(L + (size_t)jr * NSRC * K, NSRC, K, K, K, part_keys + (size_t)(row_base + jr) * K * nch + c,
                        nch);
        MaxSum x{-INFINITY, 0.f};
        if (lane < NSRC) {
            const float2 p = M[jr * NSRC + lane];
            x = MaxSum{p.x, p.y};
        }
        x = wave_ms_reduce(x);
        if (lane == 0) part_ms[(size_t)(row_base + jr) * nch + c] = make_float2(x.m, x.s);
    }
}

// Streaming head with whole-line loads.  The plain MFMA operand layout makes
// every wave load 16 rows x 64 B; with non-temporal loads, reads of at least
// 128 B per row per instruction stream markedly faster.  Here a tile is 8
// vocabulary rows and a k-step covers 64 channels as two 32-channel segments
// a and b: MFMA rows 0-7 carry segment a of the 8 rows and rows 8-15 carry
// segment b, while B-operand columns 0-7 carry the hidden rows at segment a
// and columns 8-15 the same rows at segment b.  The two diagonal 8x8 blocks
// of the product then hold the two partial dot products, one lane shuffle
// adds them, and each load instruction reads 8 rows x 128 contiguous bytes.
template <int NW, int U>
__global__ __launch_bounds__(NW * kWave) void head_pair_kernel(
    const uint16_t* __restrict__ y, int rows_total, int D, const uint16_t* __restrict__ W, int V, int nch, int K,
    uint64_t* __restrict__ part_keys, float2* __restrict__ part_ms, float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int KL = 16;
    constexpr int NSRC = NW * 2;  // two lanes per row per wave carry results
    static_assert(NSRC <= 16 && kRowsPass <= 8, "the lists of a row fit in one DPP row; two waves merge");
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * kRowsPass;
    const int rows = min(kRowsPass, rows_total - row_base);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int S = D / 64;
    const int i16 = lane & 15, q = lane >> 4;

    // Chunk c owns tiles c, c + nch, c + 2 nch, ... (wave w its w-th, (w +
    // NW)-th, ... of them), so that at any time the workgroups stream
    // neighbouring tiles.
    const int64_t T = ((int64_t)V + 7) / 8;
    const int cnt_c = (int)((T - c + nch - 1) / nch);
    const int my_n = max(0, (cnt_c - wave + NW - 1) / NW);
    const int GPT = S / U;
    const int total = my_n * GPT;
    const int a_off = 32 * (i16 >> 3) + 8 * q;

    auto tile_ptr = [&](int i) -> const uint16_t* {
        const int tt = c + nch * (wave + i * NW);
        const int v = min(tt * 8 + (i16 & 7), V - 1);
        return W + (size_t)v * D + a_off;
    };
    auto ldw = [](const uint16_t* p) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
    };

    // Hidden rows -> LDS.  16-B unit (s, q, j): row j & 7, channels
    // 64s + 32(j >> 3) + 8q .. +7, so the B operand of k-step s is one
    // contiguous 1 KB read by the 64 lanes.  The hidden rows' loads go out
    // first, all together (a row past `rows` reads row 0 and is stored as
    // zeros), then the first weight loads, which do not depend on them.
    // Loads complete in order, so the LDS stores wait on the hidden rows
    // only and the weight loads stay in flight meanwhile.  (Staged one unit
    // at a time, every store waited on all loads before it: ten L2 round
    // trips per workgroup with its weight stream idle.)
    constexpr int YB = 16;  // hidden-row units per thread in the first batch
    uint4* ys = (uint4*)smem;
    const int nyu = S * 64;
    auto yaddr = [&](int u) -> const uint4* {
        const int j = u & 15, qq = (u >> 4) & 3, s = u >> 6, row = j & 7;
        return (const uint4*)(y + (size_t)(row_base + (row < rows ? row : 0)) * D + 64 * s + 32 * (j >> 3) + 8 * qq);
    };
    uint4 yv[YB];
#pragma unroll
    for (int i = 0; i < YB; ++i) yv[i] = *yaddr(min((int)threadIdx.x + i * NW * kWave, nyu - 1));
    __builtin_amdgcn_sched_barrier(0);
    // (Unconditional: with no tile for this wave the address is still a
    // weight row, clamped, and the data goes unused.)
    bf16x8 a[U];
    const uint16_t* cur = tile_ptr(0);
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = ldw(cur + 64 * u);
    __builtin_amdgcn_sched_barrier(0);
    // No branch below either (a unit past the end stores the last unit's
    // data again), so that the wait counts stay exact and no store waits
    // on the weight loads.
#pragma unroll
    for (int i = 0; i < YB; ++i) {
        const int u = min((int)threadIdx.x + i * NW * kWave, nyu - 1);
        const uint32_t keep = ((u & 7) < rows) ? 0xFFFFFFFFu : 0u;
        ys[u] = uint4{yv[i].x & keep, yv[i].y & keep, yv[i].z & keep, yv[i].w & keep};
    }
    for (int u = threadIdx.x + YB * NW * kWave; u < nyu; u += NW * kWave)  // past the first batch
        ys[u] = ((u & 7) < rows) ? *yaddr(u) : uint4{0u, 0u, 0u, 0u};
    // The tail's lists live past the hidden rows, which the other waves still
    // read while a wave that is done stores its own.
    uint64_t* run = (uint64_t*)(smem + (size_t)nyu * 16);  // [kRowsPass][KL]
    float2* MW = (float2*)(run + kRowsPass * KL);            // [NW][kRowsPass]
    int* arrived = (int*)(MW + NW * kRowsPass);
    int* merged = arrived + 1;
    if (threadIdx.x == 0) {
        *arrived = 0;
        *merged = 0;
    }
    __syncthreads();
    const uint4* ysb = (const uint4*)smem + q * 16 + i16;

    uint64_t lst[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) lst[i] = 0ull;
    MaxSum ms{-INFINITY, 0.f};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // Lanes 0-7 and 16-23 own results: row i16, vocabulary 4q .. 4q+3 of the
    // tile; their partner lane + 40 holds the segment-b half.
    const bool owner = (i16 < 8) && (q < 2) && (i16 < rows);

    int ti = 0, gi = 0;
    for (int g = 0; g < total; ++g) {
        int nti = ti, ngi = gi + 1;
        if (ngi == GPT) {
            ngi = 0;
            nti = ti + 1;
        }
        const uint16_t* nxt = (g + 1 < total) ? (ngi == 0 ? tile_ptr(nti) : cur + 64 * U) : cur;
        const int s0 = gi * U;
        if (g + 1 < total) {  // wave-uniform
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bf16x8 b = *(const bf16x8*)(ysb + (size_t)(s0 + u) * 64);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc, 0, 0, 0);
                a[u] = ldw(nxt + 64 * u);
            }
        } else {
            // The last group issues no loads: nothing follows, and the
            // barrier after the loop would wait for them (an 8 KB reload per
            // wave, with its latency, at the end of the slowest wave).
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bf16x8 b = *(const bf16x8*)(ysb + (size_t)(s0 + u) * 64);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc, 0, 0, 0);
            }
        }
        if (ngi == 0) {
            float v4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v4[r] = acc[r] + __shfl(acc[r], (lane + 40) & (kWave - 1), kWave);
            const int v0 = (c + nch * (wave + ti * NW)) * 8 + 4 * q;
            if (owner) {
                float mnew = ms.m;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (v0 + r < V) mnew = fmaxf(mnew, v4[r]);
                float s = (ms.m == -INFINITY) ? 0.f : ms.s * __expf(ms.m - mnew);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (v0 + r < V) {
                        s += __expf(v4[r] - mnew);
                        const uint64_t key = make_key(v4[r], (uint32_t)(v0 + r));
                        if (key > lst[KL - 1]) list_insert<KL>(lst, key);
                        if (logits) logits[(size_t)(row_base + i16) * V + v0 + r] = v4[r];
                    }
                }
                ms = MaxSum{mnew, s};
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        cur = nxt;
        ti = nti;
        gi = ngi;
    }
    // Tail, per wave as soon as its own tiles are done.  Lane i16 < 8 (q =
    // 0) takes the list and (max, sum of exp) of lane i16 + 16 (q = 1, the
    // same row, the other half of the tile's vocabulary) through
    // v_permlane16_swap and merges them.  The waves then fold their lists
    // into running lists in LDS in the order they arrive (lane r: row r),
    // each waiting for the wave before it, so the last wave merges once.
    // The union's top KL keys do not depend on that order.  The (max, sum of
    // exp) pairs go to LDS per wave, and the last wave folds them in a fixed
    // tree (lane 8 r + w: row r, wave w; wave w with w ^ 1, w ^ 2, then the
    // mirrored half), which pairs the same operands as a butterfly over the
    // 2 NW lists in (wave, half) order.  (After a barrier for all waves, a
    // tournament over the 16 lists of every row took 4.4 us from the last
    // wave's last tile to the stored partials; a tree over the waves' lists
    // in the last wave, 4.3 us: one wave64 issues a VALU operation every
    // four cycles.)
    {
        uint64_t oth[KL];
#pragma unroll
        for (int i = 0; i < KL; ++i) {
            const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)lst[i], (uint32_t)lst[i], false, false);
            const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(lst[i] >> 32), (uint32_t)(lst[i] >> 32),
                                                             false, false);
            oth[i] = ((uint64_t)hi[1] << 32) | lo[1];  // rows 0 and 2 of the wave: lane + 16
        }
        merge_top<KL>(lst, oth);
        const auto pm = __builtin_amdgcn_permlane16_swap(__float_as_uint(ms.m), __float_as_uint(ms.m), false, false);
        const auto ps = __builtin_amdgcn_permlane16_swap(__float_as_uint(ms.s), __float_as_uint(ms.s), false, false);
        ms = ms_combine(ms, MaxSum{__uint_as_float(pm[1]), __uint_as_float(ps[1])});
    }
    if (lane < kRowsPass) MW[wave * kRowsPass + lane] = make_float2(ms.m, ms.s);
    int ticket = 0;
    if (lane == 0) ticket = __hip_atomic_fetch_add(arrived, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    uint64_t* my_run = run + (size_t)(lane & (kRowsPass - 1)) * KL;
    if (ticket > 0) {
        // The wave before this one in arrival order has its lists in: it
        // started before this wave arrived and waits for no later wave.
        // (The bound only guards against a hang; it is never reached.)
        for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__hip_atomic_load(merged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == ticket) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane < kRowsPass) {
            uint64_t oth[KL];
#pragma unroll
            for (int i = 0; i < KL; i += 2) {
                const u64x2 v = *(const u64x2*)(my_run + i);
                oth[i] = v[0];
                oth[i + 1] = v[1];
            }
            merge_top<KL>(lst, oth);
        }
    }
    if (ticket < NW - 1) {
        if (lane < kRowsPass) {
#pragma unroll
            for (int i = 0; i < KL; i += 2) *(u64x2*)(my_run + i) = u64x2{lst[i], lst[i + 1]};
        }
        if (lane == 0) __hip_atomic_store(merged, ticket + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        return;  // wave-uniform
    }
    // The last wave: lane r < 8 holds the workgroup's top KL keys of row r.
    if (lane < rows) {
        uint64_t* out = part_keys + (size_t)(row_base + lane) * K * nch + c;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (i < K) out[(size_t)i * nch] = lst[i];
    }
    static_assert(NW == 8 && kRowsPass == 8, "lane 8 r + w: row r, wave w");
    const int r = lane >> 3, w = lane & 7;
    const float2 p = MW[w * kRowsPass + r];
    MaxSum x{p.x, p.y};
    x = ms_dpp_step<kDppQuadXor1>(x);
    x = ms_dpp_step<kDppQuadXor2>(x);
    x = ms_dpp_step<kDppHalfMirror>(x);
    if (w == 0 && r < rows) part_ms[(size_t)(row_base + r) * nch + c] = make_float2(x.m, x.s);
}

// Chunk partials -> candidates.  Partial keys are stored element-major,
// [row][k][chunk], so that threads reading consecutive chunks coalesce.
// lse = M + log S with (M, S) the combined (max, sum of exp), combined in a
// fixed order.
// K > 16 (merge64_kernel, below): the same gather-and-rank with an exact
// threshold.
// K <= 16, nch <= 256 (merge16_kernel): one workgroup of 1024 threads per row.  Thread t owns
// keys 4*(t/256) .. +3 of chunk t%256 (coalesced loads).  The threshold
// theta is the minimum over 16 groups of the group's largest key, the
// groups being 16 consecutive keys of the first 256 partial keys in
// element-major order (the heads of all chunks, then their second entries,
// ...).  The 16 group maxima are distinct real keys >= theta (or theta is 0
// and every key passes), so every key of the row's top K is >= theta.  The
// keys >= theta (a few dozen for ordinary data) are gathered in LDS and each
// is placed by its rank among them (keys are distinct).  If more than
// kCandCap keys pass (massively tied logits), wave 0 merges all the lists
// with bitonic levels instead.  Both give the exact top K.
__global__ __launch_bounds__(1024) void merge16_kernel(const uint64_t* __restrict__ part_keys,
                                                       const float2* __restrict__ part_ms, int nch, int K,
                                                       int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp,
                                                       float* __restrict__ lse_out) {
    __shared__ uint64_t gmax[16];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint64_t fin[16];
    __shared__ float2 wms[4];
    __shared__ int cnt;
    __shared__ uint64_t theta_sh;
    __shared__ float z_sh;
    const int row = blockIdx.x, t = threadIdx.x;
    const int lane = t & (kWave - 1), wave = t / kWave;
    const int c = t & 255, sub = t >> 8;
    const uint64_t* base = part_keys + (size_t)row * K * nch;
    uint64_t k4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * sub + e;
        k4[e] = (c < nch && i < K) ? base[(size_t)i * nch + c] : 0ull;
    }
    if (t == 0) cnt = 0;
    if (sub == 0) {  // waves 0-3: the (max, sum) partials and the first 256 keys
        MaxSum x{-INFINITY, 0.f};
        if (c < nch) {
            const float2 p = part_ms[(size_t)row * nch + c];
            x = MaxSum{p.x, p.y};
        }
        x = wave_ms_reduce(x);
        if (lane == 0) wms[wave] = make_float2(x.m, x.s);
        uint64_t h = t < nch * K ? base[t] : 0ull;
        h = umax64(h, dpp_u64<kDppQuadXor1>(h));
        h = umax64(h, dpp_u64<kDppQuadXor2>(h));
        h = umax64(h, dpp_u64<kDppHalfMirror>(h));
        h = umax64(h, dpp_u64<kDppMirror>(h));
        if ((lane & 15) == 0) gmax[wave * 4 + lane / 16] = h;
    }
    __syncthreads();
    if (t == 0) {
        uint64_t th = gmax[0];
        for (int g = 1; g < 16; ++g) th = umin64(th, gmax[g]);
        theta_sh = th;
        MaxSum zz{-INFINITY, 0.f};
        for (int w = 0; w < 4; ++w) zz = ms_combine(zz, MaxSum{wms[w].x, wms[w].y});
        z_sh = (zz.m == -INFINITY) ? -INFINITY : zz.m + logf(zz.s);
    }
    __syncthreads();
    const uint64_t theta = theta_sh;
    bool pass[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pass[e] = k4[e] >= theta && k4[e] != 0ull;
    // Slots: wave-aggregated offsets from ballots, one LDS atomic per wave.
    const uint64_t lt = (1ull << lane) - 1ull;
    int before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint64_t bal = __ballot(pass[e]);
        before += __popcll(bal & lt);
        total += __popcll(bal);
    }
    int wbase = 0;
    if (lane == 0 && total > 0) wbase = atomicAdd(&cnt, total);
    wbase = __shfl(wbase, 0, kWave);
    __syncthreads();
    const int n = cnt;
    if (n <= kCandCap) {
        int p = wbase + before;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (pass[e]) cand[p++] = k4[e];
        __syncthreads();
        for (int i = t; i < n; i += blockDim.x) {
            const uint64_t key = cand[i];
            int rank = 0;
            for (int j = 0; j < n; ++j) rank += cand[j] > key ? 1 : 0;
            if (rank < K) fin[rank] = key;
        }
    } else if (wave == 0) {
        uint64_t l4[4][16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cc = lane + kWave * j;
#pragma unroll
            for (int i = 0; i < 16; ++i) l4[j][i] = (cc < nch && i < K) ? base[(size_t)i * nch + cc] : 0ull;
        }
        merge_top<16>(l4[0], l4[1]);
        merge_top<16>(l4[2], l4[3]);
        merge_top<16>(l4[0], l4[2]);
        wave_merge_top<16>(l4[0]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) fin[i] = l4[0][i];
        }
    }
    __syncthreads();
    const float z = z_sh;
    if (t < K) {
        const uint64_t key = fin[t];
        cand_ids[(size_t)row * K + t] = key_id(key);
        cand_logp[(size_t)row * K + t] = key_value(key) - z;
    }
    if (t == 0) lse_out[row] = z;
}

// K in 17..64, nch <= 256: one workgroup of 1024 threads per row.  Thread t
// owns keys 16*(t/256) .. +15 of chunk t%256.  The threshold theta is the
// exact K-th largest of the first 256 partial keys in element-major order
// (ranked by counting): at least K keys are >= theta.  The keys >= theta are
// gathered in LDS and ranked; if more than kMergeCap pass (massive ties),
// theta is raised to the exact K-th largest key by bisection over the
// 64-bit key range, after which exactly K keys pass.
constexpr int kMergeCap = 1024;

__global__ __launch_bounds__(1024) void merge64_kernel(const uint64_t* __restrict__ part_keys,
                                                       const float2* __restrict__ part_ms, int nch, int K,
                                                       int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp,
                                                       float* __restrict__ lse_out) {
    __shared__ uint64_t held[256];
    __shared__ uint64_t cand[kMergeCap];
    __shared__ uint64_t fin[64];
    __shared__ float2 wms[4];
    __shared__ int wcnt[16];
    __shared__ int cnt;
    __shared__ uint64_t theta_sh, top_sh;
    __shared__ float z_sh;
    const int row = blockIdx.x, t = threadIdx.x;
    const int lane = t & (kWave - 1), wave = t / kWave;
    const int c = t & 255, sub = t >> 8;
    const uint64_t* base = part_keys + (size_t)row * K * nch;
    uint64_t k16[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = 16 * sub + e;
        k16[e] = (c < nch && i < K) ? base[(size_t)i * nch + c] : 0ull;
    }
    if (t == 0) {
        cnt = 0;
        theta_sh = 0ull;
        top_sh = 0ull;
    }
    if (sub == 0) {  // waves 0-3: the (max, sum) partials and the first 256 keys
        MaxSum x{-INFINITY, 0.f};
        if (c < nch) {
            const float2 p = part_ms[(size_t)row * nch + c];
            x = MaxSum{p.x, p.y};
        }
        x = wave_ms_reduce(x);
        if (lane == 0) wms[wave] = make_float2(x.m, x.s);
        held[t] = t < nch * K ? base[t] : 0ull;
    }
    __syncthreads();
    if (sub == 0) {
        const uint64_t hk = held[t];
        int rank = 0;
        for (int j = 0; j < 256; ++j) rank += held[j] > hk ? 1 : 0;
        if (rank == K - 1 && hk != 0ull) theta_sh = hk;  // fewer than K keys: theta stays 0
        if (rank == 0 && hk != 0ull) top_sh = hk;
    }
    if (t == 0) {
        MaxSum zz{-INFINITY, 0.f};
        for (int w = 0; w < 4; ++w) zz = ms_combine(zz, MaxSum{wms[w].x, wms[w].y});
        z_sh = (zz.m == -INFINITY) ? -INFINITY : zz.m + logf(zz.s);
    }
    __syncthreads();
    uint64_t theta = theta_sh;
    // The row's largest key: the first 256 element-major keys hold every
    // chunk head (nch <= 256), so it is the top-ranked one.
    const uint64_t top = top_sh;
    const uint64_t lt = (1ull << lane) - 1ull;
    int n = 0;
    for (int attempt = 0; attempt < 2; ++attempt) {
        int before = 0, total = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint64_t bal = __ballot(k16[e] >= theta && k16[e] != 0ull);
            before += __popcll(bal & lt);
            total += __popcll(bal);
        }
        int wbase = 0;
        if (lane == 0 && total > 0) wbase = atomicAdd(&cnt, total);
        wbase = __shfl(wbase, 0, kWave);
        __syncthreads();
        n = cnt;
        if (n <= kMergeCap) {
            int p = wbase + before;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (k16[e] >= theta && k16[e] != 0ull) cand[p++] = k16[e];
            break;
        }
        // Too many (massive ties): the exact K-th largest key by bisection;
        // more than kMergeCap >= K keys are >= theta, so it lies in [theta, top].
        uint64_t lo = theta, hi = top;
        while (lo < hi) {
            const uint64_t mid = lo + (hi - lo) / 2 + 1;
            int cc = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) cc += __popcll(__ballot(k16[e] >= mid));
            if (lane == 0) wcnt[wave] = cc;
            __syncthreads();
            int all = 0;
            for (int w = 0; w < 16; ++w) all += wcnt[w];
            __syncthreads();
            if (all >= K) lo = mid;
            else hi = mid - 1;
        }
        theta = lo;
        __syncthreads();  // every thread has read cnt
        if (t == 0) cnt = 0;
        __syncthreads();
    }
    if (n > kMergeCap) n = 0;  // unreachable: exactly K <= kMergeCap keys pass the exact threshold
    __syncthreads();
    for (int i = t; i < n; i += blockDim.x) {
        const uint64_t key = cand[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) rank += cand[j] > key ? 1 : 0;
        if (rank < K) fin[rank] = key;
    }
    for (int i = n + t; i < K; i += blockDim.x) fin[i] = 0ull;
    __syncthreads();
    const float z = z_sh;
    if (t < K) {
        const uint64_t key = fin[t];
        cand_ids[(size_t)row * K + t] = key_id(key);
        cand_logp[(size_t)row * K + t] = key_value(key) - z;
    }
    if (t == 0) lse_out[row] = z;
}

int pick_u(int S) {
    for (int u : {8, 4, 2, 1})
        if (S % u == 0) return u;
    return 1;
}

// K is the number of keys per chunk partial the kernel keeps (<= KL).
template <int NW, int U, int KL>
hipError_t launch_head_bf16_t(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    static_assert(KL == 16, "per-lane lists hold 16 keys");
    const int S = d.D / 32;
    size_t lds = (size_t)S * 4 * kRowsPass * 16;
    const size_t merge = (size_t)kRowsPass * NW * 4 * K * 8 + (size_t)kRowsPass * NW * 4 * 8;
    lds = std::max(std::max(lds, merge), kMinHeadLds);
    auto fn = head_bf16_kernel<NW, U, KL>;
    static LdsAttr attr;
    hipError_t e = ensure_lds(attr, (const void*)fn, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + kRowsPass - 1) / kRowsPass);
    fn<<<grid, NW * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V, nch, K, keys, ms,
                                     logits);
    return hipGetLastError();
}

template <int NW, int KL>
hipError_t launch_head_bf16_u(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    switch (pick_u(d.D / 32)) {
        case 8: return launch_head_bf16_t<NW, 8, KL>(d, K, y, W, nch, keys, ms, logits, s);
        case 4: return launch_head_bf16_t<NW, 4, KL>(d, K, y, W, nch, keys, ms, logits, s);
        case 2: return launch_head_bf16_t<NW, 2, KL>(d, K, y, W, nch, keys, ms, logits, s);
        default: return launch_head_bf16_t<NW, 1, KL>(d, K, y, W, nch, keys, ms, logits, s);
    }
}

template <int NW, int U>
hipError_t launch_head_pair_t(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    const int S = d.D / 64;
    // hidden rows, then the tail's running lists, pairs and counters
    const size_t lds = std::max((size_t)S * 64 * 16 + (size_t)kRowsPass * 16 * 8 + (size_t)NW * kRowsPass * 8 + 16,
                                kMinHeadLds);
    auto fn = head_pair_kernel<NW, U>;
    static LdsAttr attr;
    hipError_t e = ensure_lds(attr, (const void*)fn, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + kRowsPass - 1) / kRowsPass);
    fn<<<grid, NW * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V, nch, K, keys, ms,
                                     logits);
    return hipGetLastError();
}

// Up to 8 rows: the weight-stream kernel (whole-line variant when
// D % 64 == 0), which ranks as it streams.
hipError_t launch_head_stream(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    if (d.D % 64 == 0) {
        const int S = d.D / 64;
        if (S % 8 == 0) return launch_head_pair_t<8, 8>(d, K, y, W, nch, keys, ms, logits, s);
        if (S % 4 == 0) return launch_head_pair_t<8, 4>(d, K, y, W, nch, keys, ms, logits, s);
        if (S % 2 == 0) return launch_head_pair_t<8, 2>(d, K, y, W, nch, keys, ms, logits, s);
        return launch_head_pair_t<8, 1>(d, K, y, W, nch, keys, ms, logits, s);
    }
    return launch_head_bf16_u<16, 16>(d, K, y, W, nch, keys, ms, logits, s);
}

hipError_t launch_merge(const Dims& d, int nch, const uint64_t* keys, const float2* ms, int32_t* cand_ids,
                        float* cand_logp, float* lse, hipStream_t s) {
    if (d.K <= 16)
        merge16_kernel<<<d.rows(), 1024, 0, s>>>(keys, ms, nch, d.K, cand_ids, cand_logp, lse);
    else
        merge64_kernel<<<d.rows(), 1024, 0, s>>>(keys, ms, nch, d.K, cand_ids, cand_logp, lse);
    return hipGetLastError();
}

}  // namespace

int head_chunks(const Dims& d) {
    const int64_t tiles = ((int64_t)d.V + 15) / 16;
    return (int)std::min<int64_t>(256, tiles);
}

WsLayout ws_layout(const Dims& d) {
    WsLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    const size_t rows = (size_t)d.rows(), K = (size_t)d.K, nch = (size_t)head_chunks(d);
    const bool ranks_streaming = d.bf16 && d.K <= 16 && !use_gemm_head(d);
    // the GEMM head writes segment partials that the segment merge reads
    const bool ranks_segments = use_gemm_head(d) && d.K <= 16;
    L.y = take(rows * d.D * (d.bf16 ? 2 : 4));
    L.keys = take(rows * nch * K * 8);  // also what dfs_topk_logits ranks into
    L.ms = take(rows * nch * 8);
    L.logits = take(ranks_streaming ? 0 : rows * (size_t)d.V * 4);
    L.segms = take(ranks_segments ? rows * gemm_seg_geom(d).nseg * 8 : 0);
    L.T = take((size_t)d.batch * (d.B - 1) * K * K * 4);
    L.cids = take(rows * K * 4);
    L.clogp = take(rows * K * 4);
    L.lse = take(rows * 4);
    L.zpart = take(conv_ws_bytes(d));
    L.total = o;
    return L;
}

// Per-chunk partials of the head (keys and (max, sum of exp)); *nparts is
// the number of chunks the merge reads.
hipError_t launch_head_partials(const Dims& d, const void* y, const void* W, float* logits_f32, char* ws,
                                int* nparts, hipStream_t s) {
    const WsLayout L = ws_layout(d);
    uint64_t* keys = (uint64_t*)(ws + L.keys);
    float2* ms = (float2*)(ws + L.ms);
    if (d.bf16 && d.K <= 16 && !use_gemm_head(d)) {
        *nparts = head_chunks(d);
        return launch_head_stream(d, d.K, y, W, *nparts, keys, ms, logits_f32, s);
    }
    float* logits = logits_f32 ? logits_f32 : (float*)(ws + L.logits);
    hipError_t e;
    if (use_gemm_head(d)) {
        e = launch_head_gemm(d, y, W, logits, nullptr, s);
    } else if (d.bf16) {
        // K > 16 on few rows: per-lane register lists of 64 keys would spill,
        // so the streaming kernel also writes the logits and the slice top-K
        // ranks them, overwriting the 16-key partials it leaves behind.
        e = launch_head_stream(d, 16, y, W, head_chunks(d), keys, ms, logits, s);
    } else {
        e = launch_head_f32(d, y, W, logits, s);
    }
    if (e != hipSuccess) return e;
    *nparts = logits_slices(d);
    return launch_logits_partials(d, logits, *nparts, keys, ms, s);
}

hipError_t launch_head_topk(const Dims& d, const void* y, const void* W, int32_t* cand_ids, float* cand_logp,
                            float* lse, float* logits_f32, char* ws, hipStream_t s) {
    if (use_gemm_head(d) && d.K <= 16) {
        const WsLayout L = ws_layout(d);
        float* logits = logits_f32 ? logits_f32 : (float*)(ws + L.logits);
        float2* segms = (float2*)(ws + L.segms);
        hipError_t e = launch_head_gemm(d, y, W, logits, segms, s);
        if (e != hipSuccess) return e;
        return launch_merge_segs(d, logits, segms, cand_ids, cand_logp, lse, s);
    }
    int nparts = 0;
    hipError_t e = launch_head_partials(d, y, W, logits_f32, ws, &nparts, s);
    if (e != hipSuccess) return e;
    const WsLayout L = ws_layout(d);
    return launch_merge(d, nparts, (const uint64_t*)(ws + L.keys), (const float2*)(ws + L.ms), cand_ids, cand_logp,
                        lse, s);
}

hipError_t launch_topk_logits(const Dims& d, const float* logits, int32_t* cand_ids, float* cand_logp, float* lse,
                              char* ws, hipStream_t s) {
    const WsLayout L = ws_layout(d);
    const int nsl = logits_slices(d);
    uint64_t* keys = (uint64_t*)(ws + L.keys);
    float2* ms = (float2*)(ws + L.ms);
    hipError_t e = launch_logits_partials(d, logits, nsl, keys, ms, s);
    if (e != hipSuccess) return e;
    return launch_merge(d, nsl, keys, ms, cand_ids, cand_logp, lse, s);
}

}  // namespace dfs
