// Steps 2-3 of the draft-block path: the vocabulary head (the target's
// shared lm_head), log-softmax and the per-slot top-K candidates (vLLM
// release-note article on DFlash2, section "two additions": keep the target
// head's top-K per slot).  The logits are never written to HBM: the head
// kernel keeps, per vocabulary chunk, each row's top-K keys and its
// (max, sum of exp) pair, and a merge kernel combines the chunks.
//
// bf16 head (rows <= 8 per pass): the work is a stream of the [V, D] weight
// (2.5 GB at D 5120, V 248 320) against a tiny [rows, D] operand, so it is
// bound by HBM.  One persistent workgroup per CU owns a contiguous range of
// 16-row vocabulary tiles; the hidden rows sit in LDS for the whole kernel,
// pre-swizzled into MFMA B-operand order, and every wave streams its tiles
// with v_mfma_f32_16x16x32_bf16 while U k-steps of weight loads (1 KB each)
// are in flight.  The MFMA's 16 output columns hold the (<= 8) rows, so half
// of each MFMA is padding -- harmless, the kernel waits on HBM.  Each lane
// then owns 4 consecutive vocabulary entries of one row per tile and keeps a
// sorted register list of its best keys plus an online (max, sum of exp).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

constexpr int kRowsPass = 8;
constexpr size_t kMinHeadLds = 82 * 1024;  // > 80 KB: one workgroup per CU

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

    const int64_t T = ((int64_t)V + 15) / 16;
    const int t_beg = (int)(T * c / nch), t_end = (int)(T * (c + 1) / nch);
    const int my_n = (t_end - t_beg - wave + NW - 1) / NW;
    const int i16 = lane & 15, q = lane >> 4, jrow = lane & 15;
    const int GPT = S / U;  // k-step groups per tile
    const int total = my_n * GPT;
    const uint4* ysb = (const uint4*)smem + q * kRowsPass + (lane & 7);

    auto tile_ptr = [&](int i) -> const uint16_t* {
        const int tt = t_beg + wave + i * NW;
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
            const int v0 = (t_beg + wave + ti * NW) * 16 + 4 * q;
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
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * kRowsPass;
    const int rows = min(kRowsPass, rows_total - row_base);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int S = D / 64;
    const int i16 = lane & 15, q = lane >> 4;

    const int64_t T = ((int64_t)V + 7) / 8;
    const int t_beg = (int)(T * c / nch), t_end = (int)(T * (c + 1) / nch);
    const int my_n = (t_end - t_beg - wave + NW - 1) / NW;
    const int GPT = S / U;
    const int total = my_n * GPT;
    const int a_off = 32 * (i16 >> 3) + 8 * q;

    auto tile_ptr = [&](int i) -> const uint16_t* {
        const int tt = t_beg + wave + i * NW;
        const int v = min(tt * 8 + (i16 & 7), V - 1);
        return W + (size_t)v * D + a_off;
    };
    auto ldw = [](const uint16_t* p) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)p));
    };

    // The first weight loads do not depend on the hidden rows: issue them
    // before staging those.
    bf16x8 a[U];
    const uint16_t* cur = tile_ptr(0);
    if (total > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = ldw(cur + 64 * u);
    }

    // Hidden rows -> LDS.  16-B unit (s, q, j): row j & 7, channels
    // 64s + 32(j >> 3) + 8q .. +7, so the B operand of k-step s is one
    // contiguous 1 KB read by the 64 lanes.
    {
        uint4* ys = (uint4*)smem;
        for (int u = threadIdx.x; u < S * 64; u += NW * kWave) {
            const int j = u & 15, qq = (u >> 4) & 3, s = u >> 6, row = j & 7;
            uint4 v = {0u, 0u, 0u, 0u};
            if (row < rows) v = *(const uint4*)(y + (size_t)(row_base + row) * D + 64 * s + 32 * (j >> 3) + 8 * qq);
            ys[u] = v;
        }
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
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bf16x8 b = *(const bf16x8*)(ysb + (size_t)(s0 + u) * 64);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b, acc, 0, 0, 0);
            a[u] = ldw(nxt + 64 * u);
        }
        if (ngi == 0) {
            float v4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v4[r] = acc[r] + __shfl(acc[r], (lane + 40) & (kWave - 1), kWave);
            const int v0 = (t_beg + wave + ti * NW) * 8 + 4 * q;
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
    __syncthreads();  // LDS switches from hidden rows to the merge lists

    uint64_t* L = (uint64_t*)smem;                                     // [kRowsPass][NSRC][K]
    float2* M = (float2*)(smem + (size_t)kRowsPass * NSRC * K * 8);  // [kRowsPass][NSRC]
    if (owner) {
        const int src = wave * 2 + q;
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (i < K) L[((size_t)i16 * NSRC + src) * K + i] = lst[i];
        M[i16 * NSRC + src] = make_float2(ms.m, ms.s);
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

// Head for many rows (more than 8 per call, up to 256 per pass): a GEMM
// logit[v][row] = <W[v], y[row]> on v_mfma_f32_32x32x16_bf16 that writes
// the fp32 logits; the slice top-K kernel below ranks them.
//  - One persistent workgroup per CU owns a contiguous vocabulary range and
//    walks it in tiles of 256 rows of W against every hidden row, in stages
//    of KC channels (64 when D % 64 == 0, else 32).
//  - Producer and consumer waves.  NWB consumer waves each own 32 hidden
//    rows and all 256 vocabulary rows of the tile (8 accumulator tiles of
//    32x32); they only read LDS, issue MFMAs and store logits.  Four
//    producer waves move the operands by direct global->LDS loads, two for W
//    (a ring of RW stages) and two for the hidden rows (RY stages; L2
//    resident, so a shallower ring).  A wave's count of outstanding memory
//    operations drains in order for its own loads, so each producer waits on
//    exactly its own stage; one barrier per stage then publishes it.  The
//    consumers' logit stores never sit in front of a load in any wave's
//    count, so they drain while the next tile computes.
//  - The loads are issued from inline assembly: the compiler, unable to tell
//    the ring slots apart, would otherwise wait for every load in flight
//    before each LDS read.
//  - An LDS row holds KC / 8 units of 16 B; unit u of row v is stored at
//    unit u ^ f(v) with f(v) = (v >> 2) & 3 (4 units) or (v >> 1) & 7 (8
//    units), so the 32-row operand reads of a wave hit distinct banks in
//    every group of 16 lanes.
//  - In the 32x32 output layout a lane holds one hidden row and, per tile,
//    4 runs of 4 consecutive vocabulary entries, stored as 16-B writes.
// Ranking inside this kernel (a sorted per-lane list) was tried first: the
// lists of the 64 lanes of a wave take their insertions at different values,
// so the wave ran nearly every insertion and the epilogue cost about a
// quarter of the kernel.  Writing the logits costs a tenth of the weight
// stream and the ranking then runs at the speed of reading them.
constexpr int kGemmTV = 256;

template <int KC>
__device__ __forceinline__ int gemm_swz(int row) {
    return KC == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}
template <int KC>
__device__ __forceinline__ int gemm_unit(int row, int u) {
    return row * (KC / 8) + (u ^ gemm_swz<KC>(row));
}

// 16-B global -> LDS copy per lane; lane L writes lds_base + 16 L.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(g)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

constexpr int kGemmProducers = 4;  // two W loaders, two hidden-row loaders

// s_waitcnt with at most n vector-memory operations outstanding (n a
// multiple of 4 up to 48: the counts the producers use).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define DFS_WAIT_VM(k)                                                                          \
    case k:                                                                                     \
        __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | ((k) & 0xF) | (((k) >> 4) << 14)); \
        break;
        DFS_WAIT_VM(4) DFS_WAIT_VM(8) DFS_WAIT_VM(12) DFS_WAIT_VM(16) DFS_WAIT_VM(20) DFS_WAIT_VM(24)
        DFS_WAIT_VM(28) DFS_WAIT_VM(32) DFS_WAIT_VM(36) DFS_WAIT_VM(40) DFS_WAIT_VM(44) DFS_WAIT_VM(48)
#undef DFS_WAIT_VM
        default:
            __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4));
            break;
    }
}

template <int NWB, int KC, int RW, int RY>
__global__ __launch_bounds__((NWB + kGemmProducers) * kWave) void head_gemm_kernel(
    const uint16_t* __restrict__ y, int rows_total, int D, const uint16_t* __restrict__ W, int V, int nch,
    float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int RP = 32 * NWB;
    constexpr int UPR = KC / 8;                 // 16-B units per LDS row
    constexpr int RPI = kWave / UPR;            // rows per 1-KB load instruction
    constexpr int WBYTES = kGemmTV * KC * 2;    // one W stage
    constexpr int YBYTES = RP * KC * 2;         // one hidden-row stage
    constexpr int WI = WBYTES / 1024 / 2;       // load instructions per W producer per stage
    constexpr int YI = YBYTES / 1024 / 2;       // per hidden-row producer per stage
    static_assert(WI * 2048 == WBYTES && YI * 2048 == YBYTES, "whole load instructions per producer");
    static_assert((RW - 2) * WI <= 48 && (RW - 2) * WI % 4 == 0 && (RY - 2) * YI <= 48 && (RY - 2) * YI % 4 == 0,
                  "wait counts");
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * RP;
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = D / KC;
    const int64_t T32 = ((int64_t)V + 31) / 32;
    const int b_beg = (int)(T32 * c / nch), b_end = (int)(T32 * (c + 1) / nch);
    const int v_beg = b_beg * 32, v_end = min(b_end * 32, V);
    const int ntiles = (b_end - b_beg + 7) / 8;
    const int total = ntiles * S;
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    const uint32_t ybase = smem_base + RW * WBYTES;

    if (wave >= NWB) {
        // Producers.  Stage g (tile g / S, channel block g % S) goes to slot
        // g % RW (W) or g % RY (hidden rows).  A 1-KB load instruction covers
        // RPI rows x 2 KC bytes; lane L takes row L / UPR, stored unit
        // L % UPR, i.e. logical unit (L % UPR) ^ f(row).
        const bool wl = wave < NWB + 2;
        const int pw = wl ? wave - NWB : wave - NWB - 2;
        auto issue_w = [&](int g) {
            const int k0 = (g % S) * KC, v0 = v_beg + (g / S) * kGemmTV;
            const uint32_t base = smem_base + (uint32_t)((g % RW) * WBYTES);
#pragma unroll
            for (int i = 0; i < WI; ++i) {
                const int n = pw + 2 * i;
                const int vr = RPI * n + lane / UPR;
                const int u = (lane % UPR) ^ gemm_swz<KC>(vr);
                const int v = min(v0 + vr, v_end - 1);  // past the range: re-read its last row (cache hit)
                dma16(W + (size_t)v * D + k0 + 8 * u, base + n * 1024);
            }
        };
        auto issue_y = [&](int g) {
            const int k0 = (g % S) * KC;
            const uint32_t base = ybase + (uint32_t)((g % RY) * YBYTES);
#pragma unroll
            for (int i = 0; i < YI; ++i) {
                const int n = pw + 2 * i;
                const int r = RPI * n + lane / UPR;
                const int u = (lane % UPR) ^ gemm_swz<KC>(r);
                const int row = min(row_base + r, rows_total - 1);
                dma16(y + (size_t)row * D + k0 + 8 * u, base + n * 1024);
            }
        };
        const int R = wl ? RW : RY, per = wl ? WI : YI;
        for (int g = 0; g < R - 1 && g < total; ++g) wl ? issue_w(g) : issue_y(g);
        for (int g = 0; g < total; ++g) {
            // stage g landed: at most the later stages' loads outstanding
            wait_vm(min(R - 2, total - 1 - g) * per);
            __syncthreads();  // publish stage g; the slot read in stage g - 1 is free
            if (g + R - 1 < total) wl ? issue_w(g + R - 1) : issue_y(g + R - 1);
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // Consumers.
    const int j = lane & 31, half = lane >> 5;
    const int rl = wave * 32 + j;
    const int my_row = row_base + rl;
    const bool row_ok = my_row < rows_total;
    const bool vec4 = (V & 3) == 0;  // rows of the logits are 16-B aligned
    f32x16 acc[8];
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[vb][r] = 0.f;
    int tile = 0, st = 0;
    for (int g = 0; g < total; ++g) {
        __syncthreads();  // stage g published
        const uint4* sw = (const uint4*)(smem + (size_t)(g % RW) * WBYTES);
        const uint4* sy = (const uint4*)(smem + (size_t)RW * WBYTES + (size_t)(g % RY) * YBYTES);
#pragma unroll
        for (int ks = 0; ks < KC / 16; ++ks) {
            const int u = 2 * ks + half;
            const bf16x8 b = __builtin_bit_cast(bf16x8, sy[gemm_unit<KC>(rl, u)]);
            // Rows past the range hold copies of its last row; their results
            // are dropped below.
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, sw[gemm_unit<KC>(vb * 32 + j, u)]);
                acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[vb], 0, 0, 0);
            }
        }
        if (st == S - 1) {
            // Tile done.  Lane holds, for vocabulary block vb, logit[v][my_row]
            // in acc[vb][r] with v = base + 32 vb + 8 (r / 4) + 4 half + r % 4.
            const int vt = v_beg + tile * kGemmTV;
            if (row_ok) {
                float* out = logits + (size_t)my_row * V;
#pragma unroll
                for (int vb = 0; vb < 8; ++vb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int v = vt + 32 * vb + 8 * q + 4 * half;
                        if (vec4 && v + 3 < v_end) {
                            *(f32x4*)(out + v) = f32x4{acc[vb][4 * q], acc[vb][4 * q + 1], acc[vb][4 * q + 2],
                                                       acc[vb][4 * q + 3]};
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (v + e < v_end) out[v + e] = acc[vb][4 * q + e];
                        }
                    }
                }
            }
#pragma unroll
            for (int vb = 0; vb < 8; ++vb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[vb][r] = 0.f;
            ++tile;
            st = 0;
        } else {
            ++st;
        }
    }
}

// fp32 correctness path: plain dot products, logits written out.
__global__ __launch_bounds__(256) void head_f32_kernel(const float* __restrict__ y, const float* __restrict__ W,
                                                       float* __restrict__ logits, int rows, int D, int V) {
    const int v = blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= V) return;
    for (int row = 0; row < rows; ++row) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += y[(size_t)row * D + c] * W[(size_t)v * D + c];
        logits[(size_t)row * V + v] = acc;
    }
}

// Top-K keys and (max, sum of exp) of one slice of one row of fp32 logits;
// one workgroup of 512 threads per (slice, row), K <= 64, two workgroups per
// CU so that one loads while the other ranks.
//  - Thread t holds 32 values of the slice in registers: with 16-B aligned
//    rows (V % 4 == 0) the 4-value units t, t + 512, ..., else the values
//    t, t + 512, ...  Consecutive threads read consecutive addresses.
//  - Every 8-lane group takes the largest key of its values: 64 group
//    maxima, distinct keys unless 0 (an empty group).  Their K-th largest,
//    theta, has at least K keys >= theta in the slice, so every key of the
//    slice's top K is >= theta; for ordinary data a few dozen keys pass.
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
__global__ __launch_bounds__(kSliceThreads, 4) void slice_topk_kernel(const float* __restrict__ logits, int V,
                                                                      int nsl, int K, uint64_t* __restrict__ part_keys,
                                                                      float2* __restrict__ part_ms) {
    constexpr int NWV = kSliceThreads / kWave;
    __shared__ uint64_t gmax[64];
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
    if (t < 64) {
        const uint64_t g = gmax[t];
        int rank = 0;
        for (int i = 0; i < 64; ++i) rank += gmax[i] > g ? 1 : 0;
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

// Chunk partials -> candidates.  Partial keys are stored element-major,
// [row][k][chunk], so that threads reading consecutive chunks coalesce.
//  K <= 64: one workgroup (4 waves) per row: a K-round tournament per wave
//    over its 64 chunk lists, then over the 4 wave lists.
// lse = M + log S with (M, S) the combined (max, sum of exp), combined in a
// fixed order.
// K <= 16, nch <= 256: one workgroup of 1024 threads per row.  Thread t owns
// keys 4*(t/256) .. +3 of chunk t%256 (coalesced loads).  The threshold
// theta is the K-th largest of the first 256 partial keys (in element-major
// order: the heads of all chunks, then their second entries, ...), found by
// ranking them; at least K keys are >= theta, so every key of the row's top
// K is.  The keys >= theta (a few dozen for ordinary data) are gathered in
// LDS and each is placed by its rank among them (keys are distinct).  If
// more than kCandCap keys pass (massively tied logits), wave 0 merges all
// the lists with bitonic levels instead.  Both give the exact top K.
__global__ __launch_bounds__(1024) void merge16_kernel(const uint64_t* __restrict__ part_keys,
                                                       const float2* __restrict__ part_ms, int nch, int K,
                                                       int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp,
                                                       float* __restrict__ lse_out) {
    __shared__ uint64_t held[256];
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
    if (t == 0) {
        cnt = 0;
        theta_sh = 0ull;
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
        const uint64_t h = held[t];
        int rank = 0;
        for (int j = 0; j < 256; ++j) rank += held[j] > h ? 1 : 0;
        if (rank == K - 1 && h != 0ull) theta_sh = h;  // fewer than K keys: theta stays 0
    }
    if (t == 0) {
        MaxSum zz{-INFINITY, 0.f};
        for (int w = 0; w < 4; ++w) zz = ms_combine(zz, MaxSum{wms[w].x, wms[w].y});
        z_sh = (zz.m == -INFINITY) ? -INFINITY : zz.m + logf(zz.s);
    }
    __syncthreads();
    const uint64_t theta = theta_sh;
    bool pass[4];
    int mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pass[e] = k4[e] >= theta && k4[e] != 0ull;
        mine += pass[e] ? 1 : 0;
    }
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

__global__ __launch_bounds__(256) void merge64_kernel(const uint64_t* __restrict__ part_keys,
                                                      const float2* __restrict__ part_ms, int nch, int K,
                                                      int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp,
                                                      float* __restrict__ lse_out) {
    constexpr int KL = 64;
    __shared__ uint64_t tops[4][KL + 1];
    __shared__ uint64_t fin[KL];
    __shared__ float2 wms[4];
    __shared__ float zsh;
    const int row = blockIdx.x, t = threadIdx.x;
    const int lane = t & (kWave - 1), wave = t / kWave;
    const bool have = t < nch;
    const uint64_t* src = part_keys + (size_t)row * K * nch + (have ? t : 0);
    uint64_t lst[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) lst[i] = (have && i < K) ? src[(size_t)i * nch] : 0ull;
    MaxSum x{-INFINITY, 0.f};
    if (have) {
        const float2 p = part_ms[(size_t)row * nch + t];
        x = MaxSum{p.x, p.y};
    }
    x = wave_ms_reduce(x);
    if (lane == 0) wms[wave] = make_float2(x.m, x.s);
    for (int round = 0; round < K; ++round) {
        const uint64_t mx = wave_max_u64(lst[0]);
        if (lst[0] == mx && mx != 0ull) {
#pragma unroll
            for (int i = 0; i < KL - 1; ++i) lst[i] = lst[i + 1];
            lst[KL - 1] = 0ull;
        }
        if (lane == 0) tops[wave][round] = mx;
    }
    __syncthreads();
    if (wave == 0) wave_tournament(&tops[0][0], 4, KL + 1, K, K, fin);
    if (t == 0) {
        MaxSum zz{-INFINITY, 0.f};
        for (int w = 0; w < 4; ++w) zz = ms_combine(zz, MaxSum{wms[w].x, wms[w].y});
        zsh = (zz.m == -INFINITY) ? -INFINITY : zz.m + logf(zz.s);
    }
    __syncthreads();
    const float z = zsh;
    for (int k = t; k < K; k += blockDim.x) {
        const uint64_t key = fin[k];
        cand_ids[(size_t)row * K + k] = key_id(key);
        cand_logp[(size_t)row * K + k] = key_value(key) - z;
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
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
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
    size_t lds = (size_t)S * 64 * 16;
    const size_t merge = (size_t)kRowsPass * NW * 2 * K * 8 + (size_t)kRowsPass * NW * 2 * 8;
    lds = std::max(std::max(lds, merge), kMinHeadLds);
    auto fn = head_pair_kernel<NW, U>;
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + kRowsPass - 1) / kRowsPass);
    fn<<<grid, NW * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V, nch, K, keys, ms,
                                     logits);
    return hipGetLastError();
}

template <int NWB, int KC, int RW, int RY>
hipError_t launch_head_gemm_t(const Dims& d, const void* y, const void* W, int nch, float* logits, hipStream_t s) {
    constexpr int RP = 32 * NWB;
    constexpr size_t lds = ((size_t)RW * kGemmTV + (size_t)RY * RP) * KC * 2;
    static_assert(lds <= 160 * 1024, "the stage rings must fit in LDS");
    auto fn = head_gemm_kernel<NWB, KC, RW, RY>;
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + RP - 1) / RP);
    fn<<<grid, (NWB + kGemmProducers) * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V,
                                                         nch, logits);
    return hipGetLastError();
}

// More than 8 rows: one pass of the GEMM head per 256 rows instead of one
// weight stream per 8 rows.  Writes the logits.
bool use_gemm_head(const Dims& d) { return d.bf16 && d.rows() > kRowsPass; }

hipError_t launch_head_gemm(const Dims& d, const void* y, const void* W, float* logits, hipStream_t s) {
    const int nch = head_chunks(d);
    if (d.D % 64 == 0)
        return d.rows() <= 128 ? launch_head_gemm_t<4, 64, 3, 2>(d, y, W, nch, logits, s)
                               : launch_head_gemm_t<8, 64, 3, 2>(d, y, W, nch, logits, s);
    return d.rows() <= 128 ? launch_head_gemm_t<4, 32, 6, 4>(d, y, W, nch, logits, s)
                           : launch_head_gemm_t<8, 32, 6, 4>(d, y, W, nch, logits, s);
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
        merge64_kernel<<<d.rows(), 256, 0, s>>>(keys, ms, nch, d.K, cand_ids, cand_logp, lse);
    return hipGetLastError();
}

// Slices of the logits ranked per row: at most kSliceLen values each, at
// most 256 (the partial buffer's chunk count), and enough (slice, row)
// workgroups to fill the chip when there are few rows.
int logits_slices(const Dims& d) {
    const int64_t need = ((int64_t)d.V + kSliceLen - 1) / kSliceLen;
    const int64_t fill = (2048 + d.rows() - 1) / d.rows();
    const int64_t most = std::min<int64_t>(256, ((int64_t)d.V + kSliceThreads - 1) / kSliceThreads);
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
    L.y = take(rows * d.D * (d.bf16 ? 2 : 4));
    L.keys = take(rows * nch * K * 8);
    L.ms = take(rows * nch * 8);
    L.logits = take(ranks_streaming ? 0 : rows * (size_t)d.V * 4);
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
        e = launch_head_gemm(d, y, W, logits, s);
    } else if (d.bf16) {
        // K > 16 on few rows: per-lane register lists of 64 keys would spill,
        // so the streaming kernel also writes the logits and the slice top-K
        // ranks them, overwriting the 16-key partials it leaves behind.
        e = launch_head_stream(d, 16, y, W, head_chunks(d), keys, ms, logits, s);
    } else {
        head_f32_kernel<<<(d.V + 255) / 256, 256, 0, s>>>((const float*)y, (const float*)W, logits, d.rows(), d.D,
                                                          d.V);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    *nparts = logits_slices(d);
    return launch_logits_partials(d, logits, *nparts, keys, ms, s);
}

hipError_t launch_head_topk(const Dims& d, const void* y, const void* W, int32_t* cand_ids, float* cand_logp,
                            float* lse, float* logits_f32, char* ws, hipStream_t s) {
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
