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
// logit[v][row] = <W[v], y[row]> on v_mfma_f32_32x32x16_bf16 with the same
// fused per-chunk top-K and (max, sum of exp) as the streaming head.
//  - One persistent workgroup per CU owns a contiguous vocabulary range and
//    walks it in tiles of 256 rows of W against every hidden row.
//  - Both operands arrive in 32-channel stages (W: 256 rows x 64 B, hidden
//    rows: up to 256 x 64 B) by direct global->LDS loads into a four-stage
//    LDS ring, three stages ahead of the MFMAs, without staging registers.
//    Those loads are the only vector-memory operations of the main loop, so
//    a fixed count of outstanding operations says when a stage has landed.
//    They are issued from inline assembly: the compiler, unable to tell the
//    ring slots apart, would otherwise wait for every load in flight before
//    each LDS read.
//  - LDS rows are 64 B (4 units of 16 B); unit u of row v is stored at unit
//    u ^ ((v >> 2) & 3), so the 32-row operand reads of a wave hit distinct
//    banks in every group of 16 lanes.
//  - Wave w owns hidden rows 32w .. 32w+31 and all 256 vocabulary rows of
//    the tile: 8 accumulator tiles of 32x32.  In that output layout a lane
//    holds one hidden row (column l % 32) and 16 vocabulary entries per tile,
//    so each lane keeps a sorted register list of its best keys and an online
//    (max, sum of exp) for its row; the logits never leave registers.  At the
//    end the two lanes of every row are merged into the chunk's partial.
constexpr int kGemmTV = 256;
constexpr int kGemmKC = 32;
constexpr int kGemmRing = 4;
constexpr int kGemmWBytes = kGemmTV * kGemmKC * 2;  // 16 KB of W per stage

__device__ __forceinline__ int gemm_unit(int row, int u) { return row * 4 + (u ^ ((row >> 2) & 3)); }

// 16-B global -> LDS copy per lane; lane L writes lds_base + 16 L.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds_base)),
                 "v"(g)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

template <int NWB>
__global__ __launch_bounds__(NWB * kWave) void head_gemm_kernel(
    const uint16_t* __restrict__ y, int rows_total, int D, const uint16_t* __restrict__ W, int V, int nch, int K,
    uint64_t* __restrict__ part_keys, float2* __restrict__ part_ms, float* __restrict__ logits) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int RP = 32 * NWB;
    constexpr int KL = 16;
    constexpr int YBYTES = RP * kGemmKC * 2;
    constexpr int STAGE = kGemmWBytes + YBYTES;
    constexpr int WI = kGemmWBytes / 1024 / NWB;  // W load instructions per wave per stage
    constexpr int YI = YBYTES / 1024 / NWB;       // hidden-row load instructions per wave per stage
    constexpr int OPS = WI + YI;                  // vector-memory operations per wave per stage
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * RP;
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int j = lane & 31, half = lane >> 5;
    const int rl = wave * 32 + j;
    const int my_row = row_base + rl;
    const bool row_ok = my_row < rows_total;
    const int S = D / kGemmKC;

    const int64_t T32 = ((int64_t)V + 31) / 32;
    const int b_beg = (int)(T32 * c / nch), b_end = (int)(T32 * (c + 1) / nch);
    const int v_beg = b_beg * 32, v_end = min(b_end * 32, V);
    const int ntiles = (b_end - b_beg + 7) / 8;
    const int total = ntiles * S;
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

    // Stage g (tile g / S, channels 32 (g % S) ..) into ring slot g % 4.  A
    // 1 KB load instruction covers 16 rows x 64 B; lane L takes row L / 4,
    // stored unit L % 4, i.e. logical unit (L % 4) ^ ((row >> 2) & 3).
    auto issue_stage = [&](int g) {
        const int tile = g / S, k0 = (g % S) * kGemmKC;
        const uint32_t base = smem_base + (uint32_t)((g % kGemmRing) * STAGE);
        const int v0 = v_beg + tile * kGemmTV;
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int n = wave + i * NWB;
            const int vr = 16 * n + (lane >> 2);
            const int u = (lane & 3) ^ ((vr >> 2) & 3);
            const int v = min(v0 + vr, v_end - 1);  // past the range: re-read its last row (cache hit)
            dma16(W + (size_t)v * D + k0 + 8 * u, base + n * 1024);
        }
#pragma unroll
        for (int i = 0; i < YI; ++i) {
            const int n = wave + i * NWB;
            const int r = 16 * n + (lane >> 2);
            const int u = (lane & 3) ^ ((r >> 2) & 3);
            const int row = min(row_base + r, rows_total - 1);
            dma16(y + (size_t)row * D + k0 + 8 * u, base + kGemmWBytes + n * 1024);
        }
    };
    // Wait until this wave's loads of stage g have landed, given that the
    // stages up to g + 2 were issued after it (fewer near the end).
    auto wait_stage = [&](int g) {
        if (g + 2 < total)
            __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | ((2 * OPS) & 0xF) | (((2 * OPS) >> 4) << 14));
        else if (g + 1 < total)
            __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | (OPS & 0xF) | ((OPS >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4));
    };

    f32x16 acc[8];
#pragma unroll
    for (int vb = 0; vb < 8; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[vb][r] = 0.f;
    uint64_t lst[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) lst[i] = 0ull;
    MaxSum ms{-INFINITY, 0.f};

    for (int g = 0; g < kGemmRing - 1 && g < total; ++g) issue_stage(g);
    int tile = 0, st = 0;
    for (int g = 0; g < total; ++g) {
        wait_stage(g);
        __syncthreads();  // stage g complete for every wave; slot (g - 1) % 4 free
        if (g + kGemmRing - 1 < total) issue_stage(g + kGemmRing - 1);
        const uint4* sw = (const uint4*)(smem + (size_t)(g % kGemmRing) * STAGE);
        const uint4* sy = (const uint4*)(smem + (size_t)(g % kGemmRing) * STAGE + kGemmWBytes);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int u = 2 * ks + half;
            const bf16x8 b = __builtin_bit_cast(bf16x8, sy[gemm_unit(rl, u)]);
            // Rows past the range hold copies of its last row; their results
            // are dropped below.
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, sw[gemm_unit(vb * 32 + j, u)]);
                acc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[vb], 0, 0, 0);
            }
        }
        if (st == S - 1) {
            // Tile done.  Lane holds, for vocabulary block vb, logit[v][my_row]
            // in acc[vb][r] with v = base + 32 vb + 8 (r / 4) + 4 half + r % 4.
            const int vt = v_beg + tile * kGemmTV;
            const int nvb = min(8, b_end - (b_beg + 8 * tile));
            if (row_ok) {
#pragma unroll
                for (int vb = 0; vb < 8; ++vb) {
                    if (vb < nvb) {
                        float mnew = ms.m;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int v = vt + 32 * vb + 8 * (r >> 2) + 4 * half + (r & 3);
                            if (v < v_end) mnew = fmaxf(mnew, acc[vb][r]);
                        }
                        float sacc = (ms.m == -INFINITY) ? 0.f : ms.s * __expf(ms.m - mnew);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int v = vt + 32 * vb + 8 * (r >> 2) + 4 * half + (r & 3);
                            if (v < v_end) {
                                const float x = acc[vb][r];
                                sacc += __expf(x - mnew);
                                const uint64_t key = make_key(x, (uint32_t)v);
                                if (key > lst[KL - 1]) list_insert<KL>(lst, key);
                                if (logits) logits[(size_t)my_row * V + v] = x;
                            }
                        }
                        ms = MaxSum{mnew, sacc};
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
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every read of the ring done before it holds the lists

    // The two lanes of each row -> the chunk's partial.
    uint64_t* Lm = (uint64_t*)smem;                                // [RP][2][K]
    float2* Mm = (float2*)(smem + (size_t)RP * 2 * K * 8);       // [RP][2]
    if (row_ok) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
            if (i < K) Lm[((size_t)rl * 2 + half) * K + i] = lst[i];
        Mm[rl * 2 + half] = make_float2(ms.m, ms.s);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < RP; r += NWB * kWave) {
        const int row = row_base + r;
        if (row >= rows_total) continue;
        const uint64_t* a = Lm + (size_t)r * 2 * K;
        const uint64_t* b = a + K;
        int ia = 0, ib = 0;
        uint64_t* out = part_keys + (size_t)row * K * nch + c;
        for (int i = 0; i < K; ++i) {
            const uint64_t ka = a[ia], kb = b[ib];
            if (ka >= kb) {
                out[(size_t)i * nch] = ka;
                ++ia;
            } else {
                out[(size_t)i * nch] = kb;
                ++ib;
            }
        }
        const float2 m0 = Mm[r * 2], m1 = Mm[r * 2 + 1];
        const MaxSum z = ms_combine(MaxSum{m0.x, m0.y}, MaxSum{m1.x, m1.y});
        part_ms[(size_t)row * nch + c] = make_float2(z.m, z.s);
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

// Top-K keys and (max, sum of exp) of one chunk of one row of given logits;
// one wave per (chunk, row).
template <int KL>
__global__ __launch_bounds__(kWave) void logits_partial_kernel(const float* __restrict__ logits, int V, int nch, int K,
                                                               uint64_t* __restrict__ part_keys,
                                                               float2* __restrict__ part_ms) {
    extern __shared__ uint64_t lsm[];  // [64][K]
    const int c = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
    const int v_beg = (int)((int64_t)V * c / nch), v_end = (int)((int64_t)V * (c + 1) / nch);
    uint64_t lst[KL];
#pragma unroll
    for (int i = 0; i < KL; ++i) lst[i] = 0ull;
    MaxSum ms{-INFINITY, 0.f};
    for (int v = v_beg + lane; v < v_end; v += kWave) {
        const float x = logits[(size_t)row * V + v];
        ms = ms_combine(ms, MaxSum{x, 1.f});
        const uint64_t key = make_key(x, (uint32_t)v);
        if (key > lst[KL - 1]) list_insert<KL>(lst, key);
    }
#pragma unroll
    for (int i = 0; i < KL; ++i)
        if (i < K) lsm[lane * K + i] = lst[i];
    __syncthreads();
    wave_tournament(lsm, kWave, K, K, K, part_keys + (size_t)row * K * nch + c, nch);
    ms = wave_ms_reduce(ms);
    if (lane == 0) part_ms[(size_t)row * nch + c] = make_float2(ms.m, ms.s);
}

// Chunk partials -> candidates.  Partial keys are stored element-major,
// [row][k][chunk], so that threads reading consecutive chunks coalesce.
//  K <= 64: one workgroup (4 waves) per row: a K-round tournament per wave
//    over its 64 chunk lists, then over the 4 wave lists.
// lse = M + log S with (M, S) the combined (max, sum of exp), combined in a
// fixed order.
// K <= 16, nch <= 256: one workgroup of 1024 threads per row.  Thread t owns
// keys 4*(t/256) .. +3 of chunk t%256 (coalesced loads).  A threshold theta
// with at least 16 real keys >= theta is the minimum over 16 groups of 16
// chunks of the group's largest chunk head; every key of the row's top K is
// >= theta.  The keys >= theta (a few dozen for ordinary data) are gathered
// in LDS and each is placed by its rank among them (keys are distinct).  If
// more than kCandCap keys pass (massively tied logits), wave 0 merges all
// the lists with bitonic levels instead.  Both give the exact top K.
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
    if (sub == 0) {  // waves 0-3 hold the chunk heads (key 0 of every chunk)
        MaxSum x{-INFINITY, 0.f};
        if (c < nch) {
            const float2 p = part_ms[(size_t)row * nch + c];
            x = MaxSum{p.x, p.y};
        }
        x = wave_ms_reduce(x);
        if (lane == 0) wms[wave] = make_float2(x.m, x.s);
        uint64_t h = k4[0];
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

template <int NWB>
hipError_t launch_head_gemm_t(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    constexpr int RP = 32 * NWB;
    constexpr size_t ring = (size_t)kGemmRing * (kGemmWBytes + RP * kGemmKC * 2);
    static_assert(ring <= 160 * 1024, "the stage ring must fit in LDS");
    const size_t lds = std::max(ring, (size_t)RP * 2 * K * 8 + (size_t)RP * 2 * 8);
    auto fn = head_gemm_kernel<NWB>;
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + RP - 1) / RP);
    fn<<<grid, NWB * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V, nch, K, keys, ms,
                                      logits);
    return hipGetLastError();
}

// Head dispatch.  Rows <= 8: the weight-stream kernel (whole-line variant
// when D % 64 == 0).  More rows: the GEMM head.
hipError_t launch_head_stream(const Dims& d, int K, const void* y, const void* W, int nch, uint64_t* keys,
                              float2* ms, float* logits, hipStream_t s) {
    if (d.rows() > 8 && d.D % kGemmKC == 0) {
        // many rows: one pass of the GEMM head per 256 rows instead of one
        // weight stream per 8 rows
        return d.rows() <= 128 ? launch_head_gemm_t<4>(d, K, y, W, nch, keys, ms, logits, s)
                               : launch_head_gemm_t<8>(d, K, y, W, nch, keys, ms, logits, s);
    }
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

hipError_t launch_logits_partials(const Dims& d, const float* logits, int nch, uint64_t* keys, float2* ms,
                                  hipStream_t s) {
    dim3 grid(nch, d.rows());
    const size_t lds = (size_t)kWave * d.K * 8;
    if (d.K <= 16)
        logits_partial_kernel<16><<<grid, kWave, lds, s>>>(logits, d.V, nch, d.K, keys, ms);
    else
        logits_partial_kernel<64><<<grid, kWave, lds, s>>>(logits, d.V, nch, d.K, keys, ms);
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
    L.y = take(rows * d.D * (d.bf16 ? 2 : 4));
    L.keys = take(rows * nch * K * 8);
    L.ms = take(rows * nch * 8);
    L.logits = take((d.bf16 && d.K <= 16) ? 0 : rows * (size_t)d.V * 4);
    L.T = take((size_t)d.batch * (d.B - 1) * K * K * 4);
    L.cids = take(rows * K * 4);
    L.clogp = take(rows * K * 4);
    L.lse = take(rows * 4);
    L.zpart = take(conv_ws_bytes(d));
    L.total = o;
    return L;
}

hipError_t launch_head_partials(const Dims& d, const void* y, const void* W, float* logits_f32, char* ws,
                                hipStream_t s) {
    const WsLayout L = ws_layout(d);
    const int nch = head_chunks(d);
    uint64_t* keys = (uint64_t*)(ws + L.keys);
    float2* ms = (float2*)(ws + L.ms);
    if (d.bf16 && d.K <= 16) return launch_head_stream(d, d.K, y, W, nch, keys, ms, logits_f32, s);
    float* logits = logits_f32 ? logits_f32 : (float*)(ws + L.logits);
    hipError_t e;
    if (d.bf16) {
        // K > 16: per-lane register lists of 64 keys would spill, so the
        // logits are written out and ranked by the logits top-K kernel, which
        // overwrites the (16-key) partials the head kernel leaves behind.
        e = launch_head_stream(d, 16, y, W, nch, keys, ms, logits, s);
    } else {
        head_f32_kernel<<<(d.V + 255) / 256, 256, 0, s>>>((const float*)y, (const float*)W, logits, d.rows(), d.D,
                                                          d.V);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    return launch_logits_partials(d, logits, nch, keys, ms, s);
}

hipError_t launch_head_topk(const Dims& d, const void* y, const void* W, int32_t* cand_ids, float* cand_logp,
                            float* lse, float* logits_f32, char* ws, hipStream_t s) {
    hipError_t e = launch_head_partials(d, y, W, logits_f32, ws, s);
    if (e != hipSuccess) return e;
    const WsLayout L = ws_layout(d);
    return launch_merge(d, head_chunks(d), (const uint64_t*)(ws + L.keys), (const float2*)(ws + L.ms), cand_ids,
                        cand_logp, lse, s);
}

hipError_t launch_topk_logits(const Dims& d, const float* logits, int32_t* cand_ids, float* cand_logp, float* lse,
                              char* ws, hipStream_t s) {
    const WsLayout L = ws_layout(d);
    const int nch = head_chunks(d);
    uint64_t* keys = (uint64_t*)(ws + L.keys);
    float2* ms = (float2*)(ws + L.ms);
    hipError_t e = launch_logits_partials(d, logits, nch, keys, ms, s);
    if (e != hipSuccess) return e;
    return launch_merge(d, nch, keys, ms, cand_ids, cand_logp, lse, s);
}

}  // namespace dfs
