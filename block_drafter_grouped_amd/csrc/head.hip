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
        wave_tournament(L + (size_t)jr * NSRC * K, NSRC, K, K, K,
                        part_keys + ((size_t)(row_base + jr) * nch + c) * K);
        MaxSum x{-INFINITY, 0.f};
        if (lane < NSRC) {
            const float2 p = M[jr * NSRC + lane];
            x = MaxSum{p.x, p.y};
        }
        x = wave_ms_reduce(x);
        if (lane == 0) part_ms[(size_t)(row_base + jr) * nch + c] = make_float2(x.m, x.s);
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
    wave_tournament(lsm, kWave, K, K, K, part_keys + ((size_t)row * nch + c) * K);
    ms = wave_ms_reduce(ms);
    if (lane == 0) part_ms[(size_t)row * nch + c] = make_float2(ms.m, ms.s);
}

// Chunk partials -> candidates.  One workgroup (4 waves) per row: each wave
// merges up to 64 chunk lists, then wave 0 merges the 4 wave lists.
// lse = M + log S with (M, S) the combined (max, sum of exp).
__global__ __launch_bounds__(256) void merge_kernel(const uint64_t* __restrict__ part_keys,
                                                    const float2* __restrict__ part_ms, int nch, int K,
                                                    int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp,
                                                    float* __restrict__ lse_out) {
    extern __shared__ uint64_t sk[];  // [nch][K] then [4][K]
    __shared__ float2 wms[4];
    __shared__ uint64_t fin[64];
    __shared__ float zsh;
    const int row = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint64_t* src = part_keys + (size_t)row * nch * K;
    for (int i = threadIdx.x; i < nch * K; i += blockDim.x) sk[i] = src[i];
    MaxSum x{-INFINITY, 0.f};
    for (int i = threadIdx.x; i < nch; i += blockDim.x) {
        const float2 p = part_ms[(size_t)row * nch + i];
        x = ms_combine(x, MaxSum{p.x, p.y});
    }
    x = wave_ms_reduce(x);
    if (lane == 0) wms[wave] = make_float2(x.m, x.s);
    __syncthreads();
    uint64_t* tops = sk + (size_t)nch * K;
    const int first = wave * kWave;
    const int n = max(0, min(kWave, nch - first));
    wave_tournament(sk + (size_t)first * K, n, K, K, K, tops + wave * K);
    __syncthreads();
    if (wave == 0) wave_tournament(tops, 4, K, K, K, fin);
    if (threadIdx.x == 0) {
        MaxSum t{-INFINITY, 0.f};
        for (int w = 0; w < 4; ++w) t = ms_combine(t, MaxSum{wms[w].x, wms[w].y});
        zsh = (t.m == -INFINITY) ? -INFINITY : t.m + logf(t.s);
    }
    __syncthreads();
    const float z = zsh;
    for (int k = threadIdx.x; k < K; k += blockDim.x) {
        const uint64_t key = fin[k];
        cand_ids[(size_t)row * K + k] = key_id(key);
        cand_logp[(size_t)row * K + k] = key_value(key) - z;
    }
    if (threadIdx.x == 0) lse_out[row] = z;
}

// Largest prefetch depth (k-steps of weight loads in flight per wave) that
// divides the k-steps of a tile; 8 keeps the kernel inside 128 VGPRs, the
// budget of 16 waves per CU.
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

hipError_t launch_merge(const Dims& d, int nch, const uint64_t* keys, const float2* ms, int32_t* cand_ids,
                        float* cand_logp, float* lse, hipStream_t s) {
    const size_t lds = ((size_t)nch * d.K + 4 * (size_t)d.K) * 8;
    hipError_t e = hipFuncSetAttribute((const void*)merge_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    merge_kernel<<<d.rows(), 256, lds, s>>>(keys, ms, nch, d.K, cand_ids, cand_logp, lse);
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
    L.total = o;
    return L;
}

hipError_t launch_head_topk(const Dims& d, const void* y, const void* W, int32_t* cand_ids, float* cand_logp,
                            float* lse, float* logits_f32, char* ws, hipStream_t s) {
    const WsLayout L = ws_layout(d);
    const int nch = head_chunks(d);
    uint64_t* keys = (uint64_t*)(ws + L.keys);
    float2* ms = (float2*)(ws + L.ms);
    hipError_t e;
    if (d.bf16 && d.K <= 16) {
        e = launch_head_bf16_u<16, 16>(d, d.K, y, W, nch, keys, ms, logits_f32, s);
    } else if (d.bf16) {
        // K > 16: per-lane register lists of 64 keys would spill, so the
        // logits are written out and ranked by the logits top-K kernel, which
        // overwrites the (16-key) partials the head kernel leaves behind.
        float* logits = logits_f32 ? logits_f32 : (float*)(ws + L.logits);
        e = launch_head_bf16_u<16, 16>(d, 16, y, W, nch, keys, ms, logits, s);
        if (e == hipSuccess) e = launch_logits_partials(d, logits, nch, keys, ms, s);
    } else {
        float* logits = logits_f32 ? logits_f32 : (float*)(ws + L.logits);
        head_f32_kernel<<<(d.V + 255) / 256, 256, 0, s>>>((const float*)y, (const float*)W, logits, d.rows(), d.D,
                                                          d.V);
        e = hipGetLastError();
        if (e == hipSuccess) e = launch_logits_partials(d, logits, nch, keys, ms, s);
    }
    if (e != hipSuccess) return e;
    return launch_merge(d, nch, keys, ms, cand_ids, cand_logp, lse, s);
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
