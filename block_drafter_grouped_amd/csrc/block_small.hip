// The whole draft block in one launch, for small shapes where the path is
// bound by launch latency rather than by bytes or flops (vLLM release-note
// article on DFlash2, cost section: the conv's 20 small calls cost 0.477 ms
// eager and 0.0096 ms once captured as one graph -- launches, not work).  One
// workgroup per block runs every step of dfs_draft_block in order, with all
// intermediates in LDS:
//   1. conv (release-note article, section "two additions"): tap logits
//      z = h . Wg, softmax over the taps, the causal taps; y is rounded to
//      the dtype as the multi-kernel path does (bf16: round to nearest even);
//   2. head, log-softmax and top-K (same section: the K tokens the target
//      head ranks highest at each slot): thread i scores whole weight rows
//      i, i + 1024, ... against every row of the block into logits in LDS;
//      then wave w takes rows w, w + 16, ...: the (max, sum of exp) of the
//      row, and K rounds that each take the row's largest remaining key
//      (larger logit first, lower id on ties);
//   3. transition scores T_t[j, k] = <P[c_{t-1,j}] (*) H_t, Q[c_{t,k}]> (Inco
//      AI post "DFlash 2: keep the draft parallel", section "lightweight path
//      selector"), one fp32 dot product per thread;
//   4. the walk of walk.h (best path, greedy or sampled).
// Results agree with the multi-kernel path within the stated tolerances
// (the sums run in another order); ids follow the same tie rules.
#include "common.h"
#include "kernels.h"
#include "walk.h"

namespace dfs {

namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallMaxB = 16;
constexpr int kSmallMaxD = 512;
constexpr int kSmallMaxTaps = 512;
constexpr int kSmallMaxV = 16 * 64;  // 16 logits per lane in the top-K
constexpr int64_t kSmallMaxVD = 1 << 17;  // vocabulary x hidden: one workgroup's head work
constexpr int kSmallMaxR = 512;
constexpr int kSmallMaxLogits = 16384;  // block x vocabulary, held in LDS

template <typename T>
__device__ __forceinline__ float elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float elem<float>(const float* p, size_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float elem<uint16_t>(const uint16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
}

// 8 consecutive elements at p (16-B aligned for bf16, 32-B run for fp32).
template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&o)[8]);
template <>
__device__ __forceinline__ void load8f<uint16_t>(const uint16_t* p, float (&o)[8]) {
    const uint4 v = *(const uint4*)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float (&o)[8]) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// The first up-to-64 channels [d0, d0 + 64) of a row, as eight loads of 8
// elements, all issued before any is used; addresses are clamped into the
// row (a branch around each load would make each wait for the one before).
template <typename T>
__device__ __forceinline__ void load_chunk(const T* row, int d0, int D, float (&w)[8][8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) load8f<T>(row + min(d0 + 8 * u, D - 8), w[u]);
}

// acc[t] += <src[t][d0 : d0 + 64], w> for the B rows of src (LDS), in
// channel order, reading src four values at a time.
__device__ __forceinline__ void dot_chunk(const float (*src)[kSmallMaxD], int B, int d0, int D,
                                          const float (&w)[8][8], float (&acc)[kSmallMaxB]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        if (d0 + 8 * u < D) {
#pragma unroll
            for (int t = 0; t < kSmallMaxB; ++t) {
                if (t < B) {
                    const f32x4 a = *(const f32x4*)&src[t][d0 + 8 * u];
                    const f32x4 c = *(const f32x4*)&src[t][d0 + 8 * u + 4];
                    acc[t] += a[0] * w[u][0] + a[1] * w[u][1] + a[2] * w[u][2] + a[3] * w[u][3] + c[0] * w[u][4] +
                              c[1] * w[u][5] + c[2] * w[u][6] + c[3] * w[u][7];
                }
            }
        }
    }
}

// <src[t], row> for the B rows of src, into acc, through one buffer of 64
// channels; `buf` already holds the row's first 64 channels when
// have_first (loaded earlier, so their latency was spent elsewhere).
template <typename T>
__device__ __forceinline__ void row_dots(const T* row, int D, int B, const float (*src)[kSmallMaxD],
                                         bool have_first, float (&buf)[8][8], float (&acc)[kSmallMaxB]) {
#pragma unroll
    for (int t = 0; t < kSmallMaxB; ++t) acc[t] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 64) {
        if (d0 > 0 || !have_first) load_chunk<T>(row, d0, D, buf);
        dot_chunk(src, B, d0, D, buf, acc);
    }
}

// NVL: logits per lane a wave holds in registers for one row (V <= 64 NVL).
template <typename T, int NVL>
__global__ __launch_bounds__(kSmallThreads) void block_small_kernel(
    const T* __restrict__ h, const int32_t* __restrict__ anchor, const T* __restrict__ wg,
    const T* __restrict__ W, const T* __restrict__ P, const T* __restrict__ Q, const float* __restrict__ gate,
    int mode, float temperature, const float* __restrict__ uniforms, int32_t* __restrict__ path,
    float* __restrict__ path_score, int32_t* __restrict__ cand_ids, float* __restrict__ cand_logp, int B, int D,
    int V, int K, int r, int gs, int ks) {
    // hs and zs serve the conv only; the logits take their place after it.
    __shared__ __attribute__((aligned(16))) float conv_or_logits[kSmallMaxB * (kSmallMaxD + kSmallMaxTaps)];
    static_assert(kSmallMaxLogits <= kSmallMaxB * (kSmallMaxD + kSmallMaxTaps), "logits fit the conv's space");
    float(*hs)[kSmallMaxD] = (float(*)[kSmallMaxD])conv_or_logits;
    float(*zs)[kSmallMaxTaps] = (float(*)[kSmallMaxTaps])(conv_or_logits + kSmallMaxB * kSmallMaxD);
    float* lg = conv_or_logits;  // [B][V]
    __shared__ __attribute__((aligned(16))) float ys[kSmallMaxB][kSmallMaxD];
    __shared__ int32_t Cs[kSmallMaxB][16];
    __shared__ float Ls[kSmallMaxB][16];
    __shared__ float Ts[kSmallMaxB - 1][16][16];
    __shared__ __attribute__((aligned(16))) uint8_t bp[kSmallMaxB][16];
    __shared__ float Us[kSmallMaxB];
    __shared__ __attribute__((aligned(16))) float ones8[8];  // the gate when there is none
    constexpr bool kBf16 = sizeof(T) == 2;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int taps = (D / gs) * ks;
    if (tid < 8) ones8[tid] = 1.f;

    // 1. conv.  The first 64 channels of this thread's generator row are
    // requested before the hidden rows are staged, so both loads overlap.
    // The anchor is read now too: the transition scores need it after the
    // top-K, and then its load would be one more round trip on their path.
    float pre[8][8];
    if (ks != 1 && wave * kWave < taps)  // wave-uniform: only the waves that own generator rows
        load_chunk<T>(wg + (size_t)min(tid, taps - 1) * D, 0, D, pre);
    const int a = anchor[b];
    const T* hb = h + (size_t)b * B * D;
    for (int i = tid; i < B * D; i += kSmallThreads) hs[i / D][i % D] = elem(hb, i);
    __syncthreads();
    if (ks == 1) {
        for (int i = tid; i < B * D; i += kSmallThreads) ys[i / D][i % D] = hs[i / D][i % D];
    } else {
        for (int cc = tid; cc < taps; cc += kSmallThreads) {
            float acc[kSmallMaxB];
            row_dots<T>(wg + (size_t)cc * D, D, B, hs, cc == tid, pre, acc);
#pragma unroll
            for (int t = 0; t < kSmallMaxB; ++t)
                if (t < B) zs[t][cc] = acc[t];
        }
        __syncthreads();
        const int G = D / gs;
        for (int i = tid; i < B * G; i += kSmallThreads) {  // softmax over each group's taps
            const int t = i / G, g = i % G;
            float m = -INFINITY;
            for (int j = 0; j < ks; ++j) m = fmaxf(m, zs[t][g * ks + j]);
            float ex[4], den = 0.f;
            for (int j = 0; j < ks; ++j) {
                ex[j] = expf(zs[t][g * ks + j] - m);
                den += ex[j];
            }
            for (int j = 0; j < ks; ++j) zs[t][g * ks + j] = ex[j] / den;
        }
        __syncthreads();
        for (int i = tid; i < B * D; i += kSmallThreads) {  // causal taps, zero before the block
            const int t = i / D, c = i % D, g = c / gs;
            float v = 0.f;
            for (int j = 0; j < ks; ++j)
                if (t - j >= 0) v += zs[t][g * ks + j] * hs[t - j][c];
            ys[t][c] = kBf16 ? bf16_to_f32(f32_to_bf16(v)) : v;
        }
    }
    __syncthreads();

    // 2. head: thread tid scores weight rows tid, tid + 1024, ... against
    // every row of the block, into logits in LDS.
    for (int v = tid; v < V; v += kSmallThreads) {
        float acc[kSmallMaxB];
        row_dots<T>(W + (size_t)v * D, D, B, ys, false, pre, acc);
#pragma unroll
        for (int t = 0; t < kSmallMaxB; ++t)
            if (t < B) lg[t * V + v] = acc[t];
    }
    __syncthreads();
    // Per row (wave w: rows w, w + 16, ...): lane l holds the logits of ids
    // l + 64 i in registers (-inf past V, where keys are 0); the row's (max,
    // sum of exp) in two passes over them, then K rounds that each take the
    // wave's largest key (keys are distinct, so one lane holds it), after
    // which that lane moves to its largest key below it.
    for (int t = wave; t < B; t += kSmallWaves) {  // wave-uniform
        float x[NVL];
        uint64_t key[NVL];
        uint64_t best = 0ull;
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int v = lane + kWave * i;
            x[i] = lg[t * V + min(v, V - 1)];
            if (v >= V) x[i] = -INFINITY;
            key[i] = v < V ? make_key(x[i], (uint32_t)v) : 0ull;
            m = fmaxf(m, x[i]);
            best = umax64(best, key[i]);
        }
        float sm = 0.f;
        if (m > -INFINITY) {
#pragma unroll
            for (int i = 0; i < NVL; ++i) sm += __expf(x[i] - m);
        }
        const MaxSum z = wave_ms_reduce(MaxSum{m, sm});
        const float lse = z.m + logf(z.s);
        for (int k = 0; k < K; ++k) {
            const uint64_t top = wave_max_u64(best);
            if (lane == 0) {
                const int32_t id = key_id(top);
                const float lp = key_value(top) - lse;
                Cs[t][k] = id;
                Ls[t][k] = lp;
                if (cand_ids) cand_ids[((size_t)b * B + t) * K + k] = id;
                if (cand_logp) cand_logp[((size_t)b * B + t) * K + k] = lp;
            }
            if (best == top) {
                uint64_t nb = 0ull;
#pragma unroll
                for (int i = 0; i < NVL; ++i) nb = key[i] < top ? umax64(nb, key[i]) : nb;
                best = nb;
            }
        }
    }
    if (a < 0 || a >= V) {  // block-uniform
        write_bad_block(b, B, path, path_score, nullptr);
        return;
    }
    if (mode == 2)
        for (int t = tid; t < B; t += kSmallThreads) Us[t] = uniforms[(size_t)b * B + t];
    __syncthreads();

    // 3. transition scores
    const int KK = K * K;
    for (int i = tid; i < (B - 1) * KK; i += kSmallThreads) {
        const int t = 1 + i / KK, j = (i / K) % K, k = i % K;
        if (t == 1 && j > 0) {
            Ts[0][j][k] = 0.f;
            continue;
        }
        const int pa = (t == 1) ? a : Cs[t - 1][j];
        const T* pr = P + (size_t)pa * r;
        const T* qr = Q + (size_t)Cs[t][k] * r;
        const float* gr = gate ? gate + ((size_t)b * B + t) * r : nullptr;
        float acc = 0.f;
        for (int c0 = 0; c0 < r; c0 += 32) {  // the loads of 32 channels in flight
            float p8[4][8], q8[4][8], g8[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {  // unconditional loads, clamped addresses
                const int c = min(c0 + 8 * u, r - 8);
                load8f<T>(pr + c, p8[u]);
                load8f<T>(qr + c, q8[u]);
                load8f<float>(gr ? gr + c : ones8, g8[u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (c0 + 8 * u < r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += p8[u][e] * g8[u][e] * q8[u][e];
                }
            }
        }
        Ts[t - 1][j][k] = acc;
    }
    __syncthreads();

    // 4. the walk
    walk_block_lds(b, a, Cs, Ls, Ts, bp, mode, 1.f / temperature, Us, path, path_score, nullptr, B, K);
}

}  // namespace

bool use_small_block(const Dims& d) {
    return d.B <= kSmallMaxB && d.K <= 16 && d.D <= kSmallMaxD && d.taps() <= kSmallMaxTaps && d.V <= kSmallMaxV &&
           (int64_t)d.V * d.D <= kSmallMaxVD && d.B * d.V <= kSmallMaxLogits && d.r <= kSmallMaxR && d.ks <= 4;
}

template <typename T, int NVL>
static void launch_small_t(const Dims& d, const SelectOpts& o, const void* h, const int32_t* anchor,
                           const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                           float* path_score, int32_t* cand_ids, float* cand_logp, hipStream_t s) {
    block_small_kernel<T, NVL><<<d.batch, kSmallThreads, 0, s>>>(
        (const T*)h, anchor, (const T*)wg_cm, (const T*)W, (const T*)P, (const T*)Q, o.gate, o.walk, o.temperature,
        o.uniforms, path, path_score, cand_ids, cand_logp, d.B, d.D, d.V, d.K, d.r, d.gs, d.ks);
}

hipError_t launch_block_small(const Dims& d, const SelectOpts& o, const void* h, const int32_t* anchor,
                              const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                              float* path_score, int32_t* cand_ids, float* cand_logp, hipStream_t s) {
    if (d.bf16)
        launch_small_t<uint16_t, 16>(d, o, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp, s);
    else
        launch_small_t<float, 16>(d, o, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp, s);
    return hipGetLastError();
}

}  // namespace dfs
