// Steps 4-5 of the draft-block path: low-rank adjacent-transition scores and
// the best path from the verified anchor (Inco AI post "DFlash 2: keep the
// draft parallel", section "lightweight path selector": every adjacent pair
// of candidates is scored at once with per-token rank-r embeddings, and the
// only sequential work is the walk over those precomputed scores; the walk
// starts from the last verified token, as in the vLLM release-note article,
// section "two additions").  The post's context gate H(h_t) is optional: the
// caller supplies it, or it is 1.
//
// Fast path (bf16 tables, K <= 16, r % 32 == 0, with or without a gate; the
// best path at any block length, greedy and sampled walks up to 16 slots):
// select_fused_kernel, below.  General path:
// sel_dots: one workgroup per (draft slot, block, 16 x 16 sub-tile) computes
// the K x K matrix
//   T_t[j, k] = sum_i P[c_{t-1, j}, i] * H_t[i] * Q[c_{t, k}, i]
// (c_0 = {anchor}: a 1 x K row) from rows gathered out of P and Q into LDS,
// fp32 accumulation.
// walk: one workgroup per block walks the scores (best path, greedy or
//   sampled) from LDS, with T streamed in ahead of the walk.
#include "common.h"
#include "kernels.h"
#include "walk.h"

namespace dfs {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&out)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&out)[8]) {
    const uint4 v = *(const uint4*)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&out)[8]) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// General transition scores: one workgroup (256 threads) per (draft slot,
// block, 16 x 16 sub-tile of the K x K matrix).  The sub-tile's 16
// predecessor rows of P (times the gate, in fp32) and 16 successor rows of Q
// are gathered into LDS in chunks of 256 channels, all loads of a chunk in
// flight together; thread (jb, kb) then accumulates the dot j = j0 + jb,
// k = k0 + kb from LDS.  Rows are padded by 4 floats, so the 16 rows a wave
// reads at one channel sit in distinct banks.  An invalid id gives a zero
// row (the walk marks such a block).
constexpr int kDotsCh = 256;
constexpr int kDotsPitch = kDotsCh + 4;

template <typename T>
__global__ __launch_bounds__(256) void sel_dots_kernel(const int32_t* __restrict__ anchor,
                                                       const int32_t* __restrict__ cand_ids, const T* __restrict__ P,
                                                       const T* __restrict__ Q, const float* __restrict__ gate,
                                                       float* __restrict__ Tout, int B, int K, int r, int V) {
    constexpr int UPR = kDotsCh / 8;  // 8-channel units per row
    __shared__ __attribute__((aligned(16))) float Ps[16 * kDotsPitch];
    __shared__ __attribute__((aligned(16))) float Qs[16 * kDotsPitch];
    const int t = blockIdx.x + 1, b = blockIdx.y;
    const int nb = (K + 15) / 16;
    const int j0 = 16 * (blockIdx.z / nb), k0 = 16 * (blockIdx.z % nb);
    const int a = anchor[b];
    const int nprev = (t == 1) ? 1 : K;
    if (a < 0 || a >= V || j0 >= nprev) return;  // uniform
    const int tid = threadIdx.x, jb = tid / 16, kb = tid % 16;
    const float* gr = gate ? gate + ((size_t)b * B + t) * r : nullptr;
    float acc = 0.f;
    for (int c0 = 0; c0 < r; c0 += kDotsCh) {
        __syncthreads();  // the previous chunk has been read
        for (int u = tid; u < 16 * UPR; u += 256) {
            const int row = u / UPR, part = u % UPR;
            const int ch = c0 + 8 * part;
            float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (ch < r) {
                const int j = j0 + row, k = k0 + row;
                if (j < nprev) {
                    const int pa = (t == 1) ? a : cand_ids[((size_t)b * B + t - 1) * K + j];
                    if (pa >= 0 && pa < V) {
                        load8<T>(P + (size_t)pa * r + ch, x);
                        if (gr) {  // context gate of slot t: (P * H) . Q
                            float g[8];
                            load8<float>(gr + ch, g);
#pragma unroll
                            for (int e = 0; e < 8; ++e) x[e] *= g[e];
                        }
                    }
                }
                if (k < K) {
                    const int qb = cand_ids[((size_t)b * B + t) * K + k];
                    if (qb >= 0 && qb < V) load8<T>(Q + (size_t)qb * r + ch, z);
                }
            }
            float* pd = Ps + row * kDotsPitch + 8 * part;
            float* qd = Qs + row * kDotsPitch + 8 * part;
            *(f32x4*)pd = f32x4{x[0], x[1], x[2], x[3]};
            *(f32x4*)(pd + 4) = f32x4{x[4], x[5], x[6], x[7]};
            *(f32x4*)qd = f32x4{z[0], z[1], z[2], z[3]};
            *(f32x4*)(qd + 4) = f32x4{z[4], z[5], z[6], z[7]};
        }
        __syncthreads();
#pragma unroll 4
        for (int i = 0; i < kDotsCh; i += 4) {
            const f32x4 pv = *(const f32x4*)(Ps + jb * kDotsPitch + i);
            const f32x4 qv = *(const f32x4*)(Qs + kb * kDotsPitch + i);
            acc += pv[0] * qv[0] + pv[1] * qv[1] + pv[2] * qv[2] + pv[3] * qv[3];
        }
    }
    const int j = j0 + jb, k = k0 + kb;
    if (j < nprev && k < K) Tout[(((size_t)b * (B - 1) + t - 1) * K + j) * K + k] = acc;
}

// The walk over precomputed transition scores, one workgroup per block.
// Candidates, node scores and uniforms go to LDS first; T streams through a
// double-buffered LDS ring, kWalkChunk floats (whole slots) per buffer, all
// four waves fetching the next chunk while the current one is walked, so
// the sequential walk never waits on HBM per slot.  Lane k = candidate k:
//  * best path (mode 0), all four waves: delta_1[k] = cand_logp[1][k] +
//    T_1[0][k]; delta_t[k] = max_j (delta_{t-1}[j] + T_t[j][k]) +
//    cand_logp[t][k], the lowest j on ties; the end is the lowest k with the
//    largest delta, then the back-pointers.
//  * greedy / sampled (modes 1, 2; Inco AI post, "lightweight path selector":
//    take the best successor of the token chosen before, or sample it from
//    the same scores), wave 0: after index p of slot t-1 (p = 0, the anchor,
//    at t = 1), s_k = cand_logp[t][k] + T_t[p][k].  Greedy: the largest s_k,
//    the lowest k on ties.  Sample: e_k = exp((s_k - max s) / temperature),
//    prefix sums E_k in lane order, and the smallest k with
//    E_k > u_t * E_{K-1} (the last candidate if rounding leaves none).
// Each decision follows the same rule as the fp64 reference, in fp32.  The
// chosen indices go to LDS; all threads then write the path.
constexpr int kWalkThreads = 256;
constexpr int kWalkChunk = 12288;  // 48 KB per buffer; >= 3 slots at K = 64
constexpr int kWalkPer = kWalkChunk / kWalkThreads;

__global__ __launch_bounds__(kWalkThreads) void walk_kernel(const int32_t* __restrict__ anchor,
                                                            const int32_t* __restrict__ cand_ids,
                                                            const float* __restrict__ cand_logp,
                                                            const float* __restrict__ Tin, int mode, float temperature,
                                                            const float* __restrict__ uniforms,
                                                            int32_t* __restrict__ path, float* __restrict__ path_score,
                                                            int32_t* __restrict__ path_idx, int B, int K, int V) {
    __shared__ float Tbuf[2][kWalkChunk];
    __shared__ int32_t Cs[64 * 64];  // slot t, candidate k at t * K + k
    __shared__ float Ls[64 * 64];
    __shared__ uint8_t bp[64 * 64];
    __shared__ float Us[64];
    __shared__ float dsh[64];  // delta of the previous slot (best path)
    __shared__ float pv[kWalkThreads / kWave][64];
    __shared__ int32_t pj[kWalkThreads / kWave][64];
    __shared__ int32_t pick_s[64];
    __shared__ float score_s;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int a = anchor[b];
    bool bad = (a < 0 || a >= V);
    for (int i = tid; i < (B - 1) * K; i += kWalkThreads) {
        const size_t g = ((size_t)b * B + 1) * K + i;
        const int id = cand_ids[g];
        bad |= (id < 0 || id >= V);
        Cs[K + i] = id;
        Ls[K + i] = cand_logp[g];
    }
    if (mode == 2)
        for (int t = tid; t < B; t += kWalkThreads) Us[t] = uniforms[(size_t)b * B + t];
    if (__syncthreads_or(bad)) {
        write_bad_block(b, B, path, path_score, path_idx);
        return;
    }

    const float* Tb = Tin + (size_t)b * (B - 1) * K * K;
    const int KK = K * K, nslot = B - 1;
    const int S = kWalkChunk / KK;  // K <= 64, so S >= 3
    const int nch = (nslot + S - 1) / S;
    float reg[kWalkPer];
    auto fetch = [&](int c) {
        const float* src = Tb + (size_t)c * S * KK;
        const int n = min(S, nslot - c * S) * KK;
#pragma unroll
        for (int u = 0; u < kWalkPer; ++u) {
            const int e = tid + kWalkThreads * u;
            reg[u] = e < n ? src[e] : 0.f;
        }
    };
    auto put = [&](int c) {
        float* dst = Tbuf[c & 1];
#pragma unroll
        for (int u = 0; u < kWalkPer; ++u) dst[tid + kWalkThreads * u] = reg[u];
    };

    const bool on = lane < K;
    const int kc = on ? lane : K - 1;  // in-bounds column for idle lanes
    const float inv_t = 1.f / temperature;
    float d = -INFINITY, total = 0.f;  // best-path state / walk total
    int prev = 0;                      // walk state: index chosen at t-1
    fetch(0);
    put(0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) fetch(c + 1);
        const float* Tc = Tbuf[c & 1];
        const int t_end = min(nslot, (c + 1) * S);
        if (mode == 0) {
            // Best path, all four waves: wave w scans predecessors
            // j = 16w .. 16w + 15 of every candidate (the first, then a strict
            // comparison), and the four partial results are combined in
            // wave order with a strict comparison, so the lowest j with the
            // largest score wins, as in a left-to-right scan.  delta_{t-1}
            // is read from LDS (dsh).
            for (int t = 1 + c * S; t <= t_end; ++t) {
                const float* Tt = Tc + (t - 1 - c * S) * KK;
                const float lp = Ls[t * K + kc];
                if (t == 1) {
                    d = on ? lp + Tt[kc] : -INFINITY;
                } else {
                    float bv = -INFINITY;
                    int bi = kWave;
                    const int j0 = 16 * wave;
                    if (j0 < K) {
                        float cv[16];
#pragma unroll
                        for (int u = 0; u < 16; ++u) {
                            const int j = min(j0 + u, K - 1);
                            cv[u] = dsh[j] + Tt[j * K + kc];
                        }
#pragma unroll
                        for (int u = 0; u < 16; ++u) {
                            const bool gt = (u == 0) | ((j0 + u < K) & (cv[u] > bv));
                            bv = gt ? cv[u] : bv;
                            bi = gt ? j0 + u : bi;
                        }
                    }
                    pv[wave][lane] = bv;
                    pj[wave][lane] = bi;
                    __syncthreads();  // partials written; dsh no longer read this slot
                    float best = pv[0][lane];
                    int bj = pj[0][lane];
#pragma unroll
                    for (int w = 1; w < kWalkThreads / kWave; ++w) {
                        const float v = pv[w][lane];
                        const bool gt = v > best;
                        best = gt ? v : best;
                        bj = gt ? pj[w][lane] : bj;
                    }
                    d = on ? best + lp : -INFINITY;
                    if (wave == 0 && on) bp[t * K + lane] = (uint8_t)bj;
                }
                if (wave == 0) dsh[lane] = d;
                __syncthreads();  // delta_t published; the partials may be rewritten
            }
        } else if (wave == 0) {
            for (int t = 1 + c * S; t <= t_end; ++t) {
                const float* Tt = Tc + (t - 1 - c * S) * KK;
                const float lp = Ls[t * K + kc];
                const float sk = on ? lp + Tt[prev * K + kc] : -INFINITY;
                const float m = wave_max_f32(sk);
                int pick;
                if (mode == 1) {
                    pick = __ffsll((unsigned long long)__ballot(on && sk == m)) - 1;
                } else {
                    float e = on ? __expf((sk - m) * inv_t) : 0.f;
                    for (int o = 1; o < kWave; o <<= 1) {  // inclusive prefix sum in lane order
                        const float v = __shfl_up(e, o, kWave);
                        if (lane >= o) e += v;
                    }
                    const float tot = readlane_f32(e, K - 1);
                    const float target = Us[t] * tot;
                    const uint64_t over = __ballot(on && e > target);
                    pick = over ? __ffsll((unsigned long long)over) - 1 : K - 1;
                }
                total += readlane_f32(sk, pick);
                prev = pick;
                if (lane == 0) pick_s[t] = pick;
            }
        }
        if (c + 1 < nch) put(c + 1);
        __syncthreads();
    }
    if (wave == 0) {
        if (mode == 0) {
            const float mx = wave_max_f32(d);
            const uint64_t ball = __ballot(on && d == mx);
            const int kb = __ffsll((unsigned long long)ball) - 1;
            if (lane == 0) {
                int k = kb;
                for (int t = B - 1; t >= 1; --t) {
                    pick_s[t] = k;
                    if (t >= 2) k = bp[t * K + k];
                }
                score_s = mx;
            }
        } else if (lane == 0) {
            score_s = total;
        }
    }
    __syncthreads();
    for (int t = tid; t < B; t += kWalkThreads) {
        const int k = t == 0 ? -1 : pick_s[t];
        path[(size_t)b * B + t] = t == 0 ? a : Cs[t * K + k];
        if (path_idx) path_idx[(size_t)b * B + t] = k;
    }
    if (tid == 0) path_score[b] = score_s;
}

// Selector for bf16 tables with K <= 16 and r % 32 == 0, with or without a
// context gate, on given candidates; any walk (mode 0: best path, 1: greedy,
// 2: sampled).
template <int NWS>
__global__ __launch_bounds__(NWS * kWave) void select_fused_kernel(
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ cand_ids, const float* __restrict__ cand_logp,
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q, const float* __restrict__ gate, int mode,
    float temperature, const float* __restrict__ uniforms, int32_t* __restrict__ path, float* __restrict__ path_score,
    int32_t* __restrict__ path_idx, int B, int K, int r, int V) {
    extern __shared__ float Tsm[];  // [B-1][16][16]
    __shared__ float Ls[64][16];
    __shared__ float Us[64];
    __shared__ int32_t Cs[64][16];
    __shared__ __attribute__((aligned(16))) uint8_t bp[64][16];
    select_block<NWS>(blockIdx.x, anchor, cand_ids, cand_logp, P, Q, gate, mode, temperature, uniforms, path,
                      path_score, path_idx, B, K, r, V, Cs, Ls, (float(*)[16][16])Tsm, bp, Us);
}

}  // namespace

hipError_t launch_select(const Dims& d, const SelectOpts& o, const int32_t* anchor, const int32_t* cand_ids,
                         const float* cand_logp, const void* P, const void* Q, int32_t* path, float* path_score,
                         int32_t* path_idx, char* ws, hipStream_t s) {
    // The fused kernel gathers each wave's slots one after another: for the
    // greedy and sampled walks it is the faster path up to 16 slots, for the
    // best path at every length measured (up to 64).
    if (d.bf16 && d.K <= 16 && d.r % 32 == 0 && (o.walk == 0 || d.B <= 16)) {
        const size_t lds = (size_t)(d.B - 1) * 16 * 16 * sizeof(float);
        static LdsAttr attr;
        hipError_t e = ensure_lds(attr, (const void*)select_fused_kernel<8>, (int)lds);
        if (e != hipSuccess) return e;
        select_fused_kernel<8><<<d.batch, 8 * kWave, lds, s>>>(anchor, cand_ids, cand_logp, (const uint16_t*)P,
                                                             (const uint16_t*)Q, o.gate, o.walk, o.temperature,
                                                             o.uniforms,
                                                             path, path_score, path_idx, d.B, d.K, d.r, d.V);
        return hipGetLastError();
    }
    const WsLayout L = ws_layout(d);
    float* T = (float*)(ws + L.T);
    const int nb = (d.K + 15) / 16;
    dim3 grid(d.B - 1, d.batch, nb * nb);
    if (d.bf16)
        sel_dots_kernel<uint16_t><<<grid, 256, 0, s>>>(anchor, cand_ids, (const uint16_t*)P, (const uint16_t*)Q,
                                                       o.gate, T, d.B, d.K, d.r, d.V);
    else
        sel_dots_kernel<float><<<grid, 256, 0, s>>>(anchor, cand_ids, (const float*)P, (const float*)Q, o.gate, T,
                                                    d.B, d.K, d.r, d.V);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    walk_kernel<<<d.batch, kWalkThreads, 0, s>>>(anchor, cand_ids, cand_logp, T, o.walk, o.temperature, o.uniforms,
                                                 path, path_score, path_idx, d.B, d.K, d.V);
    return hipGetLastError();
}

}  // namespace dfs
