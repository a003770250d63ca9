// Steps 4-5 of the draft-block path: low-rank adjacent-transition scores and
// the best path from the verified anchor (Inco AI post "DFlash 2: keep the
// draft parallel", section "lightweight path selector": every adjacent pair
// of candidates is scored at once with per-token rank-r embeddings, and the
// only sequential work is the walk over those precomputed scores; the walk
// starts from the last verified token, as in the vLLM release-note article,
// section "two additions").  The post's context gate H(h_t) is optional: the
// caller supplies it, or it is 1.
//
// Fast path (bf16 tables, K <= 16, no gate, best-path walk): select_fused_kernel,
// below.  General path:
// sel_dots: one workgroup per (draft slot, block) computes the K x K matrix
//   T_t[j, k] = sum_i P[c_{t-1, j}, i] * H_t[i] * Q[c_{t, k}, i]
// (c_0 = {anchor}: a 1 x K row) from rows gathered out of P and Q, fp32
// accumulation.
// viterbi: one wavefront per block, lane k = candidate k.  The max over
// predecessors broadcasts delta_{t-1}[j] with v_readlane; the final argmax
// uses a DPP max and a ballot (lowest lane wins ties).
// walk: the greedy and sampled walks, one wavefront per block.
#include "common.h"
#include "kernels.h"

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

template <typename T>
__global__ __launch_bounds__(256) void sel_dots_kernel(const int32_t* __restrict__ anchor,
                                                       const int32_t* __restrict__ cand_ids, const T* __restrict__ P,
                                                       const T* __restrict__ Q, const float* __restrict__ gate,
                                                       float* __restrict__ Tout, int B, int K, int r, int V) {
    const int t = blockIdx.x + 1, b = blockIdx.y;
    const int a = anchor[b];
    if (a < 0 || a >= V) return;
    const int nprev = (t == 1) ? 1 : K;
    for (int p = threadIdx.x; p < nprev * K; p += blockDim.x) {
        const int j = p / K, k = p % K;
        const int pa = (t == 1) ? a : cand_ids[((size_t)b * B + t - 1) * K + j];
        const int qb = cand_ids[((size_t)b * B + t) * K + k];
        float acc = 0.f;
        if (pa >= 0 && pa < V && qb >= 0 && qb < V) {
            const T* pr = P + (size_t)pa * r;
            const T* qr = Q + (size_t)qb * r;
            if (gate) {  // context gate of slot t: (P * H) . Q
                const float* gr = gate + ((size_t)b * B + t) * r;
                for (int i = 0; i < r; i += 8) {
                    float x[8], z[8], g[8];
                    load8<T>(pr + i, x);
                    load8<T>(qr + i, z);
                    load8<float>(gr + i, g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += (x[e] * g[e]) * z[e];
                }
            } else {
                for (int i = 0; i < r; i += 8) {
                    float x[8], z[8];
                    load8<T>(pr + i, x);
                    load8<T>(qr + i, z);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += x[e] * z[e];
                }
            }
        }
        Tout[(((size_t)b * (B - 1) + t - 1) * K + j) * K + k] = acc;
    }
}

template <int KM>
__global__ __launch_bounds__(kWave) void viterbi_kernel(const int32_t* __restrict__ anchor,
                                                        const int32_t* __restrict__ cand_ids,
                                                        const float* __restrict__ cand_logp,
                                                        const float* __restrict__ Tin, int32_t* __restrict__ path,
                                                        float* __restrict__ path_score, int32_t* __restrict__ path_idx,
                                                        int B, int K, int V) {
    __shared__ uint8_t bp[64 * 64];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int a = anchor[b];
    bool bad = (a < 0 || a >= V);
    for (int i = lane; i < (B - 1) * K; i += kWave) {
        const int id = cand_ids[((size_t)b * B + 1) * K + i];
        bad |= (id < 0 || id >= V);
    }
    if (__any(bad)) {
        for (int t = lane; t < B; t += kWave) {
            path[(size_t)b * B + t] = -1;
            if (path_idx) path_idx[(size_t)b * B + t] = -1;
        }
        if (lane == 0) path_score[b] = __int_as_float(0x7FC00000);
        return;
    }
    const float* Tb = Tin + (size_t)b * (B - 1) * K * K;
    const bool on = lane < K;
    float d = on ? cand_logp[((size_t)b * B + 1) * K + lane] + Tb[lane] : -INFINITY;
    for (int t = 2; t < B; ++t) {
        const float* Tt = Tb + (size_t)(t - 1) * K * K;
        float tc[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) tc[j] = (j < K && on) ? Tt[(size_t)j * K + lane] : 0.f;
        const float lp = on ? cand_logp[((size_t)b * B + t) * K + lane] : 0.f;
        float best = -INFINITY;
        int bj = 0;
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j < K) {
                const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), j));
                const float c = dj + tc[j];
                if (j == 0 || c > best) {
                    best = c;
                    bj = j;
                }
            }
        }
        d = on ? best + lp : -INFINITY;
        if (on) bp[t * 64 + lane] = (uint8_t)bj;
    }
    const float mx = wave_max_f32(d);
    const uint64_t ball = __ballot(on && d == mx);
    const int kb = __ffsll((unsigned long long)ball) - 1;
    __syncthreads();
    if (lane == 0) {
        int k = kb;
        for (int t = B - 1; t >= 1; --t) {
            path[(size_t)b * B + t] = cand_ids[((size_t)b * B + t) * K + k];
            if (path_idx) path_idx[(size_t)b * B + t] = k;
            if (t >= 2) k = bp[t * 64 + k];
        }
        path[(size_t)b * B] = a;
        if (path_idx) path_idx[(size_t)b * B] = -1;
        path_score[b] = mx;
    }
}

// The greedy and sampled walks (Inco AI post, "lightweight path selector":
// take the best successor of the token chosen before, or sample it from the
// same scores).  One wavefront per block, lane k = candidate k.  At slot t,
// after index p of slot t-1 (p = 0, the anchor, at t = 1), candidate k
// scores s_k = cand_logp[t][k] + T_t[p][k].  Greedy: the largest s_k, the
// lowest k on ties.  Sample: e_k = exp((s_k - max s) / temperature), prefix
// sums E_k in lane order, and the smallest k with E_k > u_t * E_{K-1} (the
// last candidate if rounding leaves none), u_t = uniforms[b, t].  Each
// decision follows the same rule as the fp64 reference, in fp32.
__global__ __launch_bounds__(kWave) void walk_kernel(const int32_t* __restrict__ anchor,
                                                     const int32_t* __restrict__ cand_ids,
                                                     const float* __restrict__ cand_logp, const float* __restrict__ Tin,
                                                     int sample, float temperature, const float* __restrict__ uniforms,
                                                     int32_t* __restrict__ path, float* __restrict__ path_score,
                                                     int32_t* __restrict__ path_idx, int B, int K, int V) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int a = anchor[b];
    bool bad = (a < 0 || a >= V);
    for (int i = lane; i < (B - 1) * K; i += kWave) {
        const int id = cand_ids[((size_t)b * B + 1) * K + i];
        bad |= (id < 0 || id >= V);
    }
    if (__any(bad)) {
        for (int t = lane; t < B; t += kWave) {
            path[(size_t)b * B + t] = -1;
            if (path_idx) path_idx[(size_t)b * B + t] = -1;
        }
        if (lane == 0) path_score[b] = __int_as_float(0x7FC00000);
        return;
    }
    const float* Tb = Tin + (size_t)b * (B - 1) * K * K;
    const bool on = lane < K;
    const float inv_t = 1.f / temperature;
    int prev = 0;
    float total = 0.f;
    for (int t = 1; t < B; ++t) {
        const float sk = on ? cand_logp[((size_t)b * B + t) * K + lane] + Tb[((size_t)(t - 1) * K + prev) * K + lane]
                            : -INFINITY;
        const float m = wave_max_f32(sk);
        int pick;
        if (!sample) {
            pick = __ffsll((unsigned long long)__ballot(on && sk == m)) - 1;
        } else {
            float e = on ? __expf((sk - m) * inv_t) : 0.f;
            for (int o = 1; o < kWave; o <<= 1) {  // inclusive prefix sum in lane order
                const float v = __shfl_up(e, o, kWave);
                if (lane >= o) e += v;
            }
            const float tot = readlane_f32(e, K - 1);
            const float target = uniforms[(size_t)b * B + t] * tot;
            const uint64_t over = __ballot(on && e > target);
            pick = over ? __ffsll((unsigned long long)over) - 1 : K - 1;
        }
        total += readlane_f32(sk, pick);
        prev = pick;
        if (lane == 0) {
            path[(size_t)b * B + t] = cand_ids[((size_t)b * B + t) * K + pick];
            if (path_idx) path_idx[(size_t)b * B + t] = pick;
        }
    }
    if (lane == 0) {
        path[(size_t)b * B] = a;
        if (path_idx) path_idx[(size_t)b * B] = -1;
        path_score[b] = total;
    }
}

// Transition scores and the walk of one block, from candidates already in
// LDS: Cs[t][k] (ids) and Ls[t][k] (node scores) for t = 1..B-1, a valid
// anchor, and a barrier between filling them and this call.  Every thread
// of the workgroup calls it.  Wave w computes T_t for t = 1 + w, 1 + w + NWS,
// ... as one 16x16 MFMA tile (A = P rows of the previous slot's candidates,
// or of the anchor for t = 1; B = Q rows of this slot's candidates), with
// every gather of a slot in flight at once; wave 0 then walks.
template <int NWS>
__device__ __forceinline__ void select_block_lds(int b, int a, const int32_t (*Cs)[16], const float (*Ls)[16],
                                                 float (*Ts)[16][16], uint8_t (*bp)[16],
                                                 const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q,
                                                 int32_t* __restrict__ path, float* __restrict__ path_score,
                                                 int32_t* __restrict__ path_idx, int B, int K, int r) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int i16 = lane & 15, q = lane >> 4, kk = min(i16, K - 1);
    const int nks = r / 32;
    for (int t = 1 + wave; t < B; t += NWS) {
        const int pa = (t == 1) ? a : Cs[t - 1][kk];
        const int qb = Cs[t][kk];
        const uint16_t* pr = P + (size_t)pa * r + 8 * q;
        const uint16_t* qr = Q + (size_t)qb * r + 8 * q;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nks; s0 += 8) {
            bf16x8 av[8], bv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = min(s0 + u, nks - 1);
                av[u] = *(const bf16x8*)(pr + 32 * s);
                bv[u] = *(const bf16x8*)(qr + 32 * s);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < nks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u], acc, 0, 0, 0);
        }
        // lane holds T_t[4q + rr][i16]
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Ts[t - 1][4 * q + rr][i16] = acc[rr];
    }
    __syncthreads();
    if (wave != 0) return;

    const bool on = lane < K;
    float d = on ? Ls[1][lane] + Ts[0][0][lane] : -INFINITY;
    for (int t = 2; t < B; ++t) {
        float tc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) tc[j] = Ts[t - 1][j][lane & 15];
        float best = -INFINITY;
        int bj = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j < K) {
                const float dj = readlane_f32(d, j);
                const float c = dj + tc[j];
                if (j == 0 || c > best) {
                    best = c;
                    bj = j;
                }
            }
        }
        d = on ? best + Ls[t][lane & 15] : -INFINITY;
        if (on) bp[t][lane] = (uint8_t)bj;
    }
    const float mx = wave_max_f32(d);
    const uint64_t ball = __ballot(on && d == mx);
    const int kb = __ffsll((unsigned long long)ball) - 1;
    if (lane == 0) {
        int k = kb;
        for (int t = B - 1; t >= 1; --t) {
            path[(size_t)b * B + t] = Cs[t][k];
            if (path_idx) path_idx[(size_t)b * B + t] = k;
            if (t >= 2) k = bp[t][k];
        }
        path[(size_t)b * B] = a;
        if (path_idx) path_idx[(size_t)b * B] = -1;
        path_score[b] = mx;
    }
}

__device__ __forceinline__ void write_bad_block(int b, int B, int32_t* path, float* path_score, int32_t* path_idx) {
    for (int t = threadIdx.x; t < B; t += blockDim.x) {
        path[(size_t)b * B + t] = -1;
        if (path_idx) path_idx[(size_t)b * B + t] = -1;
    }
    if (threadIdx.x == 0) path_score[b] = __int_as_float(0x7FC00000);
}

// Selector for bf16 tables with K <= 16 and r % 32 == 0, on given candidates.
template <int NWS>
__global__ __launch_bounds__(NWS * kWave) void select_fused_kernel(
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ cand_ids, const float* __restrict__ cand_logp,
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q, int32_t* __restrict__ path,
    float* __restrict__ path_score, int32_t* __restrict__ path_idx, int B, int K, int r, int V) {
    extern __shared__ float Tsm[];  // [B-1][16][16]
    __shared__ float Ls[64][16];
    __shared__ int32_t Cs[64][16];
    __shared__ uint8_t bp[64][16];
    const int b = blockIdx.x, t0 = threadIdx.x;
    const int a = anchor[b];
    bool bad = (a < 0 || a >= V);
    for (int i = t0; i < (B - 1) * K; i += NWS * kWave) {
        const int t = 1 + i / K, k = i % K;
        const int id = cand_ids[((size_t)b * B + t) * K + k];
        bad |= (id < 0 || id >= V);
        Cs[t][k] = id;
        Ls[t][k] = cand_logp[((size_t)b * B + t) * K + k];
    }
    if (__syncthreads_or(bad)) {
        write_bad_block(b, B, path, path_score, path_idx);
        return;
    }
    select_block_lds<NWS>(b, a, Cs, Ls, (float(*)[16][16])Tsm, bp, P, Q, path, path_score, path_idx, B, K, r);
}

}  // namespace

hipError_t launch_select(const Dims& d, const SelectOpts& o, const int32_t* anchor, const int32_t* cand_ids,
                         const float* cand_logp, const void* P, const void* Q, int32_t* path, float* path_score,
                         int32_t* path_idx, char* ws, hipStream_t s) {
    const bool plain = !o.gate && o.walk == 0;
    if (plain && d.bf16 && d.K <= 16 && d.r % 32 == 0) {
        const size_t lds = (size_t)(d.B - 1) * 16 * 16 * sizeof(float);
        hipError_t e = hipFuncSetAttribute((const void*)select_fused_kernel<8>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        select_fused_kernel<8><<<d.batch, 8 * kWave, lds, s>>>(anchor, cand_ids, cand_logp, (const uint16_t*)P,
                                                             (const uint16_t*)Q, path, path_score, path_idx, d.B,
                                                             d.K, d.r, d.V);
        return hipGetLastError();
    }
    const WsLayout L = ws_layout(d);
    float* T = (float*)(ws + L.T);
    dim3 grid(d.B - 1, d.batch);
    if (d.bf16)
        sel_dots_kernel<uint16_t><<<grid, 256, 0, s>>>(anchor, cand_ids, (const uint16_t*)P, (const uint16_t*)Q,
                                                       o.gate, T, d.B, d.K, d.r, d.V);
    else
        sel_dots_kernel<float><<<grid, 256, 0, s>>>(anchor, cand_ids, (const float*)P, (const float*)Q, o.gate, T,
                                                    d.B, d.K, d.r, d.V);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (o.walk != 0)
        walk_kernel<<<d.batch, kWave, 0, s>>>(anchor, cand_ids, cand_logp, T, o.walk == 2, o.temperature, o.uniforms,
                                              path, path_score, path_idx, d.B, d.K, d.V);
    else if (d.K <= 16)
        viterbi_kernel<16><<<d.batch, kWave, 0, s>>>(anchor, cand_ids, cand_logp, T, path, path_score, path_idx, d.B,
                                                     d.K, d.V);
    else
        viterbi_kernel<64><<<d.batch, kWave, 0, s>>>(anchor, cand_ids, cand_logp, T, path, path_score, path_idx, d.B,
                                                     d.K, d.V);
    return hipGetLastError();
}

}  // namespace dfs
