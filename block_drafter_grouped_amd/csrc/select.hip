// Steps 4-5 of the draft-block path: low-rank adjacent-transition scores and
// the best path from the verified anchor (Inco AI post "DFlash 2: keep the
// draft parallel", section "lightweight path selector": every adjacent pair
// of candidates is scored at once with per-token rank-r embeddings, and the
// only sequential work is the walk over those precomputed scores; the walk
// starts from the last verified token, as in the vLLM release-note article,
// section "two additions").  The context gate of the post is taken as 1.
//
// sel_dots: one workgroup per (draft slot, block) computes the K x K matrix
//   T_t[j, k] = <P[c_{t-1, j}], Q[c_{t, k}]>   (c_0 = {anchor}: a 1 x K row)
// from rows gathered out of P and Q, fp32 accumulation.
// viterbi: one wavefront per block, lane k = candidate k.  The max over
// predecessors broadcasts delta_{t-1}[j] with v_readlane; the final argmax
// uses a butterfly max and a ballot (lowest lane wins ties).
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
                                                       const T* __restrict__ Q, float* __restrict__ Tout, int B, int K,
                                                       int r, int V) {
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
            for (int i = 0; i < r; i += 8) {
                float x[8], z[8];
                load8<T>(pr + i, x);
                load8<T>(qr + i, z);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += x[e] * z[e];
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
    float mx = d;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
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

}  // namespace

hipError_t launch_select(const Dims& d, const int32_t* anchor, const int32_t* cand_ids, const float* cand_logp,
                         const void* P, const void* Q, int32_t* path, float* path_score, int32_t* path_idx, char* ws,
                         hipStream_t s) {
    const WsLayout L = ws_layout(d);
    float* T = (float*)(ws + L.T);
    dim3 grid(d.B - 1, d.batch);
    if (d.bf16)
        sel_dots_kernel<uint16_t><<<grid, 256, 0, s>>>(anchor, cand_ids, (const uint16_t*)P, (const uint16_t*)Q, T,
                                                       d.B, d.K, d.r, d.V);
    else
        sel_dots_kernel<float><<<grid, 256, 0, s>>>(anchor, cand_ids, (const float*)P, (const float*)Q, T, d.B, d.K,
                                                    d.r, d.V);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (d.K <= 16)
        viterbi_kernel<16><<<d.batch, kWave, 0, s>>>(anchor, cand_ids, cand_logp, T, path, path_score, path_idx, d.B,
                                                     d.K, d.V);
    else
        viterbi_kernel<64><<<d.batch, kWave, 0, s>>>(anchor, cand_ids, cand_logp, T, path, path_score, path_idx, d.B,
                                                     d.K, d.V);
    return hipGetLastError();
}

}  // namespace dfs
