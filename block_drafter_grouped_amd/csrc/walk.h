// The walk of one block over transition tiles held in LDS (K <= 16), shared
// by the fused selector and the single-launch block kernel.  Inco AI post
// "DFlash 2: keep the draft parallel", section "lightweight path selector":
// every adjacent candidate pair is scored first; the only sequential work is
// the walk over those scores, from the last verified token (vLLM
// release-note article on DFlash2, section "two additions").
#pragma once

#include "common.h"

namespace dfs {

// A block whose anchor or candidates are invalid: path -1, score NaN.
__device__ __forceinline__ void write_bad_block(int b, int B, int32_t* path, float* path_score, int32_t* path_idx) {
    for (int t = threadIdx.x; t < B; t += blockDim.x) {
        path[(size_t)b * B + t] = -1;
        if (path_idx) path_idx[(size_t)b * B + t] = -1;
    }
    if (threadIdx.x == 0) path_score[b] = __int_as_float(0x7FC00000);
}


// Wave 0 walks block b over Ts[t-1][j][k] = T_t[j][k], node scores Ls[t][k]
// and candidate ids Cs[t][k] (t = 1..B-1, K <= 16), all in LDS and published
// by a barrier before the call; the other waves return at once.  mode 0:
// best path (Viterbi); 1: greedy; 2: sampled with uniforms Us[t] and
// inv_t = 1 / temperature.  Writes path, path_idx (nullable) and path_score
// of block b.
__device__ __forceinline__ void walk_block_lds(int b, int a, const int32_t (*Cs)[16], const float (*Ls)[16],
                                               const float (*Ts)[16][16], uint8_t (*bp)[16], int mode, float inv_t,
                                               const float* Us, int32_t* __restrict__ path,
                                               float* __restrict__ path_score, int32_t* __restrict__ path_idx,
                                               int B, int K) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (wave != 0) return;

    if (mode != 0) {
        // Greedy / sampled walk (modes 1, 2), with the rules and arithmetic
        // of walk_kernel, on the tiles in LDS: lane k = candidate k.
        const bool on = lane < K;
        const int k = lane & 15;
        int prev = 0;
        float total = 0.f;
        for (int t = 1; t < B; ++t) {
            const float sk = on ? Ls[t][k] + Ts[t - 1][prev][k] : -INFINITY;
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
            if (lane == 0) {
                path[(size_t)b * B + t] = Cs[t][pick];
                if (path_idx) path_idx[(size_t)b * B + t] = pick;
            }
        }
        if (lane == 0) {
            path[(size_t)b * B] = a;
            if (path_idx) path_idx[(size_t)b * B] = -1;
            path_score[b] = total;
        }
        return;
    }

    // Lane 16 g + k: candidate k, predecessors j = 4g .. 4g + 3.  Each lane
    // scans its four j (the first, then a strict comparison), then two
    // butterfly steps combine the groups, the lower j winning ties: the
    // lowest j with the largest score, as a left-to-right scan finds it.
    // delta[k] ends up in all four lanes of k; lane j (group 0) serves
    // delta[j] to the next slot.
    const int k = lane & 15, g = lane >> 4;
    const bool on = k < K;
    float d = on ? Ls[1][k] + Ts[0][0][k] : -INFINITY;
    for (int t = 2; t < B; ++t) {
        float bv = -INFINITY;
        int bi = 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * g + i;
            const float dj = __shfl(d, j, kWave);
            const float c = (j < K) ? dj + Ts[t - 1][j][k] : -INFINITY;
            const bool gt = (i == 0) | (c > bv);
            bv = gt ? c : bv;
            bi = gt ? j : bi;
        }
#pragma unroll
        for (int o = 16; o < kWave; o <<= 1) {
            const float ov = __shfl_xor(bv, o, kWave);
            const int oi = __shfl_xor(bi, o, kWave);
            const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
            bv = take ? ov : bv;
            bi = take ? oi : bi;
        }
        d = on ? bv + Ls[t][k] : -INFINITY;
        if (on && g == 0) bp[t][k] = (uint8_t)bi;
    }
    const float mx = wave_max_f32(d);
    const uint64_t ball = __ballot(on && g == 0 && d == mx);
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


}  // namespace dfs
