// The selector of one block from LDS (K <= 16): transition tiles on MFMA and
// the walk over them, shared by the fused selector kernel and the
// single-launch block kernel.  Inco AI post
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
    // scans its four j (the first, then a strict comparison); two butterfly
    // steps then combine the four groups, the lower j winning ties: the
    // lowest j with the largest score, as a left-to-right scan finds it.
    //  - delta reaches the lanes through 16 floats of LDS: lanes 0 .. 15
    //    write delta[k], every lane reads its group's delta[4g .. 4g + 3]
    //    with one 16-B broadcast read;
    //  - the butterflies exchange across rows with v_permlane16_swap and
    //    v_permlane32_swap, which give every lane both its own and its
    //    partner's pair (a symmetric combine needs no more);
    //  - the next slot's T and node scores are read while this slot's
    //    scores are formed.
    // (Shuffles through the LDS unit for all three exchanges cost about 1000
    // cycles per slot; this walk takes a few hundred.)
    __shared__ __attribute__((aligned(16))) float dsh[16];
    const int k = lane & 15, g = lane >> 4;
    const bool on = k < K;
    auto pair_max = [](float& bv, int& bi, float ov, int oi) {
        const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
        bv = take ? ov : bv;
        bi = take ? oi : bi;
    };
    float d = on ? Ls[1][k] + Ts[0][0][k] : -INFINITY;
    float tn[4], ln = 0.f;
    auto fetch = [&](int t) {  // T_t[4g + i][k] and the node score of slot t
#pragma unroll
        for (int i = 0; i < 4; ++i) tn[i] = Ts[t - 1][4 * g + i][k];
        ln = Ls[t][k];
    };
    if (B > 2) fetch(2);
    for (int t = 2; t < B; ++t) {
        float tc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tc[i] = tn[i];
        const float lc = ln;
        if (lane < 16) dsh[lane] = d;
        const f32x4 d4 = *(const f32x4*)&dsh[4 * g];
        fetch(min(t + 1, B - 1));  // unconditional (the last slot re-reads itself): no wait for it here
        float bv = -INFINITY;
        int bi = 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * g + i;
            const float c = (j < K) ? d4[i] + tc[i] : -INFINITY;
            const bool gt = (i == 0) | (c > bv);
            bv = gt ? c : bv;
            bi = gt ? j : bi;
        }
        {
            const auto v = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
            const auto x = __builtin_amdgcn_permlane16_swap((uint32_t)bi, (uint32_t)bi, false, false);
            bv = __uint_as_float(v[0]);
            bi = (int)x[0];
            pair_max(bv, bi, __uint_as_float(v[1]), (int)x[1]);
        }
        {
            const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
            const auto x = __builtin_amdgcn_permlane32_swap((uint32_t)bi, (uint32_t)bi, false, false);
            bv = __uint_as_float(v[0]);
            bi = (int)x[0];
            pair_max(bv, bi, __uint_as_float(v[1]), (int)x[1]);
        }
        d = on ? bv + lc : -INFINITY;
        if (on && g == 0) bp[t][k] = (uint8_t)bi;
    }
    const float mx = wave_max_f32(d);
    const uint64_t ball = __ballot(on && g == 0 && d == mx);
    // Backtrack.  The back-pointer table (bytes bp[t][k], word 4 t + k / 4)
    // goes to registers, four words per lane; the chase then runs on the
    // scalar unit through v_readlane, and lane t keeps the index of slot t,
    // so that every lane writes its own path element (no dependent LDS read
    // per slot).
    uint32_t bpw[4];
    const int nw = 4 * B;  // words in use
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int w = lane + 64 * m;
        bpw[m] = (m * 64 < nw) ? ((const uint32_t*)bp)[min(w, nw - 1)] : 0u;
    }
    int kk = __ffsll((unsigned long long)ball) - 1;  // uniform
    int kt = 0;                                     // lane t: the index of slot t
    for (int t = B - 1; t >= 1; --t) {
        kt = lane == t ? kk : kt;
        if (t >= 2) {
            const int w = 4 * t + (kk >> 2);
            const int m = w >> 6, l = w & 63;
            const uint32_t word = m == 0   ? (uint32_t)__builtin_amdgcn_readlane((int)bpw[0], l)
                                  : m == 1 ? (uint32_t)__builtin_amdgcn_readlane((int)bpw[1], l)
                                  : m == 2 ? (uint32_t)__builtin_amdgcn_readlane((int)bpw[2], l)
                                           : (uint32_t)__builtin_amdgcn_readlane((int)bpw[3], l);
            kk = (int)((word >> (8 * (kk & 3))) & 0xFFu);
        }
    }
    if (lane < B) {
        path[(size_t)b * B + lane] = lane == 0 ? a : Cs[lane][kt];
        if (path_idx) path_idx[(size_t)b * B + lane] = lane == 0 ? -1 : kt;
    }
    if (lane == 0) path_score[b] = mx;
}


// One transition tile T_t (16 x 16, K <= 16) on MFMA, as one wave:
// A = P rows (or P (*) H rows with a context gate) of the predecessors, B =
// Q rows of the successors.  Lane 16 q + i holds predecessor row pr and
// successor row qr of index i (both already offset by 8 q elements) and the
// gate row gr (offset the same, or null); every gather of the tile is in
// flight at once.  With a gate, P (*) H is formed in fp32 and split into
// bf16 hi + lo parts that take one MFMA each, so the product keeps about 16
// significant bits beyond bf16 (the rounding of the split is 2^-17
// relative).  Returns the lane's part of the tile: T[4 q + rr][i], rr = 0..3.
__device__ __forceinline__ f32x4 transition_tile_mfma(const uint16_t* __restrict__ pr, const uint16_t* __restrict__ qr,
                                                      const float* __restrict__ gr, int nks) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!gr) {
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
    } else {
        for (int s0 = 0; s0 < nks; s0 += 4) {
            uint4 pv[4];
            bf16x8 bv[4];
            f32x4 g0[4], g1[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = min(s0 + u, nks - 1);
                pv[u] = *(const uint4*)(pr + 32 * s);
                bv[u] = *(const bf16x8*)(qr + 32 * s);
                g0[u] = *(const f32x4*)(gr + 32 * s);
                g1[u] = *(const f32x4*)(gr + 32 * s + 4);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (s0 + u >= nks) continue;
                const uint32_t w4[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
                uint16_t hi[8], lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t bits = (e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16);
                    const float x = __uint_as_float(bits) * (e < 4 ? g0[u][e] : g1[u][e - 4]);
                    hi[e] = f32_to_bf16(x);
                    lo[e] = f32_to_bf16(x - bf16_to_f32(hi[e]));
                }
                bf16x8 ah, al;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ah[e] = __builtin_bit_cast(__bf16, hi[e]);
                    al[e] = __builtin_bit_cast(__bf16, lo[e]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv[u], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv[u], acc, 0, 0, 0);
            }
        }
    }
    return acc;
}

// Transition tiles of one block on MFMA, from candidates already in LDS:
// Cs[t][k] (ids) for t = 1..B-1, a valid anchor, and a barrier between
// filling them and this call.  Every thread of the workgroup calls it.  Wave
// w computes T_t for t = 1 + w, 1 + w + NWS, ... into LDS (row gate_rows +
// t * r of the gate goes with slot t).
template <int NWS>
__device__ __forceinline__ void transition_tiles_mfma(int a, const int32_t (*Cs)[16], float (*Ts)[16][16],
                                                      const uint16_t* __restrict__ P,
                                                      const uint16_t* __restrict__ Q,
                                                      const float* __restrict__ gate_rows, int B, int K, int r) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int i16 = lane & 15, q = lane >> 4, kk = min(i16, K - 1);
    for (int t = 1 + wave; t < B; t += NWS) {
        const int pa = (t == 1) ? a : Cs[t - 1][kk];
        const int qb = Cs[t][kk];
        const f32x4 acc = transition_tile_mfma(P + (size_t)pa * r + 8 * q, Q + (size_t)qb * r + 8 * q,
                                               gate_rows ? gate_rows + (size_t)t * r + 8 * q : nullptr, r / 32);
        // lane holds T_t[4q + rr][i16]
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Ts[t - 1][4 * q + rr][i16] = acc[rr];
    }
}


// The whole selector of block b (bf16 tables, K <= 16, r % 32 == 0): stages
// the block's candidates (global cand_ids / cand_logp) and uniforms in LDS,
// marks a block with an invalid anchor or id, computes the transition tiles
// and walks.  Every thread of the workgroup calls it; Cs, Ls, bp hold at
// least B rows, Ts at least B - 1 tiles, Us B entries.
template <int NWS>
__device__ __forceinline__ void select_block(int b, const int32_t* __restrict__ anchor,
                                             const int32_t* __restrict__ cand_ids,
                                             const float* __restrict__ cand_logp, const uint16_t* __restrict__ P,
                                             const uint16_t* __restrict__ Q, const float* __restrict__ gate, int mode,
                                             float temperature, const float* __restrict__ uniforms,
                                             int32_t* __restrict__ path, float* __restrict__ path_score,
                                             int32_t* __restrict__ path_idx, int B, int K, int r, int V,
                                             int32_t (*Cs)[16], float (*Ls)[16], float (*Ts)[16][16],
                                             uint8_t (*bp)[16], float* Us) {
    const int t0 = threadIdx.x;
    const int a = anchor[b];
    bool bad = (a < 0 || a >= V);
    for (int i = t0; i < (B - 1) * K; i += NWS * kWave) {
        const int t = 1 + i / K, k = i % K;
        const int id = cand_ids[((size_t)b * B + t) * K + k];
        bad |= (id < 0 || id >= V);
        Cs[t][k] = id;
        Ls[t][k] = cand_logp[((size_t)b * B + t) * K + k];
    }
    if (mode == 2)
        for (int t = t0; t < B; t += NWS * kWave) Us[t] = uniforms[(size_t)b * B + t];
    if (__syncthreads_or(bad)) {
        write_bad_block(b, B, path, path_score, path_idx);
        return;
    }
    transition_tiles_mfma<NWS>(a, Cs, Ts, P, Q, gate ? gate + (size_t)b * B * r : nullptr, B, K, r);
    __syncthreads();
    walk_block_lds(b, a, Cs, Ls, Ts, bp, mode, 1.f / temperature, Us, path, path_score, path_idx, B, K);
}

}  // namespace dfs
