// Step 1 of the draft-block path: grouped dynamic depthwise causal conv
// inside each block (vLLM release-note article on DFlash2, section "two
// additions"; constants from the checkpoint's dflash_config in the RTX 4090
// report, section 4: 16 channels per group, 2 taps).
//
//   z[row, g*ks + j] = <h[row, :], wg_cm[g*ks + j, :]>      (generator)
//   w[row, g, :]     = softmax_j z[row, g*ks + j]            (tap weights)
//   y[b, t, c]       = sum_j w[b*B+t, c/gs, j] * h[b, t-j, c], zero before t = 0
//
// bf16: the generator is a dense [rows, D] x [D, G*ks] contraction and runs
// on MFMA (v_mfma_f32_16x16x32_bf16).  Both operands are K-contiguous in HBM
// (h row-major, the generator channel-major), so every lane loads 16 B
// straight into its MFMA operand registers.  fp32: a plain VALU kernel.
#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

// The generator reads the whole [G*ks, D] weight (6.5 MB at the page shape)
// for only a few rows, so a per-column-tile workgroup would leave most CUs
// idle and be bound by per-CU bandwidth.  The D reduction is therefore split
// over kConvSplit workgroups per tile, whose partial tiles go to the
// workspace; a second kernel sums them in a fixed order, applies the tap
// softmax and the causal taps.  Six splits put the 40 tiles of the page
// shape on 240 CUs: the conv took 14.6, 21.0 and 24.3 us at 64, 128 and 256
// rows against 15.8, 23.0 and 26.6 us with four splits; seven and eight
// (more workgroups than CUs) were slower at 64 and 256 rows.
constexpr int kConvSplit = 6;
constexpr int kConvNarrowRows = 64;
constexpr int kGenWaves = 4;

// NC generator-column fragments x NF row fragments (16 each) per
// workgroup.  Each wave puts the loads of G k-steps in flight together.  A
// wave's k-range and its MFMA order do not depend on NC or NF, so neither
// does z.
template <int NF, int NC, int G>
__global__ __launch_bounds__(kGenWaves * kWave) void conv_gen_kernel(const uint16_t* __restrict__ h,
                                                                   const uint16_t* __restrict__ wg,
                                                                   float* __restrict__ zpart, int rows, int D,
                                                                   int C) {
    // grid z = layer * kConvSplit + split; layers are independent [rows, D]
    // inputs with their own generator.
    __shared__ float red[kGenWaves][NC][NF][4][kWave];
    const int col0 = blockIdx.x * 16 * NC;
    const int row0 = blockIdx.y * 16 * NF;
    const int split = blockIdx.z % kConvSplit, layer = blockIdx.z / kConvSplit;
    h += (size_t)layer * rows * D;
    wg += (size_t)layer * C * D;
    zpart += (size_t)layer * kConvSplit * rows * C;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int i16 = lane & 15, q = lane >> 4;
    const int nf = min(NF, (rows - row0 + 15) / 16);
    const int S = D / 32;
    const int w_beg = (int)((int64_t)S * split / kConvSplit), w_end = (int)((int64_t)S * (split + 1) / kConvSplit);
    const int s_beg = w_beg + (w_end - w_beg) * wave / kGenWaves;
    const int s_end = w_beg + (w_end - w_beg) * (wave + 1) / kGenWaves;

    // MFMA operands: A = generator rows (i = column of z), B = hidden rows
    // (j = row of z); each lane loads 8 consecutive channels of one row.
    // Columns past C read row C - 1 again; their results are dropped.
    const uint16_t* arow[NC];
#pragma unroll
    for (int cf = 0; cf < NC; ++cf) arow[cf] = wg + (size_t)min(col0 + 16 * cf + i16, C - 1) * D + 8 * q;
    const uint16_t* brow[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) brow[f] = h + (size_t)min(row0 + 16 * f + i16, rows - 1) * D + 8 * q;

    f32x4 acc[NC][NF];
#pragma unroll
    for (int cf = 0; cf < NC; ++cf)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[cf][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_beg; s0 < s_end; s0 += G) {
        bf16x8 av[G][NC], bv[G][NF];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int s = min(s0 + u, s_end - 1);
#pragma unroll
            for (int cf = 0; cf < NC; ++cf) av[u][cf] = *(const bf16x8*)(arow[cf] + 32 * s);
#pragma unroll
            for (int f = 0; f < NF; ++f)
                if (f < nf) bv[u][f] = *(const bf16x8*)(brow[f] + 32 * s);
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (s0 + u < s_end) {
#pragma unroll
                for (int cf = 0; cf < NC; ++cf)
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        if (f < nf)
                            acc[cf][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][cf], bv[u][f], acc[cf][f], 0,
                                                                                 0, 0);
            }
        }
    }
#pragma unroll
    for (int cf = 0; cf < NC; ++cf)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][cf][f][r][lane] = acc[cf][f][r];
    __syncthreads();
    // Sum the waves in order; MFMA output lane l, register r holds
    // z[col 4*(l/16) + r][row l%16] of its fragment pair.
    for (int e = threadIdx.x; e < NC * NF * 4 * kWave; e += kGenWaves * kWave) {
        const int cf = e / (NF * 4 * kWave), f = (e / (4 * kWave)) % NF, r = (e / kWave) & 3, ln = e & (kWave - 1);
        const int row = row0 + 16 * f + (ln & 15), col = col0 + 16 * cf + 4 * (ln >> 4) + r;
        if (row >= rows || col >= C) continue;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kGenWaves; ++w) sum += red[w][cf][f][r][ln];
        zpart[((size_t)split * rows + row) * C + col] = sum;
    }
}

// Sums the split partials of a 16-column x 16-row tile of z in split order,
// applies the softmax over each group's taps, then the causal taps to the
// 16/ks groups the columns cover.  With gs % 8 == 0 a thread computes 8
// consecutive channels of one row from 16-B loads of the hidden rows, and
// the loads of its first 8 channels go out before the partial sums, which
// they do not depend on: the tile's loads then take one round instead of a
// round per output.  MK: compile-time bound of the taps.
template <int MK>
__global__ __launch_bounds__(256) void conv_apply_kernel(const uint16_t* __restrict__ h,
                                                         const float* __restrict__ zpart, uint16_t* __restrict__ y,
                                                         float* __restrict__ y_f32, int rows, int B, int D, int gs,
                                                         int ks, int C) {
    __shared__ float zt[16][17];
    __shared__ float wt[16][17];
    const int col0 = blockIdx.x * 16, row0 = blockIdx.y * 16;
    const int t0 = threadIdx.x;
    {  // grid z = layer
        const size_t l = blockIdx.z;
        h += l * rows * D;
        zpart += l * kConvSplit * rows * C;
        y += l * rows * D;
        if (y_f32) y_f32 += l * rows * D;
    }
    const int ncol = min(16, C - col0);  // a multiple of ks
    const int ng = ncol / ks;
    const int c0 = (col0 / ks) * gs;
    const int nch = ng * gs;
    const bool vec = gs % 8 == 0;
    const int nvec = vec ? 16 * (nch / 8) : 0;  // 8-channel outputs of the tile
    // Hidden rows r, r - 1, ... at this thread's first 8 channels (addresses
    // clamped; rows before the block or past the end are not used).
    auto hvec = [&](int e, uint4 (&hv)[MK]) {
        const int rr = e / (nch / 8), row = min(row0 + rr, rows - 1), c = c0 + 8 * (e % (nch / 8));
#pragma unroll
        for (int j = 0; j < MK; ++j) hv[j] = *(const uint4*)(h + (size_t)max(row - j, 0) * D + c);
    };
    uint4 hv0[MK];
    if (vec) hvec(min(t0, nvec - 1), hv0);
    {
        const int rr = t0 / 16, cc = t0 % 16, row = row0 + rr, col = col0 + cc;
        float z = 0.f;
        if (row < rows && col < C)
            for (int k = 0; k < kConvSplit; ++k) z += zpart[((size_t)k * rows + row) * C + col];
        zt[rr][cc] = z;
    }
    __syncthreads();
    for (int e = t0; e < 16 * ng; e += blockDim.x) {
        const int rr = e / ng, gl = e % ng;
        float m = -INFINITY;
        for (int j = 0; j < ks; ++j) m = fmaxf(m, zt[rr][gl * ks + j]);
        float ex[4], den = 0.f;
        for (int j = 0; j < ks; ++j) {
            ex[j] = expf(zt[rr][gl * ks + j] - m);
            den += ex[j];
        }
        for (int j = 0; j < ks; ++j) wt[rr][gl * ks + j] = ex[j] / den;
    }
    __syncthreads();
    if (vec) {
        for (int e = t0; e < nvec; e += blockDim.x) {
            uint4 hv[MK];
            if (e == t0) {
#pragma unroll
                for (int j = 0; j < MK; ++j) hv[j] = hv0[j];
            } else {
                hvec(e, hv);
            }
            const int rr = e / (nch / 8), row = row0 + rr, cl = 8 * (e % (nch / 8)), gl = cl / gs;
            if (row >= rows) continue;
            const int t = row % B;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < MK; ++j) {
                if (j < ks && t - j >= 0) {
                    const float wj = wt[rr][gl * ks + j];
                    const uint32_t q[4] = {hv[j].x, hv[j].y, hv[j].z, hv[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] += wj * __uint_as_float(q[i] << 16);
                        v[2 * i + 1] += wj * __uint_as_float(q[i] & 0xFFFF0000u);
                    }
                }
            }
            const size_t o = (size_t)row * D + c0 + cl;
            uint32_t packed[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                packed[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
            *(uint4*)(y + o) = uint4{packed[0], packed[1], packed[2], packed[3]};
            if (y_f32) {
                *(f32x4*)(y_f32 + o) = f32x4{v[0], v[1], v[2], v[3]};
                *(f32x4*)(y_f32 + o + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
        return;
    }
    for (int e = t0; e < 16 * nch; e += blockDim.x) {
        const int rr = e / nch, cc = e % nch;
        const int row = row0 + rr;
        if (row >= rows) continue;
        const int t = row % B, c = c0 + cc, gl = cc / gs;
        float v = 0.f;
        for (int j = 0; j < ks; ++j)
            if (t - j >= 0) v += wt[rr][gl * ks + j] * bf16_to_f32(h[(size_t)(row - j) * D + c]);
        y[(size_t)row * D + c] = f32_to_bf16(v);
        if (y_f32) y_f32[(size_t)row * D + c] = v;
    }
}

// Sums each of N values (N = 16 or 64) over the 64 lanes of a wave in one
// transposed butterfly: every step halves the values a lane holds and
// exchanges the other half with the partner lane, so N sums cost about N
// exchanges instead of N full reductions.  The steps pair lanes across bit
// 5 (v_permlane32_swap), bit 4 (v_permlane16_swap), then bits 3, 2, 1, 0
// (DPP row mirror, half-row mirror, quad permutes); a pair is added in a
// fixed order, so the result does not vary from run to run.  On return the
// wave's sum of value o is in lane 4 o (N = 16; lanes 4 o .. 4 o + 3 hold
// it) or lane o (N = 64).
template <int N>
__device__ __forceinline__ float wave_sum_transposed(const float (&v)[N]) {
    static_assert(N == 16 || N == 64, "16 or 64 values");
    const int lane = threadIdx.x & (kWave - 1);
    float w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {  // lanes < 32 keep value i, lanes >= 32 value i + N/2
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + N / 2]), false,
                                                        false);
        w[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    float u[N / 4];
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {  // even rows of 16 lanes keep value i, odd rows i + N/4
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[i]), __float_as_uint(w[i + N / 4]), false,
                                                        false);
        u[i] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    // A lane keeps the half its bit selects and sends the other half to the
    // partner, whose bit is the opposite.
    auto halve = [&](float a, float b, bool bit, auto dpp) {
        const float send = bit ? a : b;
        return (bit ? b : a) + dpp(send);
    };
    const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
    const auto mir = [](float x) { return dpp_f32<kDppMirror>(x); };
    const auto hmir = [](float x) { return dpp_f32<kDppHalfMirror>(x); };
    const auto x2 = [](float x) { return dpp_f32<kDppQuadXor2>(x); };
    const auto x1 = [](float x) { return dpp_f32<kDppQuadXor1>(x); };
    if constexpr (N == 16) {
        const float t0 = halve(u[0], u[2], b3, mir), t1 = halve(u[1], u[3], b3, mir);
        float s = halve(t0, t1, b2, hmir);
        s += x2(s);
        return s + x1(s);
    } else {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = halve(u[i], u[i + 8], b3, mir);
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = halve(t[i], t[i + 4], b2, hmir);
        const float r0 = halve(q[0], q[2], b1, x2), r1 = halve(q[1], q[3], b1, x2);
        return halve(r0, r1, b0, x1);
    }
}

// Few rows (at most kConvRowsMax, bf16): the whole conv in one launch, no
// workspace.  One workgroup per (channel group, layer) computes the group's
// ks tap logits over the full D for every row, their softmax, and the causal
// taps of the group's gs channels.  Thread t takes 8-channel chunks t, t +
// NT, ... of the generator rows and of every hidden row.  At 8 rows of the
// page shape that is 320 workgroups, all resident at once, each reading the
// hidden rows (80 KB, from L2) and its generator rows (20 KB).
//
// Timestamped at the page shape, the workgroup of an earlier form (256
// threads, one chunk's loads at a time) was a chain of latencies: three
// rounds of loads (2.7 us), sixteen wave reductions one after another (1.2
// us), the softmax behind a barrier (0.5 us), then a round trip for the
// causal taps' hidden values (0.6 us).  Here the loads of CPT chunks go out
// together, the hidden values of the causal taps are loaded first (they do
// not depend on the tap weights), the partial sums take one transposed wave
// reduction, and each thread of the causal taps forms its row's softmax from
// the wave partials, with no branch.  Measured per call (graph-replayed, 8
// rows): 6.4 -> 4.9 us at D 5120 and 5.1 -> 3.6 us at D 2560 with 320
// threads (two chunks per thread at D 5120, one at D 2560); 256 threads
// with three chunks took 5.5 us at D 5120, 384 threads 5.7 us, 640 threads
// 6.7 us, and two groups per workgroup (256 workgroups, no CU running two)
// 5.9 us.  At 16 rows (256 threads, one chunk in flight): 12.3 -> 10.2 us
// and 9.0 -> 6.3 us.
constexpr int kConvRowsMax = 16;

// MR, MK: compile-time bounds of the rows and taps (8 and 2 for the page
// shape at batch 1; 16 and 4 otherwise); NT threads; CPT chunks per thread
// in flight together.
template <int MR, int MK, int NT, int CPT>
__global__ __launch_bounds__(NT) void conv_rows_kernel(const uint16_t* __restrict__ h,
                                                        const uint16_t* __restrict__ wg, uint16_t* __restrict__ y,
                                                        float* __restrict__ y_f32, int rows, int B, int D, int gs,
                                                        int ks, int C) {
    constexpr int NWV = NT / kWave, NV = MR * MK;
    __shared__ float part[NWV][NV];  // [wave][row * MK + tap]: each wave's sums
    const int g = blockIdx.x;
    {  // grid y = layer
        const size_t l = blockIdx.y;
        h += l * rows * D;
        wg += l * C * D;
        y += l * rows * D;
        if (y_f32) y_f32 += l * rows * D;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    // This thread's first causal-tap output (row r0, channel c0) and its
    // hidden values (rows before the block are never used).
    const int napply = rows * gs;
    const int e0 = min(tid, napply - 1);
    const int r0 = e0 / gs, c0 = g * gs + e0 % gs, t0 = r0 % B;
    float hp[MK];
#pragma unroll
    for (int j = 0; j < MK; ++j) hp[j] = bf16_to_f32(h[(size_t)max(r0 - j, 0) * D + c0]);

    const uint16_t* wrow[MK];
#pragma unroll
    for (int j = 0; j < MK; ++j) wrow[j] = wg + (size_t)(g * ks + min(j, ks - 1)) * D;
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
    const int nchunk = D / 8;
    for (int cb = tid; cb < nchunk; cb += NT * CPT) {
        uint4 wv[CPT][MK], hv[CPT][MR];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ch = min(cb + NT * i, nchunk - 1);
#pragma unroll
            for (int j = 0; j < MK; ++j) wv[i][j] = *(const uint4*)(wrow[j] + 8 * ch);
#pragma unroll
            for (int r = 0; r < MR; ++r) hv[i][r] = *(const uint4*)(h + (size_t)min(r, rows - 1) * D + 8 * ch);
        }
        // Every load above is issued before the first is used: a chunk past
        // the end (its address clamped) is zeroed instead of branched around,
        // and the scheduler may not sink the loads below this point.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const bool live = cb + NT * i < nchunk;
            float w8[MK][8];
#pragma unroll
            for (int j = 0; j < MK; ++j) {
                const uint4 v = wv[i][j];
                const uint32_t q[4] = {live ? v.x : 0u, live ? v.y : 0u, live ? v.z : 0u, live ? v.w : 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w8[j][2 * e] = __uint_as_float(q[e] << 16);
                    w8[j][2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
                }
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const uint4 v = hv[i][r];
                const uint32_t q[4] = {live ? v.x : 0u, live ? v.y : 0u, live ? v.z : 0u, live ? v.w : 0u};
                float h8[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h8[2 * e] = __uint_as_float(q[e] << 16);
                    h8[2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
                }
#pragma unroll
                for (int j = 0; j < MK; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r * MK + j] += h8[e] * w8[j][e];
            }
        }
    }
    {
        const float sm = wave_sum_transposed<NV>(acc);
        if ((lane & (kWave / NV - 1)) == 0) part[wave][lane / (kWave / NV)] = sm;
    }
    __syncthreads();
    // Causal taps, zero before the block: the tap logits are the wave
    // partials summed in wave order, then their softmax (taps past ks get
    // weight 0).
    auto tap = [&](int r, int c, int t, const float (&hv)[MK]) {
        float z[MK], m = -INFINITY;
#pragma unroll
        for (int j = 0; j < MK; ++j) {
            float zz = part[0][r * MK + j];
#pragma unroll
            for (int w = 1; w < NWV; ++w) zz += part[w][r * MK + j];
            z[j] = j < ks ? zz : -INFINITY;
            m = fmaxf(m, z[j]);
        }
        float ex[MK], den = 0.f;
#pragma unroll
        for (int j = 0; j < MK; ++j) {
            ex[j] = j < ks ? expf(z[j] - m) : 0.f;
            den += ex[j];
        }
        const float inv = 1.f / den;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < MK; ++j)
            if (j < ks && t - j >= 0) v += (ex[j] * inv) * hv[j];
        y[(size_t)r * D + c] = f32_to_bf16(v);
        if (y_f32) y_f32[(size_t)r * D + c] = v;
    };
    if (tid < napply) tap(r0, c0, t0, hp);
    for (int e = tid + NT; e < napply; e += NT) {
        const int r = e / gs, c = g * gs + e % gs, t = r % B;
        float hv[MK];
#pragma unroll
        for (int j = 0; j < MK; ++j) hv[j] = bf16_to_f32(h[(size_t)max(r - j, 0) * D + c]);
        tap(r, c, t, hv);
    }
}

// fp32 correctness path: one workgroup per row.
__global__ __launch_bounds__(256) void conv_f32_kernel(const float* __restrict__ h, const float* __restrict__ wg,
                                                       float* __restrict__ y, float* __restrict__ y_f32, int rows,
                                                       int B, int D, int gs, int ks, int C) {
    extern __shared__ float sm[];  // z[C] then w[C]
    const int row = blockIdx.x, t = row % B;
    {  // grid y = layer
        const size_t l = blockIdx.y;
        h += l * rows * D;
        wg += l * C * D;
        y += l * rows * D;
        if (y_f32) y_f32 += l * rows * D;
    }
    for (int col = threadIdx.x; col < C; col += blockDim.x) {
        float acc = 0.f;
        for (int c = 0; c < D; ++c) acc += h[(size_t)row * D + c] * wg[(size_t)col * D + c];
        sm[col] = acc;
    }
    __syncthreads();
    for (int g = threadIdx.x; g < C / ks; g += blockDim.x) {
        float m = -INFINITY;
        for (int j = 0; j < ks; ++j) m = fmaxf(m, sm[g * ks + j]);
        float den = 0.f;
        for (int j = 0; j < ks; ++j) den += expf(sm[g * ks + j] - m);
        for (int j = 0; j < ks; ++j) sm[C + g * ks + j] = expf(sm[g * ks + j] - m) / den;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        const int g = c / gs;
        float v = 0.f;
        for (int j = 0; j < ks; ++j)
            if (t - j >= 0) v += sm[C + g * ks + j] * h[(size_t)(row - j) * D + c];
        y[(size_t)row * D + c] = v;
        if (y_f32) y_f32[(size_t)row * D + c] = v;
    }
}

}  // namespace

size_t conv_ws_bytes(const Dims& d) {
    // only the split-D generator (bf16, more than kConvRowsMax rows) keeps partials
    return d.bf16 && d.rows() > kConvRowsMax ? (size_t)kConvSplit * d.rows() * d.taps() * sizeof(float) : 0;
}

hipError_t launch_conv(const Dims& d, const void* h, const void* wg_cm, void* y, float* y_f32, char* ws,
                       hipStream_t s, int layers) {
    const int C = d.taps();
    if (d.ks == 1 && !y_f32) {
        // One tap: the tap softmax is 1, so y = h (already in the dtype).
        return hipMemcpyAsync(y, h, (size_t)layers * d.rows() * d.D * (d.bf16 ? 2 : 4), hipMemcpyDeviceToDevice,
                              s);
    }
    if (d.bf16 && d.rows() <= kConvRowsMax) {
        const dim3 grid(d.groups(), layers);
        const auto* hb = (const uint16_t*)h;
        const auto* wb = (const uint16_t*)wg_cm;
        auto* yb = (uint16_t*)y;
        if (d.rows() <= 8 && d.ks <= 2) {
            if (d.D / 8 > 320)
                conv_rows_kernel<8, 2, 320, 2><<<grid, 320, 0, s>>>(hb, wb, yb, y_f32, d.rows(), d.B, d.D, d.gs, d.ks,
                                                                    C);
            else
                conv_rows_kernel<8, 2, 320, 1><<<grid, 320, 0, s>>>(hb, wb, yb, y_f32, d.rows(), d.B, d.D, d.gs, d.ks,
                                                                    C);
        } else {
            conv_rows_kernel<kConvRowsMax, 4, 256, 1><<<grid, 256, 0, s>>>(hb, wb, yb, y_f32, d.rows(), d.B, d.D, d.gs,
                                                                          d.ks, C);
        }
        return hipGetLastError();
    }
    if (d.bf16) {
        float* zpart = (float*)(ws + ws_layout(d).zpart);  // more than kConvRowsMax rows here
        if (d.rows() <= kConvNarrowRows) {
            // Up to kConvNarrowRows rows: 16 columns x 64 rows, so that enough
            // workgroups still stream the generator (two k-steps in flight:
            // 40 rows, 16.6 -> 14.4 us).
            dim3 grid((C + 15) / 16, (d.rows() + 63) / 64, kConvSplit * layers);
            conv_gen_kernel<4, 1, 2><<<grid, kGenWaves * kWave, 0, s>>>((const uint16_t*)h, (const uint16_t*)wg_cm,
                                                                       zpart, d.rows(), d.D, C);
        } else {
            // Many rows: 64 x 64 tiles of z, so that each hidden row is read
            // by C / 64 workgroups instead of C / 16.  Two k-steps in flight
            // per wave: at 256 rows of the page shape the conv took 26.8 us,
            // against 28.4 us with four and 27.7 us with one.
            dim3 grid((C + 63) / 64, (d.rows() + 63) / 64, kConvSplit * layers);
            conv_gen_kernel<4, 4, 2><<<grid, kGenWaves * kWave, 0, s>>>((const uint16_t*)h, (const uint16_t*)wg_cm,
                                                                       zpart, d.rows(), d.D, C);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        dim3 grid2((C + 15) / 16, (d.rows() + 15) / 16, layers);
        if (d.ks <= 2)
            conv_apply_kernel<2><<<grid2, 256, 0, s>>>((const uint16_t*)h, zpart, (uint16_t*)y, y_f32, d.rows(), d.B,
                                                       d.D, d.gs, d.ks, C);
        else
            conv_apply_kernel<4><<<grid2, 256, 0, s>>>((const uint16_t*)h, zpart, (uint16_t*)y, y_f32, d.rows(), d.B,
                                                       d.D, d.gs, d.ks, C);
    } else {
        conv_f32_kernel<<<dim3(d.rows(), layers), 256, 2 * (size_t)C * sizeof(float), s>>>(
            (const float*)h, (const float*)wg_cm, (float*)y, y_f32, d.rows(), d.B, d.D, d.gs, d.ks, C);
    }
    return hipGetLastError();
}

}  // namespace dfs
