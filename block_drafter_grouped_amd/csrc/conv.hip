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
// 16/ks groups the columns cover.
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
    {
        const int rr = t0 / 16, cc = t0 % 16, row = row0 + rr, col = col0 + cc;
        float z = 0.f;
        if (row < rows && col < C)
            for (int k = 0; k < kConvSplit; ++k) z += zpart[((size_t)k * rows + row) * C + col];
        zt[rr][cc] = z;
    }
    __syncthreads();
    const int ncol = min(16, C - col0);  // a multiple of ks
    const int ng = ncol / ks;
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
    const int c0 = (col0 / ks) * gs;
    const int nch = ng * gs;
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

// Few rows (at most kConvRowsMax, bf16): the whole conv in one launch, no
// workspace.  One workgroup per (channel group, layer) computes the group's
// ks tap logits over the full D for every row, their softmax, and the causal
// taps of the group's gs channels.  Thread t takes 8-channel chunks t, t +
// NT, ... of the generator rows and of every hidden row (all the loads of a
// chunk in flight together, addresses clamped), the partial sums are reduced
// across each wave in a fixed order and across the waves in order.  The
// hidden rows are read once per group from L2; at 8 rows of the page shape
// that is 320 workgroups of 100 KB each, against two launches and a round
// trip of partials through the workspace for the split-D generator below.
constexpr int kConvRowsMax = 16;

// MR, MK: compile-time bounds of the rows and taps (8 and 2 for the page
// shape at batch 1; 16 and 4 otherwise); NT threads.  With 256 threads
// every workgroup of the page shape (320) is resident at once; 1024 threads
// took 11.0 us against 7.1 us there (two rounds of workgroups).
template <int MR, int MK, int NT>
__global__ __launch_bounds__(NT) void conv_rows_kernel(const uint16_t* __restrict__ h,
                                                        const uint16_t* __restrict__ wg, uint16_t* __restrict__ y,
                                                        float* __restrict__ y_f32, int rows, int B, int D, int gs,
                                                        int ks, int C) {
    __shared__ float part[NT / kWave][MR][MK];  // [wave][row][tap]
    __shared__ float wts[MR][MK];      // tap weights
    const int g = blockIdx.x;
    {  // grid y = layer
        const size_t l = blockIdx.y;
        h += l * rows * D;
        wg += l * C * D;
        y += l * rows * D;
        if (y_f32) y_f32 += l * rows * D;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    float acc[MR][MK];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int j = 0; j < MK; ++j) acc[r][j] = 0.f;
    const int nchunk = D / 8;
    for (int ch = tid; ch < nchunk; ch += NT) {
        float w8[MK][8], h8[MR][8];
#pragma unroll
        for (int j = 0; j < MK; ++j) {
            const uint4 v = *(const uint4*)(wg + (size_t)(g * ks + min(j, ks - 1)) * D + 8 * ch);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w8[j][2 * e] = __uint_as_float(q[e] << 16);
                w8[j][2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const uint4 v = *(const uint4*)(h + (size_t)min(r, rows - 1) * D + 8 * ch);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h8[r][2 * e] = __uint_as_float(q[e] << 16);
                h8[r][2 * e + 1] = __uint_as_float(q[e] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int j = 0; j < MK; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][j] += h8[r][e] * w8[j][e];
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
#pragma unroll
        for (int j = 0; j < MK; ++j) {
            if (r < rows && j < ks) {  // uniform
                const float sm = wave_sum_f32(acc[r][j]);
                if (lane == 0) part[wave][r][j] = sm;
            }
        }
    }
    __syncthreads();
    if (tid < rows) {  // tap logits in wave order, then the softmax over the taps
        const int r = tid;
        float z[MK], m = -INFINITY;
        for (int j = 0; j < ks; ++j) {
            z[j] = part[0][r][j];
            for (int w = 1; w < NT / kWave; ++w) z[j] += part[w][r][j];
            m = fmaxf(m, z[j]);
        }
        float ex[MK], den = 0.f;
        for (int j = 0; j < ks; ++j) {
            ex[j] = expf(z[j] - m);
            den += ex[j];
        }
        for (int j = 0; j < ks; ++j) wts[r][j] = ex[j] / den;
    }
    __syncthreads();
    for (int e = tid; e < rows * gs; e += NT) {  // causal taps, zero before the block
        const int r = e / gs, c = g * gs + e % gs, t = r % B;
        float v = 0.f;
        for (int j = 0; j < ks; ++j)
            if (t - j >= 0) v += wts[r][j] * bf16_to_f32(h[(size_t)(r - j) * D + c]);
        y[(size_t)r * D + c] = f32_to_bf16(v);
        if (y_f32) y_f32[(size_t)r * D + c] = v;
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
        if (d.rows() <= 8 && d.ks <= 2)
            conv_rows_kernel<8, 2, 256><<<grid, 256, 0, s>>>((const uint16_t*)h, (const uint16_t*)wg_cm,
                                                            (uint16_t*)y, y_f32, d.rows(), d.B, d.D, d.gs, d.ks, C);
        else
            conv_rows_kernel<kConvRowsMax, 4, 256><<<grid, 256, 0, s>>>((const uint16_t*)h,
                                                                       (const uint16_t*)wg_cm, (uint16_t*)y, y_f32,
                                                                       d.rows(), d.B, d.D, d.gs, d.ks, C);
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
        conv_apply_kernel<<<grid2, 256, 0, s>>>((const uint16_t*)h, zpart, (uint16_t*)y, y_f32, d.rows(), d.B, d.D,
                                                d.gs, d.ks, C);
    } else {
        conv_f32_kernel<<<dim3(d.rows(), layers), 256, 2 * (size_t)C * sizeof(float), s>>>(
            (const float*)h, (const float*)wg_cm, (float*)y, y_f32, d.rows(), d.B, d.D, d.gs, d.ks, C);
    }
    return hipGetLastError();
}

}  // namespace dfs
