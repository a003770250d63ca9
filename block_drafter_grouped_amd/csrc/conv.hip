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
// straight into its MFMA operand registers.  A workgroup owns a 16-column x
// 64-row tile of z; its waves split D and sum their partial tiles in LDS in a
// fixed order, then the same workgroup applies the softmax and the causal
// taps for the 16/ks groups its columns cover.  fp32: a plain VALU kernel.
#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

constexpr int kConvRows = 64;  // rows per workgroup tile (4 MFMA fragments)
constexpr int kConvWaves = 8;  // waves splitting the D reduction

template <int NWK>
__global__ __launch_bounds__(NWK * kWave) void conv_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ wg, uint16_t* __restrict__ y,
    float* __restrict__ y_f32, int rows, int B, int D, int gs, int ks, int C) {
    __shared__ float red[NWK][4][4][kWave];
    __shared__ float zt[kConvRows][17];
    __shared__ float wt[kConvRows][17];

    const int col0 = blockIdx.x * 16;
    const int row0 = blockIdx.y * kConvRows;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int i16 = lane & 15, q = lane >> 4;
    const int nf = min(4, (rows - row0 + 15) / 16);
    const int S = D / 32;
    const int s_beg = (int)((int64_t)S * wave / NWK), s_end = (int)((int64_t)S * (wave + 1) / NWK);

    // MFMA operands: A = generator rows (i = column of z), B = hidden rows
    // (j = row of z); lane holds 8 consecutive channels of one row.
    const uint16_t* arow = wg + (size_t)min(col0 + i16, C - 1) * D + 8 * q;
    const uint16_t* brow[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) brow[f] = h + (size_t)min(row0 + 16 * f + i16, rows - 1) * D + 8 * q;

    f32x4 acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s_beg; s < s_end; ++s) {
        const bf16x8 a = *(const bf16x8*)(arow + 32 * s);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            if (f < nf) {
                const bf16x8 b = *(const bf16x8*)(brow[f] + 32 * s);
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[f], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][f][r][lane] = acc[f][r];
    __syncthreads();

    // Sum the D-split partials in wave order; MFMA output lane l, register r
    // holds z[col 4*(l/16) + r][row l%16] of its fragment.
    for (int e = threadIdx.x; e < 4 * 4 * kWave; e += NWK * kWave) {
        const int f = e / (4 * kWave), r = (e / kWave) & 3, ln = e & (kWave - 1);
        float sum = 0.f;
        for (int w = 0; w < NWK; ++w) sum += red[w][f][r][ln];
        zt[16 * f + (ln & 15)][4 * (ln >> 4) + r] = sum;
    }
    __syncthreads();

    const int ncol = min(16, C - col0);  // a multiple of ks
    const int ng = ncol / ks;
    for (int e = threadIdx.x; e < kConvRows * ng; e += NWK * kWave) {
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
    for (int e = threadIdx.x; e < kConvRows * nch; e += NWK * kWave) {
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

// fp32 correctness path: one workgroup per row.
__global__ __launch_bounds__(256) void conv_f32_kernel(const float* __restrict__ h, const float* __restrict__ wg,
                                                       float* __restrict__ y, float* __restrict__ y_f32, int rows,
                                                       int B, int D, int gs, int ks, int C) {
    extern __shared__ float sm[];  // z[C] then w[C]
    const int row = blockIdx.x, t = row % B;
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

hipError_t launch_conv(const Dims& d, const void* h, const void* wg_cm, void* y, float* y_f32, hipStream_t s) {
    const int C = d.taps();
    if (d.bf16) {
        dim3 grid((C + 15) / 16, (d.rows() + kConvRows - 1) / kConvRows);
        conv_bf16_kernel<kConvWaves><<<grid, kConvWaves * kWave, 0, s>>>(
            (const uint16_t*)h, (const uint16_t*)wg_cm, (uint16_t*)y, y_f32, d.rows(), d.B, d.D, d.gs, d.ks, C);
    } else {
        conv_f32_kernel<<<d.rows(), 256, 2 * (size_t)C * sizeof(float), s>>>(
            (const float*)h, (const float*)wg_cm, (float*)y, y_f32, d.rows(), d.B, d.D, d.gs, d.ks, C);
    }
    return hipGetLastError();
}

}  // namespace dfs
