// Step 2 of the draft-block path for more than 8 rows (vLLM release-note
// article on DFlash2, section "two additions": the target's lm_head and
// log-softmax over the block's rows): the logits of every row as one GEMM,
// and the fp32 head.  Both write fp32 logits.  With K <= 16 the GEMM also
// writes per-segment (max, sum of exp) partials and merge_seg_kernel below
// ranks the few segments that can hold a row's top K; otherwise
// slice_topk.hip ranks the logits.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dfs {

namespace {

// Head for many rows (more than 8 per call, up to 256 per pass): a GEMM
// logit[v][row] = <W[v], y[row]> on v_mfma_f32_32x32x16_bf16 that writes
// the fp32 logits (and, MS, the segment partials described below).
//  - One persistent workgroup per CU owns a contiguous vocabulary range and
//    walks it in tiles of TV = 32 TVB rows of W (256 or 512) against a pass
//    of RP hidden rows, in stages of KC channels (64 when D % 64 == 0, else
//    32).
//  - Producer and consumer waves.  The NWB consumer waves split the TV
//    vocabulary rows x RP hidden rows of a tile into blocks of NVB x
//    (8 / NVB) accumulator tiles of 32x32 each; they only read LDS, issue
//    MFMAs and store logits.  Every consumer holds 8 accumulator tiles, so
//    a wider vocabulary tile serves fewer hidden rows per pass and re-reads
//    them fewer times per weight byte.  Four
//    producer waves move the operands by direct global->LDS loads, two for W
//    (a ring of RW stages) and two for the hidden rows (RY stages; L2
//    resident, so a shallower ring).  A wave's count of outstanding memory
//    operations drains in order for its own loads, so each producer waits on
//    exactly its own stage; one barrier per stage then publishes it.  The
//    consumers' logit stores never sit in front of a load in any wave's
//    count, so they drain while the next tile computes.
//  - The loads are issued from inline assembly: the compiler, unable to tell
//    the ring slots apart, would otherwise wait for every load in flight
//    before each LDS read.
//  - An LDS row holds KC / 8 units of 16 B; unit u of row v is stored at
//    unit u ^ f(v) with f(v) = (v >> 2) & 3 (4 units) or (v >> 1) & 7 (8
//    units), so the 32-row operand reads of a wave hit distinct banks in
//    every group of 16 lanes.
//  - The MFMA takes the hidden rows as its A operand, so in the 32x32 output
//    layout a lane holds one vocabulary entry of 16 rows: each store
//    instruction writes whole 128-B lines of two rows.
//  - Loads and MFMAs for rows past the work are skipped: weight rows past a
//    CU's range in its last tile, and (RS) hidden rows past the last row in
//    a partial row pass.
// Ranking inside this kernel was tried twice.  A sorted per-lane list: the
// lists of the 64 lanes of a wave take their insertions at different values,
// so the wave ran nearly every insertion and the epilogue cost about a
// quarter of the kernel.  Appending the logits above a per-tile bound (the
// smallest of the 16 lane-pair maxima of a row) as keys: the ballots and
// scattered 8-B stores of every tile cost more than writing all the logits,
// whose plain stores cost a tenth of the weight stream.  The kernel keeps
// the stores and adds only the (max, sum of exp) of each segment, which
// lets the merge read a few segments of the written logits per row.

template <int KC>
__device__ __forceinline__ int gemm_swz(int row) {
    return KC == 32 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}
template <int KC>
__device__ __forceinline__ int gemm_unit(int row, int u) {
    return row * (KC / 8) + (u ^ gemm_swz<KC>(row));
}

// 16-B global -> LDS copy per lane; lane L writes lds_base + 16 L.  STREAM
// marks data read once (the weight): a non-temporal load, so that it does
// not push the reused hidden rows out of L2.
template <bool STREAM>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(
                         __builtin_amdgcn_readfirstlane(lds_base)),
                     "v"(g)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(
                         __builtin_amdgcn_readfirstlane(lds_base)),
                     "v"(g)
                     : "memory", "m0");
#pragma clang diagnostic pop
}

// The same copy from a wave-uniform base address (an SGPR pair) plus a
// per-lane byte offset: lane L reads sbase + voff and writes lds_base +
// 16 L.  The address arithmetic stays on the scalar unit.  Address math on
// the vector ALU (a 64-bit multiply-add per load) competes with the MFMA
// waves of the same SIMD for issue: in a probe beside 8 MFMA waves, loaders
// with vector-ALU addresses took 850 us for a stream that loaders with
// scalar addresses finished in 529 us (the MFMA work alone took 509 us).
template <bool STREAM>
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(
                         __builtin_amdgcn_readfirstlane(lds_base)),
                     "v"(voff), "s"(sbase)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                         __builtin_amdgcn_readfirstlane(lds_base)),
                     "v"(voff), "s"(sbase)
                     : "memory", "m0");
#pragma clang diagnostic pop
}

// The weight is read once, so its loads are non-temporal (they do not push
// the reused hidden rows out of L2), except with 32-channel stages: there a
// stage reads half of each 128-B weight line and the next stage the other
// half, which has to find the line still in L2.
template <int KC>
constexpr bool kGemmStreamW = KC == 64;

constexpr int kGemmProducers = 4;  // two W loaders, two hidden-row loaders

// s_waitcnt with at most n vector-memory operations outstanding, n in
// 0..48 (a larger n waits for all of them, which is always safe).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define DFS_WAIT_VM(k)                                                                          \
    case k:                                                                                     \
        __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | ((k) & 0xF) | (((k) >> 4) << 14)); \
        break;
#define DFS_WAIT_VM4(k) DFS_WAIT_VM(k) DFS_WAIT_VM(k + 1) DFS_WAIT_VM(k + 2) DFS_WAIT_VM(k + 3)
        DFS_WAIT_VM4(1) DFS_WAIT_VM4(5) DFS_WAIT_VM4(9) DFS_WAIT_VM4(13) DFS_WAIT_VM4(17) DFS_WAIT_VM4(21)
        DFS_WAIT_VM4(25) DFS_WAIT_VM4(29) DFS_WAIT_VM4(33) DFS_WAIT_VM4(37) DFS_WAIT_VM4(41) DFS_WAIT_VM4(45)
#undef DFS_WAIT_VM4
#undef DFS_WAIT_VM
        default:
            __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4));
            break;
    }
}

// Segment partials (MS): besides the logits, every (row, segment) gets the
// (max, sum of exp) of its logits.  A segment is the part of a tile one
// consumer wave holds: the 32 NVB vocabulary entries of its blocks, for one
// row (a row of a wave's tile is held by the 32 lanes of one half-wave, NVB
// per lane).  The ranking kernel below combines the partials into the lse
// and reads only the segments whose maximum can reach the row's top K.
// Reductions over the 32 lanes of each half-wave; every lane receives its
// half's result.  Four DPP steps reduce each 16-lane row; a swizzle that
// swaps the two rows of a half (xor 16) combines them.
__device__ __forceinline__ float swap_rows_of_half(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1F));
}
__device__ __forceinline__ float max_of_half(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppMirror>(x));
    return fmaxf(x, swap_rows_of_half(x));
}
// In a fixed order (the same on every run; the last add is commutative).
__device__ __forceinline__ float sum_of_half(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppHalfMirror>(x);
    x += dpp_f32<kDppMirror>(x);
    return x + swap_rows_of_half(x);
}

// Consumer layout of a configuration: NVW waves across the TV vocabulary
// rows of a tile, NRW across the RP hidden rows of a pass.
template <int NWB, int NVB, int TVB>
struct GemmShape {
    static constexpr int TV = 32 * TVB;
    static constexpr int NRB = 8 / NVB;
    static constexpr int NVW = TVB / NVB;
    static constexpr int NRW = NWB / NVW;
    static constexpr int RP = 32 * NRB * NRW;
    static_assert(NVB * NRB == 8 && TVB % NVB == 0 && NWB % NVW == 0 && NRW >= 1, "consumer layout");
};

template <int NWB, int KC, int RW, int RY, int NVB, int TVB, bool RS, bool MS>
__global__ __launch_bounds__((NWB + kGemmProducers) * kWave) void head_gemm_kernel(
    const uint16_t* __restrict__ y, int rows_total, int D, const uint16_t* __restrict__ W, int V, int nch,
    float* __restrict__ logits, float2* __restrict__ cms, int nt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using G = GemmShape<NWB, NVB, TVB>;
    constexpr int TV = G::TV, RP = G::RP;
    constexpr int UPR = KC / 8;                 // 16-B units per LDS row
    constexpr int RPI = kWave / UPR;            // rows per 1-KB load instruction
    constexpr int WBYTES = TV * KC * 2;         // one W stage
    constexpr int YBYTES = RP * KC * 2;         // one hidden-row stage
    constexpr int WI = WBYTES / 1024 / 2;       // load instructions per W producer per stage
    constexpr int YI = YBYTES / 1024 / 2;       // per hidden-row producer per stage
    static_assert(WI * 2048 == WBYTES && YI * 2048 == YBYTES, "whole load instructions per producer");
    static_assert((RW - 2) * WI <= 48 && (RY - 2) * YI <= 48, "wait counts");
    const int c = blockIdx.x;
    const int row_base = blockIdx.y * RP;
    const int lane = threadIdx.x & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int S = D / KC;
    const int64_t T32 = ((int64_t)V + 31) / 32;
    const int b_beg = (int)(T32 * c / nch), b_end = (int)(T32 * (c + 1) / nch);
    const int v_beg = b_beg * 32, v_end = min(b_end * 32, V);
    const int ntiles = (b_end - b_beg + TVB - 1) / TVB;
    const int total = ntiles * S;
    const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
    const uint32_t ybase = smem_base + RW * WBYTES;

    if (wave >= NWB) {
        // Producers.  Stage g (tile g / S, channel block g % S) goes to slot
        // g % RW (W) or g % RY (hidden rows).  A 1-KB load instruction covers
        // RPI rows x 2 KC bytes; lane L takes row L / UPR, stored unit
        // L % UPR, i.e. logical unit (L % UPR) ^ f(row).
        const bool wl = wave < NWB + 2;
        const int pw = wl ? wave - NWB : wave - NWB - 2;
        // Byte offset of lane L within a load instruction whose RPI rows are
        // all in bounds: row L / UPR of the instruction, logical unit
        // (L % UPR) ^ f(row).  f of tile row RPI n + r depends on n only
        // through its parity (KC 64: f = (4 n + r / 2) & 7 with RPI 8; KC 32:
        // f = (r / 4) & 3 with RPI 16), and a producer's instructions n = pw,
        // pw + 2, ... share one parity, so one offset serves all of them, for
        // W and for the hidden rows alike (both have rows of D elements).
        const int lr = lane / UPR;
        const uint32_t voff = (uint32_t)(lr * D * 2 + 16 * ((lane % UPR) ^ gemm_swz<KC>(RPI * (pw & 1) + lr)));
        // W load instructions of this producer in stage g: instruction n
        // covers tile rows RPI n .. RPI n + RPI - 1 and is skipped when all of
        // them lie past the range (the last tile of the range).
        auto w_count = [&](int g) {
            const int nv = min(TV, v_end - (v_beg + (g / S) * TV));
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < WI; ++i) cnt += (RPI * (pw + 2 * i) < nv) ? 1 : 0;
            return cnt;
        };
        auto issue_w = [&](int g) {
            const int k0 = (g % S) * KC, v0 = v_beg + (g / S) * TV;
            const int nv = min(TV, v_end - v0);
            const uint32_t base = smem_base + (uint32_t)((g % RW) * WBYTES);
            // Instruction n = pw + 2 i.  All address arithmetic is scalar.  A
            // full tile issues straight-line code (a wave stalls on each
            // taken branch); in the last tile of a range n grows with i, so
            // the first instruction past the range ends the stage.
            const uint16_t* wp = W + ((size_t)v0 + RPI * pw) * D + k0;
            if (nv == TV) {
#pragma unroll
                for (int i = 0; i < WI; ++i, wp += (size_t)2 * RPI * D)
                    dma16s<kGemmStreamW<KC>>(wp, voff, base + (pw + 2 * i) * 1024);
                return;
            }
#pragma unroll 1
            for (int i = 0; i < WI; ++i, wp += (size_t)2 * RPI * D) {
                const int n = pw + 2 * i;
                if (RPI * n >= nv) break;  // wave-uniform
                if (RPI * (n + 1) <= nv) {
                    dma16s<kGemmStreamW<KC>>(wp, voff, base + n * 1024);
                } else {
                    // the one instruction across the end of the vocabulary
                    const int vr = RPI * n + lane / UPR;
                    const int u = (lane % UPR) ^ gemm_swz<KC>(vr);
                    const int v = min(v0 + vr, v_end - 1);  // past the range: re-read its last row (cache hit)
                    dma16<kGemmStreamW<KC>>(W + (size_t)v * D + k0 + 8 * u, base + n * 1024);
                }
            }
        };
        // Hidden-row load instructions of this producer per stage: with RS
        // (the last row pass is partial), those whose RPI rows all lie past
        // the last row are skipped.
        const int ny = RS ? rows_total - row_base : RP;
        int y_cnt = YI;
        if (RS) {
            y_cnt = 0;
#pragma unroll
            for (int i = 0; i < YI; ++i) y_cnt += (RPI * (pw + 2 * i) < ny) ? 1 : 0;
        }
        auto issue_y = [&](int g) {
            const int k0 = (g % S) * KC;
            const uint32_t base = ybase + (uint32_t)((g % RY) * YBYTES);
            const uint16_t* yp = y + ((size_t)row_base + RPI * pw) * D + k0;
            if (!RS || ny >= RP) {
#pragma unroll
                for (int i = 0; i < YI; ++i, yp += (size_t)2 * RPI * D)
                    dma16s<false>(yp, voff, base + (pw + 2 * i) * 1024);
                return;
            }
#pragma unroll 1
            for (int i = 0; i < YI; ++i, yp += (size_t)2 * RPI * D) {
                const int n = pw + 2 * i;
                if (RS && RPI * n >= ny) break;  // wave-uniform
                if (!RS || RPI * (n + 1) <= ny) {
                    dma16s<false>(yp, voff, base + n * 1024);
                } else {
                    // the one instruction across the last row
                    const int r = RPI * n + lane / UPR;
                    const int u = (lane % UPR) ^ gemm_swz<KC>(r);
                    const int row = min(row_base + r, rows_total - 1);
                    dma16<false>(y + (size_t)row * D + k0 + 8 * u, base + n * 1024);
                }
            }
        };
        const int R = wl ? RW : RY;
        for (int g = 0; g < R - 1 && g < total; ++g) wl ? issue_w(g) : issue_y(g);
        for (int g = 0; g < total; ++g) {
            // stage g landed: at most the later stages' loads outstanding (a
            // wave's loads complete in order)
            int later = 0;
            for (int g2 = g + 1; g2 <= min(g + R - 2, total - 1); ++g2) later += wl ? w_count(g2) : y_cnt;
            wait_vm(later);
            __syncthreads();  // publish stage g; the slot read in stage g - 1 is free
            if (g + R - 1 < total) wl ? issue_w(g + R - 1) : issue_y(g + R - 1);
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // Consumers.  Wave w computes NVB vocabulary blocks x NRB row blocks of
    // 32x32 (NVB * NRB = 8): vocabulary blocks NVB * (w % NVW) .., row blocks
    // NRB * (w / NVW) ..; NVW waves span the TV vocabulary rows, NRW waves the
    // RP hidden rows.  Per 16 channels a wave reads NVB + NRB operand
    // fragments from LDS for 8 MFMAs.
    constexpr int NRB = G::NRB, NVW = G::NVW;
    const int j = lane & 31, half = lane >> 5;
    const int vw = wave % NVW, rw = wave / NVW;
    // row blocks of this wave that hold rows (RS: the last row pass is
    // partial); the others are skipped
    const int nrb = RS ? min(NRB, max(0, (rows_total - row_base - 32 * rw * NRB + 31) / 32)) : NRB;
    f32x16 acc[NVB][NRB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[vb][rb][r] = 0.f;
    // MS: the wave's list (its vocabulary blocks of the chunk's range) and
    // its segments, one per tile.
    const int nseg = nch * NVW * nt;
    const int list = c * NVW + vw;
    if constexpr (MS) {
        // segments of tiles past this list's range are empty
        for (int tt = ntiles; tt < nt; ++tt) {
            for (int i = lane; i < NRB * 32; i += kWave) {
                const int row = row_base + rw * NRB * 32 + i;
                if (row < rows_total) cms[(size_t)row * nseg + (size_t)list * nt + tt] = make_float2(-INFINITY, 0.f);
            }
        }
    }
    // LDS byte offsets of this lane's operand fragments (row block 0 and
    // vocabulary block 0) at k-substep 0.  The stored unit of logical unit
    // 2 ks + half is (half ^ f(row)) ^ 2 ks, so k-substep ks reads at the
    // offset XOR 32 ks; rows 32 apart share f, so block b sits kBlk b bytes
    // further.  Two registers then address every fragment of a stage.
    constexpr uint32_t kBlk = 32 * KC * 2;
    const uint32_t yo = 16u * (uint32_t)gemm_unit<KC>(rw * NRB * 32 + j, half);
    const uint32_t wo = 16u * (uint32_t)gemm_unit<KC>(vw * NVB * 32 + j, half);
    int tile = 0, st = 0;
    for (int g = 0; g < total; ++g) {
        // vocabulary blocks of this wave that hold rows of the range (the
        // last tile of the range is partial); the others are skipped
        const int nvb = min(NVB, max(0, (v_end - (v_beg + tile * TV) - 32 * vw * NVB + 31) / 32));
        __syncthreads();  // stage g published
        const uint8_t* sw = smem + (size_t)(g % RW) * WBYTES;
        const uint8_t* sy = smem + (size_t)RW * WBYTES + (size_t)(g % RY) * YBYTES;
        // Every MFMA of the stage runs, also for blocks past the end of the
        // range in its last tile (or past the last hidden row): their rows
        // hold copies of the last row or stale data, each output depends on
        // its own weight row and hidden row only, and those results are
        // dropped below.  Straight-line code lets the compiler issue the LDS
        // reads of later fragments ahead of the MFMAs that use earlier ones;
        // with a branch around each block every read waited for its data
        // right before its MFMA.
        // The stage's fragment reads form one sequence, q = ks NF + i: the
        // NRB hidden-row fragments of k-substep ks, then its NVB weight
        // fragments.  Each read is issued kAhead reads before the MFMAs of
        // the weight fragment it runs level with, so the LDS latency hides
        // behind earlier MFMAs (the scheduling barriers keep the compiler
        // from sinking the reads back to their uses, which it does at this
        // register budget).
        constexpr int KS = KC / 16, NF = NRB + NVB, NQ = KS * NF, kAhead = 3;
        bf16x8 F[NQ];
        auto frag = [&](int q) {
            const int ks = q / NF, i = q % NF;
            const uint8_t* p = i < NRB ? sy + (yo ^ (32u * ks)) + kBlk * i : sw + (wo ^ (32u * ks)) + kBlk * (i - NRB);
            return *(const bf16x8*)p;
        };
        int issued = 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const int qa = ks * NF + NRB + vb;
                const int upto = min(qa + kAhead, NQ - 1);
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if (q >= issued && q <= upto) F[q] = frag(q);
                issued = max(issued, upto + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)  // hidden rows as A, weight rows as B: see the store below
                    acc[vb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[ks * NF + rb], F[qa], acc[vb][rb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (st == S - 1) {
            if constexpr (MS) {
                // Segment partials.  Register r of row block rb holds row
                // 8 (r / 4) + 4 half + r % 4 of the block.  Entries past the
                // range (the last tile of a list) read as -inf here; they are
                // not stored either.
                const int vt = v_beg + tile * TV;
                const int seg = list * nt + tile;
                if (nvb < NVB || vt + 32 * (vw * NVB + nvb) > v_end) {
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) {
                        const bool ok = vt + 32 * (vw * NVB + vb) + j < v_end;
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) acc[vb][rb][r] = ok ? acc[vb][rb][r] : -INFINITY;
                    }
                }
                // lanes 0 and 32 store the partials of their half's row
                float2* const ms_lane = cms + (size_t)(4 * half) * nseg + seg;
                const bool ms_writer = j == 0;
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    if (rb >= nrb) continue;  // wave-uniform: no rows in this block
                    const int rowblk = row_base + (rw * NRB + rb) * 32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row0 = rowblk + 8 * (r >> 2) + (r & 3);  // the row of half 0
                        const int row = row0 + 4 * half;
                        float lm = acc[0][rb][r];
#pragma unroll
                        for (int vb = 1; vb < NVB; ++vb) lm = fmaxf(lm, acc[vb][rb][r]);
                        const float m = max_of_half(lm);
                        float sl = 0.f;
                        if (m > -INFINITY) {
#pragma unroll
                            for (int vb = 0; vb < NVB; ++vb) sl += __expf(acc[vb][rb][r] - m);
                        }
                        const float ssum = sum_of_half(sl);
                        if (ms_writer && row < rows_total) ms_lane[(size_t)row0 * nseg] = make_float2(m, ssum);
                        __builtin_amdgcn_sched_barrier(0);  // one row at a time: bounded registers
                    }
                }
            }
            // Tile done.  For vocabulary block vb and row block rb the lane
            // holds logit[v][row] in acc[vb][rb][r], with v = the block's
            // vocabulary entry j and row = its row 8 (r / 4) + 4 half + r % 4.
            // One store instruction (fixed vb, rb, r) thus writes 32
            // consecutive logits of one row from each half-wave: two whole
            // 128-B lines.  (With the operands the other way round each lane
            // held one row, and a 16-B store touched 32 lines, 32 B of each.)
            // Addresses: a wave-uniform base per (row block, vocabulary block,
            // register) and one lane offset (half-wave row, entry j) for all.
            const int vt = v_beg + tile * TV;
            const uint32_t lane_off = (uint32_t)(4 * half * V + j);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                const int row0 = row_base + (rw * NRB + rb) * 32;
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const int v0 = vt + 32 * (vw * NVB + vb);
                    const bool vok = v0 + j < v_end;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rt = 8 * (r >> 2) + (r & 3);
                        float* base = logits + ((size_t)(row0 + rt) * V + v0);
                        if (vok && row0 + rt + 4 * half < rows_total) base[lane_off] = acc[vb][rb][r];
                    }
                }
            }
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[vb][rb][r] = 0.f;
            ++tile;
            st = 0;
        } else {
            ++st;
        }
    }
}

// fp32 path: plain dot products, logits written out.  A thread owns one
// vocabulary row and walks it in 16-B pieces against up to 8 hidden rows at a
// time (the hidden-row addresses are uniform across the wave, so those loads
// are shared); the loads of several pieces are in flight together.
__global__ __launch_bounds__(256) void head_f32_kernel(const float* __restrict__ y, const float* __restrict__ W,
                                                       float* __restrict__ logits, int rows, int D, int V) {
    const int v = blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= V) return;
    const float* wr = W + (size_t)v * D;
    for (int r0 = 0; r0 < rows; r0 += 8) {
        const int nr = min(8, rows - r0);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int c = 0; c < D; c += 4) {
            const f32x4 w = *(const f32x4*)(wr + c);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r < nr) {
                    const f32x4 x = *(const f32x4*)(y + (size_t)(r0 + r) * D + c);
                    acc[r] += x[0] * w[0] + x[1] * w[1] + x[2] * w[2] + x[3] * w[3];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r < nr) logits[(size_t)(r0 + r) * V + v] = acc[r];
    }
}


// Written logits + segment partials -> candidates (K <= 16).  One
// workgroup of 1024 threads per row; wave w looks at segments w, w + 16, ...
//  - lse = M + log S from the segments' (max, sum of exp), combined in a
//    fixed order (lanes, then waves in order).
//  - theta = the minimum over the 16 waves of the largest segment maximum a
//    wave saw (-inf if a wave saw no logit): 16 distinct logits of the row
//    are >= theta, so every logit of the row's top K is >= theta.
//  - Only segments whose maximum is >= theta can hold such a logit; for
//    ordinary logits a few dozen of a row's segments.  They are listed in
//    LDS, and theta is raised to the K-th largest of their maxima, which
//    leaves about K segments.  The workgroup then reads their logits (one
//    contiguous run of at most 256 per segment) with every thread holding
//    several loads in flight, gathers the keys >= theta in LDS and places
//    each by its rank among them (keys are distinct).  With more live
//    segments than the list holds, each wave reads its own segments in turn
//    instead.
//  - If more than kSegGather keys pass (massively tied logits), the key
//    threshold is raised to the exact K-th largest key by bisection,
//    counting the keys >= the midpoint in the same segments; exactly K keys
//    then pass.
constexpr int kSegGather = 2048;
constexpr int kSegLive = 2048;  // live segments listed in LDS
constexpr int kSegUnroll = 16;  // logit loads in flight per thread
constexpr int kSegRefine = 512; // at most this many live segments: tighter theta

struct SegGeom {
    int nch, nvw, nvb, nt, t32, V, span_log2, tv;  // span: 32 nvb logits; tv: tile width
    // vocabulary run [beg, end) of segment sg (list sg / nt, tile sg % nt)
    __device__ __forceinline__ void range(int sg, int& beg, int& end) const {
        const int list = sg / nt, tile = sg - list * nt;
        const int c = list / nvw, vw = list - c * nvw;
        const int vb = (int)((int64_t)t32 * c / nch) * 32;
        const int ve = min((int)((int64_t)t32 * (c + 1) / nch) * 32, V);
        beg = vb + tile * tv + 32 * vw * nvb;
        end = min(beg + 32 * nvb, ve);
    }
};

__global__ __launch_bounds__(1024) void merge_seg_kernel(const float* __restrict__ logits,
                                                         const float2* __restrict__ cms, SegGeom gm, int K,
                                                         int32_t* __restrict__ cand_ids,
                                                         float* __restrict__ cand_logp,
                                                         float* __restrict__ lse_out) {
    __shared__ uint64_t cand[kSegGather];
    __shared__ int lbeg[kSegLive], lend[kSegLive];
    __shared__ float lmax[kSegLive];
    __shared__ int lbeg2[kSegRefine], lend2[kSegRefine];
    __shared__ int nlive, nlive2;
    __shared__ uint32_t th2_code;
    __shared__ uint64_t fin[16];
    __shared__ float2 wms[16];
    __shared__ float gmax[16];
    __shared__ uint64_t wtop[16];
    __shared__ int wcnt[16];
    __shared__ int cnt;
    __shared__ float z_sh, th_sh;
    __shared__ uint64_t top_sh;
    const int row = blockIdx.x, t = threadIdx.x;
    const int lane = t & (kWave - 1), wave = t / kWave;
    const uint64_t lt = (1ull << lane) - 1ull;
    constexpr int NWV = 16;
    const int nseg = gm.nch * gm.nvw * gm.nt;
    const float2* ms = cms + (size_t)row * nseg;
    const float* lrow = logits + (size_t)row * gm.V;
    MaxSum x{-INFINITY, 0.f};
    float g = -INFINITY;
    float m_first = -INFINITY;  // maximum of this thread's first segment
    for (int sg = wave + NWV * lane; sg < nseg; sg += NWV * kWave) {
        const float2 p = ms[sg];
        if (sg < NWV * kWave) m_first = p.x;
        x = ms_combine(x, MaxSum{p.x, p.y});
        g = fmaxf(g, p.x);
    }
    x = wave_ms_reduce(x);
    g = wave_max_f32(g);
    if (lane == 0) {
        wms[wave] = make_float2(x.m, x.s);
        gmax[wave] = g;
    }
    if (t == 0) {
        cnt = 0;
        nlive = 0;
        nlive2 = 0;
        th2_code = 0xFFFFFFFFu;
    }
    __syncthreads();
    if (wave == 0) {  // the 16 wave partials, combined in a fixed order
        MaxSum zz{-INFINITY, 0.f};
        float th = INFINITY;
        if (lane < NWV) {
            zz = MaxSum{wms[lane].x, wms[lane].y};
            th = gmax[lane];
        }
        zz = wave_ms_reduce(zz);
        th = -wave_max_f32(-th);
        if (lane == 0) {
            z_sh = (zz.m == -INFINITY) ? -INFINITY : zz.m + logf(zz.s);
            th_sh = th;
        }
    }
    __syncthreads();
    float th = th_sh;
    // The live segments (maximum >= th), listed in LDS; thread (w, l) looks
    // at segments w + 16 (64 q + l), as above.
    for (int q = 0; q * NWV * kWave < nseg; ++q) {
        const int sg = wave + NWV * (kWave * q + lane);
        const float msg = sg < nseg ? (q == 0 ? m_first : ms[sg].x) : -INFINITY;
        const bool live = sg < nseg && msg >= th;
        const uint64_t bal = __ballot(live);
        if (bal == 0ull) continue;
        int slot = 0;
        if (lane == 0) slot = atomicAdd(&nlive, __popcll(bal));
        slot = __shfl(slot, 0, kWave) + __popcll(bal & lt);
        if (live && slot < kSegLive) {
            int b0, e0;
            gm.range(sg, b0, e0);
            lbeg[slot] = b0;
            lend[slot] = e0;
            lmax[slot] = msg;
        }
    }
    __syncthreads();
    int nl = nlive;
    const int* lb = lbeg;
    const int* le = lend;
    if (nl >= K && nl <= kSegRefine) {
        // Tighter: th2 = the K-th largest maximum of the listed segments (the
        // smallest one with fewer than K larger).  The maxima of K distinct
        // segments are >= th2, so it bounds the row's K-th largest logit
        // too, and only the segments whose maximum is >= th2 (K of them,
        // ties aside) stay.  (With fewer than K listed segments there is no
        // such bound.)
        for (int i = t; i < nl; i += blockDim.x) {
            const float mi = lmax[i];
            int larger = 0;
#pragma unroll 8
            for (int q = 0; q < nl; ++q) larger += lmax[q] > mi ? 1 : 0;
            if (larger < K) atomicMin(&th2_code, (uint32_t)(make_key(mi, 0u) >> 32));
        }
        __syncthreads();
        const uint32_t c2 = th2_code;
        for (int i0 = 0; i0 < nl; i0 += blockDim.x) {  // wave-aggregated slots
            const int i = i0 + t;
            const bool keep = i < nl && (uint32_t)(make_key(lmax[i], 0u) >> 32) >= c2;
            const uint64_t bal = __ballot(keep);
            if (bal == 0ull) continue;
            int slot = 0;
            if (lane == 0) slot = atomicAdd(&nlive2, __popcll(bal));
            slot = __shfl(slot, 0, kWave) + __popcll(bal & lt);
            if (keep) {
                lbeg2[slot] = lbeg[i];
                lend2[slot] = lend[i];
            }
        }
        __syncthreads();
        nl = nlive2;
        lb = lbeg2;
        le = lend2;
        th = key_value((uint64_t)c2 << 32);
    }
    // keys of logits >= th: the high word of a key orders the values
    uint64_t theta = (uint64_t)(uint32_t)(make_key(th, 0u) >> 32) << 32;
    // Calls f(key) for every logit of every live segment (all lanes call it;
    // key 0 where a lane has no logit).
    auto for_live = [&](auto&& f) {
        if (nl <= kSegLive) {
            const int total = nl << gm.span_log2;
            const int smask = (1 << gm.span_log2) - 1;
            for (int base = 0; base < total; base += 1024 * kSegUnroll) {
                // All loads first (in-range addresses, no branches), so that
                // they are in flight together; then the keys.  Only as many
                // groups of 4 loads as the live logits need.
                const int groups = min(kSegUnroll / 4, (total - base + 4095) / 4096);
                for (int gq = 0; gq < groups; ++gq) {
                    float val[4];
                    int vid[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int iu = base + 1024 * (4 * gq + u) + t;
                        const int i = min(iu, total - 1);
                        const int ls = i >> gm.span_log2;
                        const int v = lb[ls] + (i & smask);
                        const bool ok = iu < total && v < le[ls];
                        vid[u] = ok ? v : -1;
                        val[u] = lrow[ok ? v : 0];
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) f(vid[u] >= 0 ? make_key(val[u], (uint32_t)vid[u]) : 0ull);
                }
            }
            return;
        }
        // Too many to list: lane l of wave w looks at segments w + 16 (64 q
        // + l), and the wave reads the live ones in turn.
        for (int q = 0; q * NWV * kWave < nseg; ++q) {
            const int sg = wave + NWV * (kWave * q + lane);
            const bool live = sg < nseg && ms[sg].x >= th;
            uint64_t todo = __ballot(live);
            while (todo) {
                const int l = __ffsll((unsigned long long)todo) - 1;
                todo &= todo - 1ull;
                int beg, end;
                gm.range(wave + NWV * (kWave * q + l), beg, end);
                for (int v0 = beg; v0 < end; v0 += kWave) {
                    const int v = v0 + lane;
                    f(v < end ? make_key(lrow[v], (uint32_t)v) : 0ull);
                }
            }
        }
    };
    // Pass 0 gathers the keys >= theta (and finds the row's largest key);
    // if too many pass, bisection raises theta and pass 1 gathers again.
    int n = 0;
    for (int attempt = 0; attempt < 2; ++attempt) {
        uint64_t top = 0ull;
        for_live([&](uint64_t key) {
            top = umax64(top, key);
            const bool p = key >= theta && key != 0ull;
            const uint64_t bal = __ballot(p);
            if (bal == 0ull) return;
            int slot = 0;
            if (lane == 0) slot = atomicAdd(&cnt, __popcll(bal));
            slot = __shfl(slot, 0, kWave) + __popcll(bal & lt);
            if (p && slot < kSegGather) cand[slot] = key;
        });
        top = wave_max_u64(top);
        if (lane == 0) wtop[wave] = top;
        __syncthreads();
        n = cnt;
        if (n <= kSegGather) break;
        if (t == 0) {
            uint64_t tp = 0ull;
            for (int w = 0; w < NWV; ++w) tp = umax64(tp, wtop[w]);
            top_sh = tp;
        }
        __syncthreads();
        // More than kSegGather >= K keys are >= theta, so the K-th largest
        // lies in [theta, top].
        uint64_t lo = theta, hi = top_sh;
        while (lo < hi) {
            const uint64_t mid = lo + (hi - lo) / 2 + 1;
            int cc = 0;
            for_live([&](uint64_t key) { cc += __popcll(__ballot(key >= mid)); });
            if (lane == 0) wcnt[wave] = cc;
            __syncthreads();
            int all = 0;
            for (int w = 0; w < NWV; ++w) all += wcnt[w];
            __syncthreads();
            if (all >= K) lo = mid;
            else hi = mid - 1;
        }
        theta = lo;
        __syncthreads();  // every thread has read cnt
        if (t == 0) cnt = 0;
        __syncthreads();
    }
    if (n > kSegGather) n = 0;  // unreachable: exactly K keys pass the exact threshold
    __syncthreads();
    for (int i = t; i < n; i += blockDim.x) {
        const uint64_t key = cand[i];
        int rank = 0;
#pragma unroll 8
        for (int q = 0; q < n; ++q) rank += cand[q] > key ? 1 : 0;
        if (rank < K) fin[rank] = key;
    }
    for (int i = n + t; i < K; i += blockDim.x) fin[i] = 0ull;
    __syncthreads();
    const float z = z_sh;
    if (t < K) {
        const uint64_t key = fin[t];
        cand_ids[(size_t)row * K + t] = key_id(key);
        cand_logp[(size_t)row * K + t] = key_value(key) - z;
    }
    if (t == 0) lse_out[row] = z;
}

}  // namespace

template <int NWB, int KC, int RW, int RY, int NVB, int TVB, bool RS, bool MS>
hipError_t launch_head_gemm_t(const Dims& d, const void* y, const void* W, int nch, float* logits, float2* ms,
                              int nt, hipStream_t s) {
    using G = GemmShape<NWB, NVB, TVB>;
    constexpr size_t lds = ((size_t)RW * G::TV + (size_t)RY * G::RP) * KC * 2;
    static_assert(lds <= 160 * 1024, "the stage rings must fit in LDS");
    auto fn = head_gemm_kernel<NWB, KC, RW, RY, NVB, TVB, RS, MS>;
    static LdsAttr attr;
    hipError_t e = ensure_lds(attr, (const void*)fn, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid(nch, (d.rows() + G::RP - 1) / G::RP);
    fn<<<grid, (NWB + kGemmProducers) * kWave, lds, s>>>((const uint16_t*)y, d.rows(), d.D, (const uint16_t*)W, d.V,
                                                         nch, logits, ms, nt);
    return hipGetLastError();
}

// More than 8 rows: one pass of the GEMM head per RP rows instead of one
// weight stream per 8 rows.
bool use_gemm_head(const Dims& d) { return d.bf16 && d.rows() > kRowsPass; }

template <int NWB, int KC, int RW, int RY, int NVB, int TVB>
hipError_t launch_head_gemm_rs(const Dims& d, const void* y, const void* W, int nch, float* logits, float2* ms,
                               int nt, hipStream_t s) {
    // row skipping only where the last row pass is partial
    const bool rs = d.rows() % GemmShape<NWB, NVB, TVB>::RP != 0;
    if (ms) {
        return rs ? launch_head_gemm_t<NWB, KC, RW, RY, NVB, TVB, true, true>(d, y, W, nch, logits, ms, nt, s)
                  : launch_head_gemm_t<NWB, KC, RW, RY, NVB, TVB, false, true>(d, y, W, nch, logits, ms, nt, s);
    }
    return rs ? launch_head_gemm_t<NWB, KC, RW, RY, NVB, TVB, true, false>(d, y, W, nch, logits, nullptr, 0, s)
              : launch_head_gemm_t<NWB, KC, RW, RY, NVB, TVB, false, false>(d, y, W, nch, logits, nullptr, 0, s);
}

// The configurations of the GEMM head, by hidden size and row count.  All
// use 8 x 1 blocks per consumer wave (fewer scalar registers than 4 x 2,
// and faster at every row count measured).
//  - 64-channel stages (D % 64 == 0):
//    * up to 128 rows: 512 x RP tiles (RP = 64 with 4 consumer waves, 128
//      with 8) and a 2-deep weight ring of 64 KB stages.  Against 256 x RP
//      tiles they read the hidden rows half as often per weight byte: at the
//      page D and V the head + top-K stage took 452 us at 64 rows (492 with
//      256 x 64 tiles) and 514 us at 128 rows (548 with 256 x 128 tiles, 576
//      with those and a 4-deep ring);
//    * more rows: 256 x 256 tiles and a 3-deep weight ring.
//  - 32-channel stages: 256 x 128 or 256 x 256 tiles, 6-deep weight rings.
enum GemmCfg { kG64x512x64, kG64x512x128, kG64x256x256, kG32x256x128, kG32x256x256 };

static GemmCfg gemm_cfg(const Dims& d) {
    if (d.D % 64 == 0) {
        if (d.rows() <= 64) return kG64x512x64;
        return d.rows() <= 128 ? kG64x512x128 : kG64x256x256;
    }
    return d.rows() <= 128 ? kG32x256x128 : kG32x256x256;
}

// (vocabulary blocks per wave, vocabulary blocks per tile) of a configuration
static void gemm_blocks(GemmCfg c, int* nvb, int* tvb) {
    switch (c) {
        case kG64x512x64:
        case kG64x512x128: *nvb = 8; *tvb = 16; return;
        default: *nvb = 8; *tvb = 8; return;
    }
}

GemmSegGeom gemm_seg_geom(const Dims& d) {
    GemmSegGeom g{};
    int tvb = 8;
    gemm_blocks(gemm_cfg(d), &g.nvb, &tvb);
    const int nch = head_chunks(d);
    const int64_t t32 = ((int64_t)d.V + 31) / 32;
    const int64_t per = (t32 + nch - 1) / nch;  // most 32-row blocks of one chunk
    g.nt = (int)((per + tvb - 1) / tvb);
    g.tv = 32 * tvb;
    g.nseg = nch * (tvb / g.nvb) * g.nt;
    return g;
}

static hipError_t head_gemm_dispatch(const Dims& d, const void* y, const void* W, float* logits, float2* ms,
                                     hipStream_t s) {
    const int nch = head_chunks(d);
    const int nt = ms ? gemm_seg_geom(d).nt : 0;
    switch (gemm_cfg(d)) {
        case kG64x512x64: return launch_head_gemm_rs<4, 64, 2, 2, 8, 16>(d, y, W, nch, logits, ms, nt, s);
        case kG64x512x128: return launch_head_gemm_rs<8, 64, 2, 2, 8, 16>(d, y, W, nch, logits, ms, nt, s);
        case kG64x256x256: return launch_head_gemm_rs<8, 64, 3, 2, 8, 8>(d, y, W, nch, logits, ms, nt, s);
        case kG32x256x128: return launch_head_gemm_rs<4, 32, 6, 4, 8, 8>(d, y, W, nch, logits, ms, nt, s);
        default: return launch_head_gemm_rs<8, 32, 6, 4, 8, 8>(d, y, W, nch, logits, ms, nt, s);
    }
}

hipError_t launch_head_gemm(const Dims& d, const void* y, const void* W, float* logits, float2* seg_ms,
                            hipStream_t s) {
    return head_gemm_dispatch(d, y, W, logits, seg_ms, s);
}

hipError_t launch_merge_segs(const Dims& d, const float* logits, const float2* seg_ms, int32_t* cand_ids,
                             float* cand_logp, float* lse, hipStream_t s) {
    const GemmSegGeom g = gemm_seg_geom(d);
    const int nch = head_chunks(d);
    const SegGeom gm{nch, g.tv / (32 * g.nvb), g.nvb, g.nt, (int)(((int64_t)d.V + 31) / 32), d.V,
                     g.nvb == 8 ? 8 : 7, g.tv};
    merge_seg_kernel<<<d.rows(), 1024, 0, s>>>(logits, seg_ms, gm, d.K, cand_ids, cand_logp, lse);
    return hipGetLastError();
}

hipError_t launch_head_f32(const Dims& d, const void* y, const void* W, float* logits, hipStream_t s) {
    head_f32_kernel<<<(d.V + 255) / 256, 256, 0, s>>>((const float*)y, (const float*)W, logits, d.rows(), d.D, d.V);
    return hipGetLastError();
}

}  // namespace dfs
