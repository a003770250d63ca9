// Launchers of the gfx950 kernels (host side).  Each enqueues on `stream`
// and returns hipGetLastError() of its launches.  Arguments are validated by
// the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace dfs {

// The dynamic-LDS limit a kernel was raised to, per device.  A launcher keeps
// one static instance per kernel; ensure_lds() calls hipFuncSetAttribute only
// when a launch needs more LDS than any earlier launch of that kernel on the
// current device, so steady-state calls make no attribute call.
constexpr int kLdsAttrDevices = 64;
struct LdsAttr {
    std::atomic<int> bytes[kLdsAttrDevices];
};
inline hipError_t ensure_lds(LdsAttr& a, const void* fn, int bytes) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kLdsAttrDevices)
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    int have = a.bytes[dev].load(std::memory_order_acquire);
    if (have >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    while (have < bytes && !a.bytes[dev].compare_exchange_weak(have, bytes, std::memory_order_acq_rel)) {
    }
    return hipSuccess;
}

struct Dims {
    int batch, B, D, V, K, r, gs, ks;
    bool bf16;
    int rows() const { return batch * B; }
    int groups() const { return D / gs; }
    int taps() const { return groups() * ks; }  // columns of the generator
};

constexpr int kRowsPass = 8;  // rows one pass of the streaming head serves

// Number of vocabulary chunks whose per-chunk top-K / (max, sum) partials the
// head writes.  A function of the shape only, so workspace sizes need no
// device query.
int head_chunks(const Dims& d);

// Workspace carve-up (byte offsets from the 256-B aligned base).
struct WsLayout {
    size_t y, keys, ms, logits, segms, T, cids, clogp, lse, zpart, total;
};
WsLayout ws_layout(const Dims& d);

// Bytes of split-reduction partials the bf16 conv keeps in the workspace,
// per layer.  They are the workspace's last section (ws_layout().zpart), so
// a conv over several layers needs zpart + layers * conv_ws_bytes bytes.
size_t conv_ws_bytes(const Dims& d);

// The conv of `layers` independent [rows, D] inputs, each with its own
// generator: h [layers, rows, D], wg_cm [layers, G*ks, D], y and y_f32
// [layers, rows, D].
hipError_t launch_conv(const Dims& d, const void* h, const void* wg_cm, void* y, float* y_f32, char* ws,
                       hipStream_t s, int layers = 1);

// Head + top-K.  Uses ws.keys / ws.ms; ws.logits when the logits are
// written (fp32, K > 16, more than 8 rows) and logits_f32 is NULL; and
// ws.segms for the GEMM head's segment partials (more than 8 rows, K <= 16).
hipError_t launch_head_topk(const Dims& d, const void* y, const void* W, int32_t* cand_ids,
                            float* cand_logp, float* lse, float* logits_f32, char* ws,
                            hipStream_t s);

// The head's per-chunk partials only (no merge); *nparts receives the number
// of chunks the merge reads.
hipError_t launch_head_partials(const Dims& d, const void* y, const void* W, float* logits_f32, char* ws,
                                int* nparts, hipStream_t s);

// Heads that write fp32 logits [rows][V]: the GEMM head (bf16, more than
// kRowsPass rows) and the fp32 head.
bool use_gemm_head(const Dims& d);
hipError_t launch_head_gemm(const Dims& d, const void* y, const void* W, float* logits, float2* seg_ms,
                            hipStream_t s);
hipError_t launch_head_f32(const Dims& d, const void* y, const void* W, float* logits, hipStream_t s);

// Segments of the GEMM head: a segment is the part of one tile that one
// consumer wave holds, for one row (at most 256 consecutive logits of a
// chunk's vocabulary range).  With seg_ms non-null the GEMM also writes the
// (max, sum of exp) of every segment, layout [row][nseg].
struct GemmSegGeom {
    int nt, nvb, nseg, tv;  // tiles per list, vocabulary blocks per wave, segments per row, tile width
};
GemmSegGeom gemm_seg_geom(const Dims& d);
// Written logits + segment partials -> sorted candidates, log-probabilities
// and lse (K <= 16).
hipError_t launch_merge_segs(const Dims& d, const float* logits, const float2* seg_ms, int32_t* cand_ids,
                             float* cand_logp, float* lse, hipStream_t s);

// Per-slice top-K keys and (max, sum of exp) of written logits, in the
// partial layout the merge reads ([row][k][slice], stride nsl).
int logits_slices(const Dims& d);
hipError_t launch_logits_partials(const Dims& d, const float* logits, int nsl, uint64_t* keys, float2* ms,
                                  hipStream_t s);

hipError_t launch_topk_logits(const Dims& d, const float* logits, int32_t* cand_ids, float* cand_logp,
                              float* lse, char* ws, hipStream_t s);

// Selector options: context gate [rows, r] (nullable: all ones); walk 0 best
// path, 1 greedy, 2 sample (temperature, uniforms [batch, B]).
struct SelectOpts {
    const float* gate;
    int walk;
    float temperature;
    const float* uniforms;
};

// The whole draft block in one launch (one workgroup per block, every step
// in LDS) for small, launch-bound shapes: block <= 16, K <= 16, hidden <= 512,
// vocabulary <= 1024 with vocabulary x hidden <= 2^17 and block x vocabulary
// <= 2^14, rank <= 512.
bool use_small_block(const Dims& d);
hipError_t launch_block_small(const Dims& d, const SelectOpts& o, const void* h, const int32_t* anchor,
                              const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                              float* path_score, int32_t* cand_ids, float* cand_logp, hipStream_t s);

hipError_t launch_select(const Dims& d, const SelectOpts& o, const int32_t* anchor, const int32_t* cand_ids,
                         const float* cand_logp, const void* P, const void* Q, int32_t* path, float* path_score,
                         int32_t* path_idx, char* ws, hipStream_t s);

}  // namespace dfs
