// C ABI of libdflash2: argument validation on the host, then kernel launches
// on the caller's stream.  No allocation and no synchronisation.
#include <stdint.h>

#include <cmath>

#include "../../include/dflash2.h"
#include "api_internal.h"
#include "kernels.h"

namespace {

using dfs::Dims;

constexpr int kMaxRows = 65536;
constexpr int kMaxHidden = 65536;
constexpr int kMaxHiddenBf16Head = 8192;  // hidden rows stay resident in LDS
constexpr int kMaxTapsF32 = 4096;         // fp32 conv keeps z and w in LDS (32 KB)
constexpr int kMaxVocab = 1 << 21;        // logits ranked in at most 256 slices of 8192

bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

size_t align_up_bytes(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_cfg(const dfs_config* c) {
    if (!c) return DFS_ERR_NULL;
    if (c->dtype != DFS_F32 && c->dtype != DFS_BF16) return DFS_ERR_UNSUPPORTED;
    if (c->batch < 1 || c->block_size < 2 || c->block_size > 64) return DFS_ERR_SHAPE;
    if ((int64_t)c->batch * c->block_size > kMaxRows) return DFS_ERR_SHAPE;
    if (c->hidden < 32 || c->hidden % 32 != 0 || c->hidden > kMaxHidden) return DFS_ERR_SHAPE;
    if (c->conv_group_size < 1 || c->hidden % c->conv_group_size != 0) return DFS_ERR_SHAPE;
    if (c->conv_kernel_size < 1) return DFS_ERR_SHAPE;
    if (c->conv_kernel_size != 1 && c->conv_kernel_size != 2 && c->conv_kernel_size != 4) return DFS_ERR_UNSUPPORTED;
    if (c->top_k < 1) return DFS_ERR_SHAPE;
    if (c->top_k > 64) return DFS_ERR_UNSUPPORTED;
    if (c->vocab < c->top_k) return DFS_ERR_SHAPE;
    if (c->vocab > kMaxVocab) return DFS_ERR_UNSUPPORTED;
    if (c->rank < 8 || c->rank % 8 != 0 || c->rank > 4096) return DFS_ERR_SHAPE;
    if (c->dtype == DFS_BF16 && c->hidden > kMaxHiddenBf16Head) return DFS_ERR_UNSUPPORTED;
    if (c->dtype == DFS_F32 && (int64_t)(c->hidden / c->conv_group_size) * c->conv_kernel_size > kMaxTapsF32)
        return DFS_ERR_UNSUPPORTED;
    return DFS_OK;
}

Dims dims_of(const dfs_config* c) {
    return Dims{c->batch, c->block_size, c->hidden, c->vocab, c->top_k, c->rank, c->conv_group_size,
                c->conv_kernel_size, c->dtype == DFS_BF16};
}

int check_ws(const dfs_config* c, const void* ws, size_t ws_bytes) {
    const size_t need = dfs::ws_layout(dims_of(c)).total;
    if (ws_bytes < need) return DFS_ERR_WORKSPACE;
    if (need > 0 && !ws) return DFS_ERR_NULL;
    if (misaligned(ws, 256)) return DFS_ERR_MISALIGNED;
    return DFS_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DFS_OK : DFS_ERR_HIP; }

// Selector options: NULL means the best-path walk without a gate.
int check_opts(const dfs_select_opts* o, dfs::SelectOpts* out) {
    *out = dfs::SelectOpts{nullptr, DFS_WALK_VITERBI, 1.f, nullptr};
    if (!o) return DFS_OK;
    if (o->walk != DFS_WALK_VITERBI && o->walk != DFS_WALK_GREEDY && o->walk != DFS_WALK_SAMPLE)
        return DFS_ERR_UNSUPPORTED;
    if (o->walk == DFS_WALK_SAMPLE) {
        if (!o->uniforms) return DFS_ERR_NULL;
        if (!(o->temperature > 0.f) || !std::isfinite(o->temperature)) return DFS_ERR_SHAPE;
    }
    if (misaligned(o->gate, 16) || misaligned(o->uniforms, 16)) return DFS_ERR_MISALIGNED;
    *out = dfs::SelectOpts{o->gate, o->walk, o->temperature, o->walk == DFS_WALK_SAMPLE ? o->uniforms : nullptr};
    return DFS_OK;
}

}  // namespace

extern "C" {

const char* dfs_status_string(int status) {
    switch (status) {
        case DFS_OK: return "ok";
        case DFS_ERR_NULL: return "a required pointer is NULL";
        case DFS_ERR_SHAPE: return "a size is out of range or inconsistent";
        case DFS_ERR_UNSUPPORTED: return "valid value the library does not implement";
        case DFS_ERR_MISALIGNED: return "tensor not 16-byte aligned (workspace: 256-byte)";
        case DFS_ERR_WORKSPACE: return "workspace smaller than dfs_workspace_size()";
        case DFS_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int dfs_validate_config(const dfs_config* cfg) { return check_cfg(cfg); }

size_t dfs_workspace_size(const dfs_config* cfg) {
    if (check_cfg(cfg) != DFS_OK) return 0;
    return dfs::ws_layout(dims_of(cfg)).total;
}

int dfs_conv(const dfs_config* cfg, const void* h, const void* wg_cm, void* y, float* y_f32, void* ws,
             size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!h || !wg_cm || !y) return DFS_ERR_NULL;
    if (misaligned(h, 16) || misaligned(wg_cm, 16) || misaligned(y, 16) || misaligned(y_f32, 16))
        return DFS_ERR_MISALIGNED;
    if ((st = check_ws(cfg, ws, ws_bytes))) return st;
    return hip_status(dfs::launch_conv(dims_of(cfg), h, wg_cm, y, y_f32, (char*)ws, (hipStream_t)stream));
}

constexpr int kMaxLayers = 64;

size_t dfs_conv_layers_workspace_size(const dfs_config* cfg, int32_t layers) {
    if (check_cfg(cfg) != DFS_OK || layers < 1 || layers > kMaxLayers) return 0;
    const Dims d = dims_of(cfg);
    return align_up_bytes(dfs::ws_layout(d).zpart + (size_t)layers * dfs::conv_ws_bytes(d), 256);
}

int dfs_conv_layers(const dfs_config* cfg, int32_t layers, const void* h, const void* wg_cm, void* y, void* ws,
                    size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (layers < 1 || layers > kMaxLayers) return DFS_ERR_SHAPE;
    if (!h || !wg_cm || !y || !ws) return DFS_ERR_NULL;
    if (misaligned(h, 16) || misaligned(wg_cm, 16) || misaligned(y, 16) || misaligned(ws, 256))
        return DFS_ERR_MISALIGNED;
    if (ws_bytes < dfs_conv_layers_workspace_size(cfg, layers)) return DFS_ERR_WORKSPACE;
    return hip_status(
        dfs::launch_conv(dims_of(cfg), h, wg_cm, y, nullptr, (char*)ws, (hipStream_t)stream, (int)layers));
}

int dfs_head_topk(const dfs_config* cfg, const void* y, const void* W, int32_t* cand_ids, float* cand_logp,
                  float* lse, float* logits_f32, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!y || !W || !cand_ids || !cand_logp || !lse) return DFS_ERR_NULL;
    if (misaligned(y, 16) || misaligned(W, 16) || misaligned(cand_ids, 16) || misaligned(cand_logp, 16) ||
        misaligned(lse, 16) || misaligned(logits_f32, 16))
        return DFS_ERR_MISALIGNED;
    if ((st = check_ws(cfg, ws, ws_bytes))) return st;
    return hip_status(dfs::launch_head_topk(dims_of(cfg), y, W, cand_ids, cand_logp, lse, logits_f32, (char*)ws,
                                            (hipStream_t)stream));
}

int dfs_topk_logits(const dfs_config* cfg, const float* logits, int32_t* cand_ids, float* cand_logp, float* lse,
                    void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!logits || !cand_ids || !cand_logp || !lse) return DFS_ERR_NULL;
    if (misaligned(logits, 16) || misaligned(cand_ids, 16) || misaligned(cand_logp, 16) || misaligned(lse, 16))
        return DFS_ERR_MISALIGNED;
    if ((st = check_ws(cfg, ws, ws_bytes))) return st;
    return hip_status(
        dfs::launch_topk_logits(dims_of(cfg), logits, cand_ids, cand_logp, lse, (char*)ws, (hipStream_t)stream));
}

int dfs_select(const dfs_config* cfg, const dfs_select_opts* opts, const int32_t* anchor, const int32_t* cand_ids,
               const float* cand_logp, const void* P, const void* Q, int32_t* path, float* path_score,
               int32_t* path_idx, void* ws, size_t ws_bytes, void* stream) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!anchor || !cand_ids || !cand_logp || !P || !Q || !path || !path_score) return DFS_ERR_NULL;
    if (misaligned(anchor, 16) || misaligned(cand_ids, 16) || misaligned(cand_logp, 16) || misaligned(P, 16) ||
        misaligned(Q, 16) || misaligned(path, 16) || misaligned(path_score, 16) || misaligned(path_idx, 16))
        return DFS_ERR_MISALIGNED;
    dfs::SelectOpts o;
    if ((st = check_opts(opts, &o))) return st;
    if ((st = check_ws(cfg, ws, ws_bytes))) return st;
    return hip_status(dfs::launch_select(dims_of(cfg), o, anchor, cand_ids, cand_logp, P, Q, path, path_score,
                                         path_idx, (char*)ws, (hipStream_t)stream));
}

int dfs_draft_block(const dfs_config* cfg, const dfs_select_opts* opts, const void* h, const int32_t* anchor,
                    const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path, float* path_score,
                    int32_t* cand_ids, float* cand_logp, void* ws, size_t ws_bytes, void* stream) {
    dfs::SelectOpts o;
    int st = dfs::check_draft_block(cfg, opts, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp, &o);
    if (st) return st;
    if ((st = check_ws(cfg, ws, ws_bytes))) return st;
    return dfs::launch_draft_block(cfg, o, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp,
                                   (char*)ws, stream);
}

}  // extern "C"

namespace dfs {

int check_draft_block(const dfs_config* cfg, const dfs_select_opts* opts, const void* h, const int32_t* anchor,
                      const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                      float* path_score, int32_t* cand_ids, float* cand_logp, SelectOpts* o) {
    int st = check_cfg(cfg);
    if (st) return st;
    if (!h || !anchor || !wg_cm || !W || !P || !Q || !path || !path_score) return DFS_ERR_NULL;
    if (misaligned(h, 16) || misaligned(anchor, 16) || misaligned(wg_cm, 16) || misaligned(W, 16) ||
        misaligned(P, 16) || misaligned(Q, 16) || misaligned(path, 16) || misaligned(path_score, 16) ||
        misaligned(cand_ids, 16) || misaligned(cand_logp, 16))
        return DFS_ERR_MISALIGNED;
    return check_opts(opts, o);
}

int launch_draft_block(const dfs_config* cfg, const SelectOpts& o, const void* h, const int32_t* anchor,
                       const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                       float* path_score, int32_t* cand_ids, float* cand_logp, char* w, void* stream) {
    const Dims d = dims_of(cfg);
    hipStream_t s = (hipStream_t)stream;
    // Small, launch-bound shapes: the whole block in one launch.
    if (use_small_block(d))
        return hip_status(
            launch_block_small(d, o, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp, s));
    const WsLayout L = ws_layout(d);
    int st;
    // One tap: the conv is the identity, so the head reads h directly.
    const void* y = d.ks == 1 ? h : (const void*)(w + L.y);
    int32_t* cids = cand_ids ? cand_ids : (int32_t*)(w + L.cids);
    float* clogp = cand_logp ? cand_logp : (float*)(w + L.clogp);
    float* lse = (float*)(w + L.lse);
    if (d.ks != 1 && (st = hip_status(launch_conv(d, h, wg_cm, w + L.y, nullptr, w, s)))) return st;
    if ((st = hip_status(launch_head_topk(d, y, W, cids, clogp, lse, nullptr, w, s)))) return st;
    return hip_status(launch_select(d, o, anchor, cids, clogp, P, Q, path, path_score, nullptr, w, s));
}

}  // namespace dfs
