// dfs_draft_block_static: dfs_draft_block on a workspace that is a static
// device buffer of the library instead of a caller's allocation, for callers
// that cannot allocate.  The buffer (`scratch`) is a file-scope __device__
// array; each GPU the library runs on holds its own copy at its own address.
// In host code the array's name is only a host-side stand-in, so the device
// address is resolved with hipGetSymbolAddress, once per device with that
// device current, and only that address is ever handed to kernels.
#include <mutex>

#include "api_internal.h"

static __device__ __align__(256) uint8_t scratch[DFS_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of the current device's buffer.
int scratch_of_current_device(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFS_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = (char*)g_scratch_ptr[dev];
    return DFS_OK;
}

}  // namespace

extern "C" int dfs_draft_block_static(const dfs_config* cfg, const dfs_select_opts* opts, const void* h,
                                      const int32_t* anchor, const void* wg_cm, const void* W, const void* P,
                                      const void* Q, int32_t* path, float* path_score, int32_t* cand_ids,
                                      float* cand_logp, void* stream) {
    dfs::SelectOpts o;
    int st = dfs::check_draft_block(cfg, opts, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp,
                                    &o);
    if (st) return st;
    if (dfs_workspace_size(cfg) > DFS_STATIC_WORKSPACE_BYTES) return DFS_ERR_WORKSPACE;
    char* ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    return dfs::launch_draft_block(cfg, o, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids, cand_logp, ws,
                                   stream);
}
