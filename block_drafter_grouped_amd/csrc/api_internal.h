// Host-side pieces of the C ABI shared by its translation units: the checks
// and launches of dfs_draft_block, split so that a variant with another
// workspace can run the same checks before any HIP call.
#pragma once

#include "../../include/dflash2.h"
#include "kernels.h"

namespace dfs {

// dfs_draft_block's argument checks, the workspace aside: DFS_OK (with the
// selector options in *o) or the first violated rule.  No HIP call.
int check_draft_block(const dfs_config* cfg, const dfs_select_opts* opts, const void* h, const int32_t* anchor,
                      const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                      float* path_score, int32_t* cand_ids, float* cand_logp, SelectOpts* o);

// The launches of dfs_draft_block on checked arguments and a workspace of at
// least dfs_workspace_size(cfg) bytes at ws (256-B aligned).
int launch_draft_block(const dfs_config* cfg, const SelectOpts& o, const void* h, const int32_t* anchor,
                       const void* wg_cm, const void* W, const void* P, const void* Q, int32_t* path,
                       float* path_score, int32_t* cand_ids, float* cand_logp, char* ws, void* stream);

}  // namespace dfs
