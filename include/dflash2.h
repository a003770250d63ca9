/*
 * dflash2.h -- C ABI of libdflash2, the MI355X (gfx950) draft-block hot path
 * of DFlash2 speculative decoding.
 *
 * One call turns the draft model's final hidden states for a block of B
 * positions (slot 0 = the last verified token, the "anchor"; slots 1..B-1 =
 * draft slots) into one proposed token path:
 *
 *   1. grouped dynamic depthwise causal conv inside the block
 *      (vLLM release-note article on DFlash2, section "two additions");
 *   2. vocabulary head (the target's lm_head) with log-softmax, over all rows
 *      (same section: the selector's candidates are ranked by the target
 *      model's head; Inco AI post "DFlash 2: keep the draft parallel",
 *      section "lightweight path selector": a candidate's node score is the
 *      drafter's own logit, taken here as its log-probability);
 *   3. per-slot top-K candidates over the full vocabulary (same section of
 *      the release-note article: rather than one argmax per draft slot, the
 *      selector retains the K tokens the target head ranks highest at every
 *      slot);
 *   4. low-rank adjacent-transition scores <P[a], Q[b]> between the
 *      candidates of neighbouring slots (Inco AI post "DFlash 2: keep the
 *      draft parallel", section "lightweight path selector", with the
 *      context gate taken as 1);
 *   5. the best path through the candidates, walked from the anchor
 *      (release-note article, "two additions"), as max-sum Viterbi.
 *
 * Constants of the published checkpoint (RTX 4090 report, section 4,
 * dflash_config): block_size 8, conv_group_size 16, conv_kernel_size 2,
 * selector_rank 256, selector_top_k 16.  block_size = 1 + draft tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - `cfg` is a HOST pointer.  Every tensor pointer is a DEVICE pointer to
 *    row-major, contiguous memory, 16-byte aligned; the workspace is 256-byte
 *    aligned.  Rows of block b are b*B .. b*B+B-1 (rows = batch * B).
 *  - Floating tensors (h, wg_cm, y, W, P, Q) have the dtype cfg->dtype:
 *    DFS_BF16 (the hot path: bf16 inputs, fp32 accumulation) or DFS_F32 (a
 *    plain correctness path).  Candidate scores, lse and logits are fp32;
 *    ids are int32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    validates its arguments on the host and enqueues kernels on `stream`:
 *    it never allocates, frees or synchronises, and returns before the work
 *    is done.  The caller synchronises before reading outputs.
 *  - Ownership: the caller owns every buffer, including the workspace
 *    (>= dfs_workspace_size(cfg) bytes; contents undefined between calls;
 *    one call at a time per workspace).  The library keeps no state besides
 *    the kernels' LDS attributes (set once per process) and, for
 *    dfs_draft_block_static only, its static per-device workspace.
 *  - Errors: the return value is a dfs_status.  All argument checks happen on
 *    the host BEFORE any HIP call, so a rejected call touches no device
 *    state.  DFS_ERR_HIP reports a failed kernel launch; faults inside a
 *    kernel surface at the caller's synchronisation.
 *  - Results are bit-identical from run to run (no atomics in any sum).
 *  - Ties: candidates with equal logits are ordered by lower vocabulary id
 *    (-0.0 and +0.0 are equal); the walk takes the lowest predecessor index
 *    and the lowest final index among equal scores.  NaN inputs are not
 *    supported.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>

/* Only the declarations below are exported from the shared library. */
#if defined(__GNUC__) || defined(__clang__)
#define DFS_API __attribute__((visibility("default")))
#else
#define DFS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFS_OK = 0,
    DFS_ERR_NULL = 1,        /* a required pointer is NULL                    */
    DFS_ERR_SHAPE = 2,       /* a size is out of range or inconsistent         */
    DFS_ERR_UNSUPPORTED = 3, /* a valid value the library does not implement */
    DFS_ERR_MISALIGNED = 4,  /* a tensor is not 16-B (workspace: 256-B) aligned */
    DFS_ERR_WORKSPACE = 5,   /* ws_bytes < dfs_workspace_size(cfg)             */
    DFS_ERR_HIP = 6          /* a kernel launch failed                         */
} dfs_status;

typedef enum { DFS_F32 = 0, DFS_BF16 = 1 } dfs_dtype;

/* Field names follow the checkpoint's dflash_config where one exists. */
typedef struct {
    int32_t batch;            /* independent blocks, >= 1                         */
    int32_t block_size;       /* B = 1 + draft slots, 2..64                       */
    int32_t hidden;           /* D, a multiple of 32 and of conv_group_size       */
    int32_t vocab;            /* V, top_k <= V <= 2^21 (2 097 152)                 */
    int32_t top_k;            /* K = selector_top_k, 1..64                         */
    int32_t rank;             /* r = selector_rank, a multiple of 8, 8..4096       */
    int32_t conv_group_size;  /* channels sharing one generated kernel (16)        */
    int32_t conv_kernel_size; /* causal taps: 1, 2 or 4 (1 = identity conv)        */
    int32_t dtype;            /* dfs_dtype                                         */
} dfs_config;

/* Bytes of workspace any entry point needs for `cfg` (0 if cfg is invalid). */
DFS_API size_t dfs_workspace_size(const dfs_config* cfg);

/* Static description of a status code (never NULL). */
DFS_API const char* dfs_status_string(int status);

/* Checks `cfg` alone (no pointers).  DFS_OK or the first violated rule. */
DFS_API int dfs_validate_config(const dfs_config* cfg);

/*
 * Step 1: grouped dynamic depthwise causal conv (release-note article,
 * "two additions": a per-position kernel generated from the hidden state,
 * shared by each group of conv_group_size channels, over the current and the
 * earlier positions of the same block).
 *
 *   z[row, g*ks + j] = sum_c h[row, c] * wg_cm[g*ks + j, c]
 *   w[row, g, :]     = softmax over the ks taps of z[row, g*ks : g*ks+ks]
 *   y[b, t, c]       = sum_{j < ks, t-j >= 0} w[b*B+t, c / conv_group_size, j] * h[b, t-j, c]
 *
 *  h      [rows, D]     dtype, hidden states (row-major, block-major rows)
 *  wg_cm  [G*ks, D]     dtype, generator weights, channel-major: row g*ks+j
 *                       holds the weights of tap j of group g over all D
 *                       channels (the transpose of the [D, G*ks] matrix)
 *  y      [rows, D]     dtype, output; bf16 is the round-to-nearest-even of
 *                       the fp32 result
 *  y_f32  [rows, D]     fp32, optional (NULL): the fp32 result before
 *                       rounding, for parity checks
 *  ws, ws_bytes         workspace (see conventions); the bf16 path keeps the
 *                       partial tap logits of its split D reduction there
 * Positions before the start of a block count as zero; the tap softmax is
 * not renormalised there.
 */
DFS_API int dfs_conv(const dfs_config* cfg, const void* h, const void* wg_cm,
             void* y, float* y_f32, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 1 for several drafter layers in one pair of launches (release-note
 * article, cost section: the conv ran as 20 small calls per step for a
 * 5-layer drafter, which reads as one conv per layer).  Layer l applies
 * dfs_conv's operation to its own hidden states with its own generator:
 *
 *  layers          1..64 (else DFS_ERR_SHAPE)
 *  h      [layers, rows, D]   dtype
 *  wg_cm  [layers, G*ks, D]   dtype, channel-major as for dfs_conv
 *  y      [layers, rows, D]   dtype out
 *  ws, ws_bytes  at least dfs_conv_layers_workspace_size(cfg, layers) bytes,
 *                256-B aligned
 * Layer results equal dfs_conv on each layer alone.
 */
DFS_API int dfs_conv_layers(const dfs_config* cfg, int32_t layers, const void* h,
                    const void* wg_cm, void* y, void* ws, size_t ws_bytes,
                    void* stream);

/* Workspace bytes dfs_conv_layers needs (0 if cfg or layers is invalid). */
DFS_API size_t dfs_conv_layers_workspace_size(const dfs_config* cfg, int32_t layers);

/*
 * Steps 2-3: vocabulary head, log-softmax and per-slot top-K for every row
 * (vLLM release-note article on DFlash2, section "two additions": the
 * selector works on the K tokens the target head scores highest at each
 * slot, in place of a per-slot argmax; its cost section sizes this stage:
 * hidden 5120, vocabulary 248 320, K 16, the vocabulary top-k done by a
 * dedicated kernel).
 *
 *   logit[row, v] = sum_c y[row, c] * W[v, c]           (fp32 accumulation)
 *   lse[row]      = log sum_v exp(logit[row, v])
 *   cand_ids[row, :K]  the K largest logits, by (logit desc, id asc)
 *   cand_logp[row, k]  = logit[row, cand_ids[row, k]] - lse[row]
 *
 *  y          [rows, D]  dtype (the conv output)
 *  W          [V, D]     dtype, the shared target lm_head
 *  cand_ids   [rows, K]  int32 out
 *  cand_logp  [rows, K]  fp32 out
 *  lse        [rows]     fp32 out
 *  logits_f32 [rows, V]  fp32, optional (NULL): also writes every logit (the
 *                        exact values the top-K was taken from), for parity
 *  ws, ws_bytes          workspace (see conventions)
 * Up to 8 rows (bf16, K <= 16) the logits are never materialised otherwise:
 * each workgroup keeps its own top-K and (max, sum of exp) partials, merged
 * by a second kernel.  With more rows the logits go to the workspace (or to
 * logits_f32) together with the (max, sum of exp) of every 256-logit
 * segment, and the merge reads only the segments that can hold a row's top
 * K (K <= 16) or ranks every slice of the logits (K > 16).  Both modes give
 * the same bits.
 */
DFS_API int dfs_head_topk(const dfs_config* cfg, const void* y, const void* W,
                  int32_t* cand_ids, float* cand_logp, float* lse,
                  float* logits_f32, void* ws, size_t ws_bytes, void* stream);

/*
 * Step 3 alone, on caller-supplied fp32 logits [rows, V] (any finite values
 * or -inf; a row of all -inf yields lse = -inf and NaN scores): the per-slot
 * vocabulary top-k and log-softmax of the release-note article's cost
 * section, which times that top-k as a kernel of its own on given logits.
 * Same outputs and ordering as dfs_head_topk.  cfg->dtype is ignored.
 */
DFS_API int dfs_topk_logits(const dfs_config* cfg, const float* logits,
                    int32_t* cand_ids, float* cand_logp, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/* Walk rules of the selector (Inco AI post, "lightweight path selector"). */
typedef enum {
    DFS_WALK_VITERBI = 0, /* the best path: max over all paths (default)         */
    DFS_WALK_GREEDY = 1,  /* at each slot, the best successor of the last choice */
    DFS_WALK_SAMPLE = 2   /* at each slot, a successor sampled from the scores   */
} dfs_walk;

/*
 * Selector options.  A NULL pointer means: no gate, DFS_WALK_VITERBI.
 *  gate        [rows, r] fp32 device, nullable: the context gate H(h_t) of
 *              each row (row b*B + t gates the transitions into slot t; the
 *              Inco AI post's pair score <A(a) * H(h_t), B(b)>).  NULL: all
 *              ones.  The pages give no form for H; the caller computes it.
 *  walk        dfs_walk.
 *  temperature DFS_WALK_SAMPLE: > 0 and finite (else DFS_ERR_SHAPE).
 *  uniforms    DFS_WALK_SAMPLE: [batch, B] fp32 device (else DFS_ERR_NULL):
 *              uniforms[b, t] in [0, 1) draws slot t of block b; column 0 is
 *              not read.  The library draws no random numbers itself.
 * bf16 tables with K <= 16 and r % 32 == 0 run one fused kernel (MFMA dot
 * products, fp32 accumulation; a gate enters as P (*) H formed in fp32 and
 * split into two bf16 parts); fp32 tables, K > 16 or other ranks run the
 * general selector kernels (fp32 dot products).
 */
typedef struct {
    const float* gate;
    int32_t walk;
    float temperature;
    const float* uniforms;
} dfs_select_opts;

/*
 * Steps 4-5: transition scores and the best path (Inco AI post, section
 * "lightweight path selector": every adjacent candidate pair is scored at
 * once; the only sequential work is the walk over the precomputed scores,
 * starting from the last verified token).
 *
 * For block b with candidates c_t = cand_ids[b*B + t, :] (t >= 1) and
 * c_0 = {anchor[b]}:
 *   T_t[j, k] = sum_i P[c_{t-1, j}, i] * H_t[i] * Q[c_{t, k}, i]   (fp32 accumulation;
 *               H_t = gate row b*B + t, or 1)
 *   delta_1[k] = cand_logp[b*B+1, k] + T_1[0, k]
 *   delta_t[k] = max_j (delta_{t-1}[j] + T_t[j, k]) + cand_logp[b*B+t, k]
 * DFS_WALK_VITERBI: the path takes argmax_k delta_{B-1}[k] and backtracks;
 * ties go to the lowest index at every step; path_score = delta_{B-1}.
 * DFS_WALK_GREEDY / DFS_WALK_SAMPLE: from p_0 = the anchor, slot t scores
 * s_t[k] = cand_logp[b*B+t, k] + T_t[p_{t-1}, k]; greedy takes the largest
 * (lowest k on ties); sampling takes the smallest k whose prefix sum of
 * exp((s_t - max s_t) / temperature), in index order, exceeds
 * uniforms[b, t] times the total (the last k if none).  path_score is the
 * sum of the chosen s_t.
 *
 *  anchor     [batch]     int32, the verified token of each block
 *  cand_ids   [rows, K]   int32, cand_logp [rows, K] fp32 (rows of slot 0 are
 *                         not read)
 *  P, Q       [V, r]      dtype: per-token selector embeddings; P is indexed
 *                         by the predecessor, Q by the successor
 *  path       [batch, B]  int32 out: path[b, 0] = anchor[b], then one
 *                         candidate id per draft slot
 *  path_score [batch]     fp32 out: the path's score (see above)
 *  path_idx   [batch, B]  int32, optional: path_idx[b, 0] = -1, then the
 *                         chosen candidate index per draft slot
 * A block whose anchor, or any of whose draft-slot candidate ids, lies
 * outside [0, V) gets path = -1 in every slot, path_idx = -1 and
 * path_score = NaN; the other blocks are unaffected.
 */
DFS_API int dfs_select(const dfs_config* cfg, const dfs_select_opts* opts,
               const int32_t* anchor, const int32_t* cand_ids, const float* cand_logp,
               const void* P, const void* Q, int32_t* path, float* path_score,
               int32_t* path_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole block: dfs_conv -> dfs_head_topk -> dfs_select on one stream
 * (release-note article, section "two additions": the hidden states of one
 * block and the verified anchor in, one proposed path out; Inco AI post,
 * section "lightweight path selector": scoring is parallel over all slots,
 * and the walk is the only sequential part).
 * cand_ids / cand_logp are optional outputs (NULL: kept in the workspace).
 * Arguments as above.  Small shapes, where the work is too little to cover
 * the launches (block <= 16, K <= 16, hidden <= 512, vocab <= 1024 with
 * vocab x hidden <= 2^17 and block x vocab <= 2^14, rank <= 512), run every
 * step in one launch, one
 * workgroup per block; their results match the three calls within the
 * stated tolerances (the sums run in another order), with the same ids.
 */
DFS_API int dfs_draft_block(const dfs_config* cfg, const dfs_select_opts* opts,
                    const void* h, const int32_t* anchor,
                    const void* wg_cm, const void* W, const void* P, const void* Q,
                    int32_t* path, float* path_score, int32_t* cand_ids,
                    float* cand_logp, void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free variant of dfs_draft_block, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks, kernels and
 * results as dfs_draft_block, but no workspace argument: the workspace is a
 * static device buffer of the library, DFS_STATIC_WORKSPACE_BYTES per GPU,
 * held from the library's load until the process ends.  The call allocates
 * and frees nothing.
 *  - Configurations with dfs_workspace_size(cfg) > DFS_STATIC_WORKSPACE_BYTES
 *    are rejected with DFS_ERR_WORKSPACE, before any HIP call (every
 *    configuration up to 8 rows with K <= 16 fits, at any vocabulary and
 *    hidden size; larger ones when their written logits fit).
 *  - The buffer of the CURRENT device is used; `stream` must belong to it.
 *    The first call on a device resolves that buffer's address (a HIP symbol
 *    query, no allocation); make it outside stream capture.
 *  - Every call on one GPU shares that GPU's buffer, which keeps what the
 *    last call left there (no part of it has to start at zero).  Calls that
 *    overlap on one GPU (two streams, or two threads) race on it: serialise
 *    them.
 */
#define DFS_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
DFS_API int dfs_draft_block_static(const dfs_config* cfg, const dfs_select_opts* opts,
                                   const void* h, const int32_t* anchor,
                                   const void* wg_cm, const void* W, const void* P,
                                   const void* Q, int32_t* path, float* path_score,
                                   int32_t* cand_ids, float* cand_logp, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH2_H */
