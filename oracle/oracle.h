/*
 * oracle.h -- plain, slow, fp64 CPU implementation of the DFlash2 draft-block
 * path: grouped dynamic depthwise causal conv, vocab head with log-softmax,
 * per-slot top-K, low-rank adjacent-transition scores and the best-path walk
 * from the verified anchor.
 *
 * TEST INFRASTRUCTURE ONLY.  It exists to check the HIP library; nothing in
 * the product path may call it.  It shares no code, header or constant with
 * the HIP side.
 *
 * Sources (web pages, cited by title and section):
 *  - vLLM release-note article on DFlash2 (page 1), section "two additions":
 *    each block gets a grouped, dynamically generated depthwise convolution
 *    through which a draft position sees the earlier positions of its block
 *    without running the backbone again; the candidate selector replaces the
 *    per-slot argmax: it retains the target head's K best tokens at every
 *    slot, scores transitions between neighbouring slots, and walks the
 *    best-scoring path onward from the anchor that verification accepted.
 *  - Inco AI post "DFlash 2: keep the draft parallel" (page 4), section
 *    "lightweight path selector": the score of candidate b after a is
 *    S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)> with 256-wide per-token
 *    embeddings A, B; all adjacent pairs are scored at once and the only
 *    sequential work is the final walk over the precomputed scores.
 *  - RTX 4090 DFlash2 report (page 3), section 4: the checkpoint's
 *    dflash_config {block_size 8, conv_group_size 16, conv_kernel_size 2,
 *    selector_rank 256, selector_top_k 16}, block_size = 1 + draft tokens.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  conv weights at position t come from h[t] alone (column g*ks+j = tap j of
 *  group g), plain softmax over the taps, zero padding before the block start
 *  with no renormalisation, no residual; the node score U is the log-softmax
 *  of the logit; the context gate H is absent (== 1); the walk is max-sum
 *  Viterbi; ties go to the lowest vocabulary id (top-K) and to the lowest
 *  candidate index (walk).
 *
 * All arithmetic is IEEE fp64.  bf16 and fp32 inputs are widened exactly.
 */
#ifndef DFS_ORACLE_H
#define DFS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch;   /* independent blocks                                  */
    int32_t block;   /* B: slot 0 = verified anchor, slots 1..B-1 = drafts  */
    int32_t hidden;  /* D                                                   */
    int32_t vocab;   /* V                                                   */
    int32_t top_k;   /* K candidates per slot                               */
    int32_t rank;    /* r, width of the selector embeddings                 */
    int32_t group;   /* channels per conv group                             */
    int32_t ksize;   /* causal taps                                         */
    int32_t bf16;    /* 1: tensors hold bf16 bit patterns; 0: fp32 values   */
} orc_shape;

/* Conv, C-def steps 1-3.  h [rows][D], wg [D][G*ks] (mathematical layout).
 * Outputs (each nullable except yhat): z [rows][G*ks] tap logits,
 * w [rows][G*ks] tap weights, yhat [rows][D] exact (fp64) conv output.
 * Returns 0, or -1 on a bad shape. */
int orc_conv(const orc_shape* s, const void* h, const void* wg,
             double* z, double* w, double* yhat);

/* Rounds n fp64 values to the tensor dtype: bf16 bits (round to nearest
 * even, from the exact value) or fp32 (round to nearest). */
void orc_round(const orc_shape* s, const double* x, void* out, int64_t n);

/* Head, C-def steps 4-6, for rows [r0, r0+nr).  y [rows][D], W [V][D].
 * logits [nr][V] (nullable), lse [nr], ids [nr][K], logp [nr][K]. */
int orc_head(const orc_shape* s, const void* y, const void* W, int r0, int nr,
             double* logits, double* lse, int32_t* ids, double* logp);

/* Top-K and log-softmax of given logits, C-def steps 5-6.
 * logits [nr][V]; ids [nr][K] sorted by (logit desc, id asc). */
int orc_topk(int nr, int V, int K, const double* logits,
             int32_t* ids, double* logp, double* lse);

/* Transition scores of one block, C-def step 7.  ids [B][K] are the block's
 * candidates (row 0 ignored).  gate [B][r] (nullable: all ones) holds the
 * context gate of each slot (row 0 ignored).  T [B-1][K][K]:
 * T[t-1][j][k] = sum_i P[prev_j][i] * gate[t][i] * Q[ids[t][k]][i]
 * with prev = {anchor} for t = 1 (only j = 0 is written; the rest are 0). */
int orc_transitions(const orc_shape* s, int32_t anchor, const int32_t* ids,
                    const void* P, const void* Q, const double* gate, double* T);

/* Best-path walk of one block, C-def step 8.  logp [B][K] (row 0 ignored),
 * T as above.  idx [B] receives idx[0] = -1 and the chosen candidate index of
 * each draft slot; *score the best path score; *margin (nullable) the gap to
 * the best path with a different index sequence (+inf if there is none). */
int orc_viterbi(int B, int K, const double* logp, const double* T,
                int32_t* idx, double* score, double* margin);

/* Other walk rules of one block (mode 1 greedy, 2 sample), C-def step 8b.
 * logp [B][K] and T as for orc_viterbi; uniforms [B] (mode 2; entry t is the
 * uniform of slot t, entry 0 ignored).  Returns -1 for a bad mode or, in
 * mode 2, a missing uniform vector or temperature <= 0. */
int orc_walk(int B, int K, const double* logp, const double* T, int mode,
             double temperature, const double* uniforms, int32_t* idx, double* score);

/* Whole path for all blocks: conv, rounding of y to the dtype, head, top-K,
 * transitions (gate [rows][r], nullable: all ones) and walk.  Outputs: path
 * [batch][B] (slot 0 = anchor; -1 for every slot of a block whose anchor is
 * outside [0, V)), score [batch] (NaN for such a block), and nullable
 * ids [rows][K], logp [rows][K], lse [rows], idx [batch][B], margin [batch]. */
int orc_draft_block(const orc_shape* s, const void* h, const int32_t* anchor,
                    const void* wg, const void* W, const void* P, const void* Q,
                    const double* gate, int32_t* path, double* score, int32_t* ids,
                    double* logp, double* lse, int32_t* idx, double* margin);

/* Number of OpenMP threads the oracle will use. */
int orc_threads(void);

#ifdef __cplusplus
}
#endif
#endif
