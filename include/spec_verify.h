/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-verification
 * library libspecverify.so.
 *
 * The operations, all over the vocabulary and all stated on the pages (each
 * declaration below cites its passages):
 *
 *  spec_verify_chain: speculative sampling of one drafted block per batch
 *    entry.  For draft position i the target distribution p_i and the draft
 *    distribution q_i are the temperature softmaxes of the given logits,
 *    taken identically for both ("Speculative decoding verifies draft tokens
 *    without changing the target sampling distribution", section "Logit
 *    processing must be consistent across verification").  Draft token x_i is
 *    accepted with probability min(1, p_i(x_i)/q_i(x_i)), left to right, and
 *    the first rejection ends the block (same page, section "Acceptance
 *    depends on both target and draft probabilities"; "JetSpec reading
 *    notes", Eq. 1 and Eq. 17).  After a rejection at position k the extra
 *    token is drawn from max(0, p_k - q_k) normalised (section "Rejection
 *    uses a residual distribution"); after a fully accepted block it is drawn
 *    from the target's bonus row p_gamma (section "A fully accepted block
 *    yields more than one committed token"; "JetSpec++", Appendix F.1).
 *
 *  spec_verify_chain_pointmass: the same with a draft that proposes each
 *    token with certainty (no draft logits read).
 *
 *  spec_verify_tree_greedy: greedy (T = 0) verification of a draft tree given
 *    as a parent array: a node is accepted iff its parent is accepted and its
 *    token equals the target argmax after the parent's path; the deepest
 *    accepted node is kept and the target argmax after it is emitted as the
 *    extra token ("JetSpec reading notes", section "Tree verification",
 *    Fig. 5 and the greedy note; Algorithm 1 for the parent array).
 *
 *  spec_verify_tree_stochastic: one Bernoulli test per tree node against its
 *    parent's target and draft rows, the deepest branch accepted throughout,
 *    and the correction drawn from the target after it.
 *
 *  spec_outcome_topk and spec_cache_lookup: the most probable verification
 *    outcomes of a block (a speculation cache) and the lookup of the outcome
 *    that verification produced.
 *
 *  spec_tree_build: draft-tree construction by best-first search over the
 *    draft's per-node logits.
 *
 * Every random draw is an explicit input: the caller passes one uniform per
 * test and one for the final draw, so results are a pure function of the
 * arguments.
 *
 * Conventions shared by every entry point:
 *  - Pointers to logits, tokens, uniforms, parents, outputs and workspace are
 *    DEVICE pointers owned by the caller; the library allocates no device
 *    memory and never synchronises the stream, and its only global state is
 *    the per-GPU address of spec_verify_chain_noalloc's static scratch.  All
 *    work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    results are valid once that stream reaches this point.
 *  - Arrays are dense, row-major, with the shapes given below.  Logits are
 *    float32 (SV_DTYPE_F32) or bfloat16 bit patterns (SV_DTYPE_BF16); each
 *    pointer must be aligned to its element size.
 *  - Host-detectable errors (a null required pointer, a size out of range, an
 *    unknown dtype, a bad temperature, a workspace that is too small or not
 *    16-byte aligned, a misaligned pointer) return a non-zero status BEFORE
 *    anything is enqueued, and nothing is written.
 *  - Data-dependent errors are reported per block (per request for trees)
 *    without any host synchronisation: accept_len[b] = -1 and every output
 *    token of that block = -1, while the other blocks are unaffected.  They
 *    are: a draft token outside [0, V); a NaN or +inf logit in any row of the
 *    block; a row without any finite logit; a row outside the numeric domain
 *    (below); for trees, a malformed parent array or a node token outside
 *    [0, V).
 *  - Numeric domain (a restriction of this library, not of the method): every
 *    row whose softmax is taken -- target and draft rows of chains and
 *    stochastic trees, decoder rows of spec_outcome_topk, draft rows of
 *    spec_tree_build -- must have |m| / T <= 2^28, m its largest finite
 *    logit.  The kernels scale logits by 1/T in single precision against an
 *    integer reference near m/T, which stays exact only within that range.
 *    A row beyond it makes its block (request) invalid as above.
 *  - -inf logits are legal and mean "masked": that token has probability 0.
 *  - The workspace is scratch owned by the caller: it needs no
 *    initialisation and its contents after a call are unspecified.  Two
 *    calls in flight at the same time need distinct workspaces.
 *  - A failure of the HIP runtime to launch returns SV_ERR_HIP.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of the logits. */
#define SV_DTYPE_F32 0
#define SV_DTYPE_BF16 1

/* Status codes. */
#define SV_OK 0
#define SV_ERR_NULL 1        /* a required pointer is NULL                        */
#define SV_ERR_SHAPE 2       /* B, gamma, n or V out of range, or sizes overflow   */
#define SV_ERR_TEMPERATURE 3 /* temperature not finite or outside [1e-6, 1e6]     */
#define SV_ERR_DTYPE 4       /* dtype is neither SV_DTYPE_F32 nor SV_DTYPE_BF16    */
#define SV_ERR_WORKSPACE 5   /* workspace too small or not 16-byte aligned         */
#define SV_ERR_HIP 6         /* the HIP runtime reported an error                  */
#define SV_ERR_ALIGN 7       /* a pointer is not aligned to its element size       */
#define SV_ERR_SCRATCH 8     /* sizes need more than SV_NOALLOC_SCRATCH_BYTES      */

/* Limits checked on the host. */
#define SV_MAX_GAMMA 255   /* draft positions per chain block                     */
#define SV_MAX_TREE_NODES 1024 /* nodes per tree, root included                   */
#define SV_MAX_VOCAB 536870912 /* vocabulary size V (2^29), every entry point     */

/* Human-readable name of a status code (static storage, never NULL). */
const char *spec_verify_status_string(int32_t status);

/* Bytes of workspace spec_verify_chain needs for these sizes; 0 if the sizes
 * or dtype are invalid. */
size_t spec_verify_chain_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype);

/* Chain verification (see the top of this file).
 *
 *  target_logits  [B][gamma+1][V] dtype: row i < gamma is the target's logits
 *                 at draft position i, row gamma the bonus row.
 *  draft_logits   [B][gamma][V] dtype: row i is the draft's logits at draft
 *                 position i (the distribution x_i was drawn from).
 *  draft_tokens   [B][gamma] int32: x_0 .. x_{gamma-1}.
 *  uniforms       [B][gamma+1] float32: entry i < gamma drives the test at
 *                 position i (accept iff u < min(1, p/q)); entry gamma drives
 *                 the final draw: the smallest token v with
 *                 sum_{t <= v} w(t) > u * sum_t w(t), w being the residual or
 *                 the bonus-row distribution (inverse CDF in ascending token
 *                 id).  Uniforms are expected in [0, 1).
 *  temperature    T, the same for every target and draft row; finite and in
 *                 [1e-6, 1e6].
 *  accept_len     out [B] int32: k in [0, gamma], or -1 for an invalid block.
 *  out_tokens     out [B][gamma+1] int32: x_0 .. x_{k-1}, then the
 *                 correction (k < gamma) or bonus (k = gamma) token, then -1.
 *  final_dist     out, NULLABLE [B][V] float32: the normalised distribution
 *                 the extra token was drawn from (zeros for invalid blocks).
 *                 When NULL it is neither computed nor written.
 *  workspace      device scratch of at least
 *                 spec_verify_chain_workspace_bytes(B, gamma, V, dtype)
 *                 bytes, 16-byte aligned (contents irrelevant).
 *  stream         hipStream_t to enqueue on (NULL = null stream).
 */
int32_t spec_verify_chain(const void *target_logits, const void *draft_logits, int32_t dtype,
                          const int32_t *draft_tokens, const float *uniforms, int32_t B,
                          int32_t gamma, int32_t V, double temperature, int32_t *accept_len,
                          int32_t *out_tokens, float *final_dist, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Scratch held by spec_verify_chain_noalloc on every GPU it runs on. */
#define SV_NOALLOC_SCRATCH_BYTES 16777216

/* Chain verification that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it.
 * Arguments, results and errors are those of spec_verify_chain without the
 * workspace (the same kernels run).  Its scratch is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES (16 MiB) in the library, one per GPU, held from
 * the first call on that GPU until the process ends; sizes whose workspace
 * (spec_verify_chain_workspace_bytes) exceeds it return SV_ERR_SCRATCH
 * before anything is enqueued.  The first call on a GPU looks the array's
 * address up (no allocation).  Every call on one GPU shares that array: two
 * calls whose work overlaps on one GPU (different streams, or host threads
 * racing) corrupt each other's scratch; calls ordered on one stream are
 * safe. */
int32_t spec_verify_chain_noalloc(const void *target_logits, const void *draft_logits,
                                  int32_t dtype, const int32_t *draft_tokens,
                                  const float *uniforms, int32_t B, int32_t gamma, int32_t V,
                                  double temperature, int32_t *accept_len, int32_t *out_tokens,
                                  float *final_dist, void *stream);

/* Bytes of workspace spec_verify_chain_pointmass needs for these sizes; 0 if
 * the sizes or dtype are invalid. */
size_t spec_verify_chain_pointmass_workspace_bytes(int32_t B, int32_t gamma, int32_t V,
                                                   int32_t dtype);

/* Point-mass ("exact-match") chain verification: the draft proposes each
 * token x_i with certainty (q_i is the point mass on x_i, as for a draft that
 * emits its argmax), so no draft logits are read ("JetSpec++", Appendix F.3
 * and Proposition 1; the worked example of Appendix F.1).  Position i passes
 * iff u_i < p_i(x_i), left to right; after a rejection at k the extra token
 * is drawn from p_k with x_k removed and the remainder renormalised, after a
 * fully accepted block from the bonus row p_gamma (inverse CDF in ascending
 * token id with u_gamma, as for spec_verify_chain).  The law of the outcome
 * equals that of spec_verify_chain with one-hot draft logits, and so do the
 * outputs for the same uniforms; the logits read are B*(gamma+1)*V instead
 * of B*(2*gamma+1)*V.
 *
 *  target_logits  [B][gamma+1][V] dtype, as for spec_verify_chain.
 *  draft_tokens   [B][gamma] int32: x_0 .. x_{gamma-1}.
 *  uniforms, temperature, accept_len, out_tokens, final_dist and stream are
 *  as for spec_verify_chain; the workspace is sized by
 *  spec_verify_chain_pointmass_workspace_bytes.  Data-dependent errors: a
 *  draft token outside [0, V), or a NaN, +inf or all -inf target row. */
int32_t spec_verify_chain_pointmass(const void *target_logits, int32_t dtype,
                                    const int32_t *draft_tokens, const float *uniforms,
                                    int32_t B, int32_t gamma, int32_t V, double temperature,
                                    int32_t *accept_len, int32_t *out_tokens, float *final_dist,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace spec_verify_tree_greedy needs; 0 if the sizes or dtype
 * are invalid. */
size_t spec_verify_tree_greedy_workspace_bytes(int32_t B, int32_t n, int32_t V, int32_t dtype);

/* Greedy tree verification (see the top of this file).
 *
 *  target_logits  [B][n][V] dtype: row j = the target's logits after the
 *                 root -> j path (row 0: after the verified context).
 *  parents        [B][n] int32: parents[0] = -1; 0 <= parents[j] < j.
 *  tokens         [B][n] int32: token of node j (tokens[0], the anchor, is
 *                 not checked).
 *  accept_len     out [B] int32: depth of the deepest accepted node (0 = no
 *                 draft token accepted), -1 for an invalid request.
 *  accept_node    out [B] int32: that node's index (0 = root; the lowest
 *                 index wins among accepted nodes of equal depth), -1 if
 *                 invalid.
 *  out_tokens     out [B][n] int32: the accepted path's tokens root -> leaf
 *                 (root excluded), then the target argmax after it (lowest
 *                 token id on ties), then -1.
 *  workspace      as for spec_verify_chain, sized by
 *                 spec_verify_tree_greedy_workspace_bytes.
 */
int32_t spec_verify_tree_greedy(const void *target_logits, int32_t dtype,
                                const int32_t *parents, const int32_t *tokens, int32_t B,
                                int32_t n, int32_t V, int32_t *accept_len, int32_t *accept_node,
                                int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Bytes of workspace spec_verify_tree_stochastic needs; 0 if the sizes or
 * dtype are invalid. */
size_t spec_verify_tree_stochastic_workspace_bytes(int32_t B, int32_t n, int32_t V, int32_t dtype);

/* Stochastic tree verification ("JetSpec" reading notes, section "Tree
 * verification": Eq. 16 and 17, Fig. 5).  For each of B requests, a
 * candidate tree of n nodes with target and draft logits per node; p_j and
 * q_j are the temperature softmax of target row j and draft row j, the
 * distributions of the token after node j's path.
 *  - Every node j >= 1 takes one Bernoulli test: accepted iff
 *    u[b][j] < min(1, p_par(y_j) / q_par(y_j)) with par = parents[j] and y_j
 *    = tokens[j] (a token of probability 0 under p is rejected; one of
 *    probability 0 under q but not under p is accepted).
 *  - A node counts as accepted iff every node on its path passed; v* is the
 *    deepest accepted node (lowest index among equally deep ones), the root
 *    if none.
 *  - The correction token is drawn from p_{v*} with u[b][0], by inverse CDF
 *    in ascending token id: the smallest v whose inclusive prefix sum
 *    exceeds u * (the total).  The pages give no residual rule for branches
 *    rejected below v*, and none is applied.
 *  THIS RULE DOES NOT PRESERVE THE TARGET DISTRIBUTION.  A child that the
 *  test rejects leaves its token's mass in p_{v*}, so a token the draft
 *  proposes more often than the target would emit it is committed too
 *  often: with one child drawn from q = (0.9, 0.1) under p = (0.5, 0.5),
 *  token 0 is committed with probability 0.7, not 0.5.  The rule is exact
 *  when every test is certain (one-hot targets give greedy verification)
 *  and when q = p.
 *
 *  target_logits, draft_logits  [B][n][V] dtype.
 *  parents, tokens  [B][n] int32, as for spec_verify_tree_greedy.
 *  uniforms      [B][n] float32 in [0, 1): u[b][0] drives the draw, u[b][j]
 *                node j's test.
 *  accept_len, accept_node, out_tokens  as for spec_verify_tree_greedy (the
 *                drawn token follows the path).
 *  final_dist    NULLABLE [B][V] float32: p_{v*} (zeros for an invalid
 *                request).
 *  An invalid request (a malformed parent array, a token outside [0, V), a
 *  NaN or +inf logit or a row without a finite logit in any target or draft
 *  row, or a row outside the numeric domain described at the top of this
 *  file) gets accept_len = accept_node = -1 and all tokens -1.
 *  workspace, stream: as for spec_verify_chain. */
int32_t spec_verify_tree_stochastic(const void *target_logits, const void *draft_logits,
                                    int32_t dtype, const int32_t *parents, const int32_t *tokens,
                                    const float *uniforms, int32_t B, int32_t n, int32_t V,
                                    double temperature, int32_t *accept_len, int32_t *accept_node,
                                    int32_t *out_tokens, float *final_dist, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Cache entries per request of spec_outcome_topk. */
#define SV_MAX_CACHE 16

/* Bytes of workspace spec_outcome_topk needs; 0 if the arguments are
 * invalid. */
size_t spec_outcome_topk_workspace_bytes(int32_t R, int32_t gamma, int32_t V, int32_t dtype,
                                         int32_t ncache);

/* Outcome scores and cache selection ("JetSpec++", Section 4.2 "Outcome
 * Selection"; Appendix F.1 and Proposition 1).  For each of R requests, row j
 * (j = 0..gamma) of `logits` is the decoder's estimate of the target's
 * next-token logits after the block's first j draft tokens; with
 * p_j = softmax(row_j / T) and x_j the draft tokens, the outcome (k, a) of
 * verifying the block -- k accepted draft tokens, then the extra token a --
 * has probability
 *   P(k, a) = prod_{i<k} p_i(x_i) * p_k(a)   for k < gamma and a != x_k,
 *   P(gamma, a) = prod_{i<gamma} p_i(x_i) * p_gamma(a).
 * The ncache most probable outcomes are returned, most probable first (equal
 * probabilities: smaller k, then smaller a); outcomes of probability 0 are
 * never returned, and unused slots hold k = a = -1, p = 0.  The hit
 * probability of that cache is the sum of the returned probabilities.
 *
 *  logits        [R][gamma+1][V] dtype (f32 or bf16 bits).
 *  draft_tokens  [R][gamma] int32.
 *  temperature   T > 0 (finite, in [1e-6, 1e6]); ncache in [1, SV_MAX_CACHE].
 *  out_k, out_a  out [R][ncache] int32; out_p out [R][ncache] double.
 *  hit           out [R] double: sum of out_p, or -1 for an invalid request
 *                (a draft token outside [0, V), a NaN or +inf logit, a row
 *                without a finite logit, or a row outside the numeric
 *                domain), whose slots are then all -1 / 0.
 *  workspace, stream: as for spec_verify_tree_greedy. */
int32_t spec_outcome_topk(const void *logits, int32_t dtype, const int32_t *draft_tokens,
                          int32_t R, int32_t gamma, int32_t V, double temperature, int32_t ncache,
                          int32_t *out_k, int32_t *out_a, double *out_p, double *hit,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Children per node, and rows times children, of spec_tree_build. */
#define SV_MAX_TREE_WIDTH 16
#define SV_MAX_TREE_SLOTS 2048

/* Bytes of workspace spec_tree_build needs; 0 if the arguments are invalid. */
size_t spec_tree_build_workspace_bytes(int32_t R, int32_t M, int32_t V, int32_t dtype, int32_t W,
                                       int32_t max_depth, int32_t budget);

/* Draft-tree construction by best-first search ("JetSpec" reading notes,
 * Algorithm 1, with the branch score of Eq. 15).  For each of R requests the
 * draft head has produced one row of logits per potential node: row m is the
 * draft distribution q_m = softmax(row_m / T) of the token after potential
 * node m's path, and row 0 belongs to the root (the verified prefix).  The
 * candidate children of a node whose row is m are the W most probable tokens
 * of q_m (ties: smaller token id; tokens of probability 0 are not
 * candidates); the child through the j-th of them has row child_row[m][j]
 * (-1: none).  The tree starts as the root (node 0, score 0); repeatedly the
 * queued node of highest score (ties: the one added first) is expanded --
 * each of its candidate children in order becomes the next node, with parent
 * the expanded node and score = parent's score + ln q_m(token) -- until the
 * tree holds `budget` nodes or nothing is left to expand.  Nodes at depth
 * max_depth and nodes without a row are never expanded.
 *
 *  draft_logits  [R][M][V] dtype (f32 or bf16 bits).
 *  child_row     NULLABLE [M][W] int32, shared by all requests, entries in
 *                [-1, M); NULL numbers the potential nodes breadth first in a
 *                complete W-ary tree: child j of row m has row m*W + 1 + j if
 *                that is below M, else none.
 *  temperature   T > 0 (finite, in [1e-6, 1e6]); W in [1, SV_MAX_TREE_WIDTH];
 *                M*W <= SV_MAX_TREE_SLOTS; max_depth >= 1; budget in
 *                [1, SV_MAX_TREE_NODES] (the root counts).
 *  parents, tokens, node_row  out [R][budget] int32: node j's parent (root
 *                -1; 0 <= parents[j] < j), token (root -1) and row (-1: none);
 *                -1 past the last node.  This is the parent/token layout
 *                spec_verify_tree_greedy takes.
 *  score         out [R][budget] double: the node's score (natural log; root
 *                0; -inf past the last node).
 *  n_nodes       out [R] int32: the number of nodes, or -1 for an invalid
 *                request (a NaN or +inf logit, a row without a finite logit,
 *                or a row outside the numeric domain, in any of its M rows,
 *                or a child_row entry outside [-1, M)), whose outputs are
 *                then all -1 / -inf.
 *  workspace, stream: as for spec_verify_tree_greedy. */
int32_t spec_tree_build(const void *draft_logits, int32_t dtype, const int32_t *child_row,
                        int32_t R, int32_t M, int32_t V, double temperature, int32_t W,
                        int32_t max_depth, int32_t budget, int32_t *parents, int32_t *tokens,
                        int32_t *node_row, double *score, int32_t *n_nodes, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Speculation-cache lookup ("JetSpec++", Section 4.2: a block drafted in
 * advance for the outcome (k, a) becomes the next block when verification
 * ends in exactly that outcome).  For each of R requests the verified outcome
 * is k = accept_len[r] and a = out_tokens[r][k]; slot[r] is the index of the
 * first cache entry with (cache_k, cache_a) = (k, a), or -1 for a miss, for an
 * invalid block (accept_len = -1) and for k outside [0, gamma].
 *
 *  accept_len      [R] int32 and out_tokens [R][gamma+1] int32, as written by
 *                  spec_verify_chain or spec_verify_chain_pointmass.
 *  cache_k, cache_a  [R][ncache] int32, as written by spec_outcome_topk for
 *                  the same block (k = -1 marks an unused slot, which never
 *                  matches).
 *  slot            out [R] int32.
 *  R >= 1, gamma in [1, SV_MAX_GAMMA], ncache in [1, SV_MAX_CACHE]; every
 *  pointer is a 4-byte aligned device pointer; one kernel on `stream`. */
int32_t spec_cache_lookup(const int32_t *accept_len, const int32_t *out_tokens, int32_t R,
                          int32_t gamma, const int32_t *cache_k, const int32_t *cache_a,
                          int32_t ncache, int32_t *slot, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
