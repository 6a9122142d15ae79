/*
 * sd.h -- C ABI of libsd, batched speculative-decoding draft verification on
 * AMD Instinct MI355X (gfx950).
 *
 * What each call computes is defined on the web page "大模型投机解码：Medusa、
 * MTP、EAGLE、DFlash、DDTree 与 DSpark" (chzhyang.github.io), cited as [SD §n]:
 * §1 (the acceptance-probability equation alpha = min(1, p/q), the A B C D
 * example of first-rejection truncation, the correction token from the
 * normalised positive residual, the extra token from p, greedy = target argmax,
 * temperature and truncation inside p and q), §2 (A excludes the correction /
 * extra token), §5 DDTree (the factorised score Q(u) = prod q_i(u_i), the
 * best-first tree under a node budget, the walk along the target's token) and
 * §5 DSpark (prefix survival s_j = prod c_i, expected advance 1 + sum s_j).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers (memory the caller allocated on the
 *   current HIP device), except `bytes` of sd_workspace_bytes (host). The caller
 *   owns every buffer; the library never allocates, frees or synchronises.
 * - Every call enqueues its kernels on `hip_stream` (a hipStream_t; NULL = the
 *   null stream) and returns. Outputs are valid once the stream has reached
 *   that point. Calls are stateless and may run concurrently on different
 *   streams when their workspaces and outputs are distinct.
 * - Rows are contiguous V-long vectors, row-major, int32 indices everywhere.
 *   Logits are fp32 (SD_F32) or bf16 (SD_BF16, raw 16-bit patterns).
 * - Alignment. The kernels read logit rows, tree marginals, KV rows and the
 *   workspace in 16-byte vectors, so those base pointers must be 16-byte
 *   aligned (any fresh device allocation is); a misaligned one returns
 *   SD_EINVAL before any HIP call.
 * - Batch layout of the chain calls. Sequence b has k_b draft positions:
 *   k_b = cu[b+1] - cu[b] when a `cu` array ([B+1], non-decreasing, cu[0] = 0)
 *   is given, else k_b = K_max with cu[b] = b*K_max. Draft row i of b is draft
 *   row cu[b]+i (i < k_b); target row i of b is target row cu[b]+b+i for
 *   i = 0..k_b, row k_b being the extra-token ("bonus") row. So a padded batch
 *   (cu == NULL) has B*(K_max+1) target rows and B*K_max draft rows, and a
 *   packed batch has cu[B]+B target rows and cu[B] draft rows, only the
 *   selected rows being read.
 * - Uniforms (chain, T > 0): uniforms[cu[b]+b+i] drives the accept test of
 *   position i; uniforms[cu[b]+b+k_b] drives the one final draw (correction or
 *   extra token). Values must lie in [0, 1).
 * - Errors. Invalid scalars or a NULL required pointer return SD_EINVAL before
 *   any HIP call, with nothing launched. A workspace smaller than
 *   sd_workspace_bytes returns SD_EWORKSPACE (nothing launched). A dtype that is
 *   not built for an op returns SD_EUNSUPPORTED. A failed launch returns SD_EHIP.
 *   Problems only the device can see do not abort a call: a draft token outside
 *   [0, V) or a non-finite row (its kept logits have no finite maximum or a NaN
 *   reaches its exponential sum) makes that position a rejection with p(y) = 0
 *   and sets bits in seq_status[b]; only positions 0..A and the row the final
 *   token is drawn from can set them. next_token is -1 when no token can be
 *   drawn (a non-finite decision row).
 * - Limits: 1 <= V < 2^24; 0 <= K_max <= 64; 1 <= B <= 2^20; tree budget
 *   2 <= N <= 64 and K <= 16; top_k <= 256; T >= 0 and finite.
 */
#ifndef SD_H_
#define SD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_ABI_VERSION 1

typedef enum {
    SD_OK = 0,
    SD_EINVAL = 1,
    SD_EUNSUPPORTED = 2,
    SD_EWORKSPACE = 3,
    SD_EHIP = 4
} sd_status_t;

typedef enum { SD_F32 = 0, SD_BF16 = 1 } sd_dtype_t;

typedef enum {
    SD_OP_CHAIN = 0,
    SD_OP_GREEDY = 1,
    SD_OP_BUILD_TREE = 2,
    SD_OP_VERIFY_TREE = 3,
    SD_OP_SELECT_LEN = 4,
    SD_OP_VERIFY_TREE_SAMPLED = 5
} sd_op_t;

/* seq_status bits */
#define SD_SEQ_BAD_TOKEN 1   /* a draft token outside [0, V) on the decision path */
#define SD_SEQ_NONFINITE 2   /* a non-finite row on the decision path             */

/* Largest supported values. */
#define SD_MAX_K 64
#define SD_MAX_TREE_N 64
#define SD_MAX_CANDIDATES 1024
#define SD_MAX_TREE_K 16
#define SD_MAX_TOPK 256
#define SD_MAX_EXPAND 64

/* Returns SD_ABI_VERSION. */
int sd_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* sd_status_str(int status);

/*
 * Workspace size in bytes (written to the HOST pointer `bytes`) that op needs
 * for these sizes. Pass the same B, K_max (tree: K), V, top_k and N as the call
 * itself (unused ones are ignored). Returns SD_EINVAL for out-of-range sizes.
 * The workspace is device memory, 256-byte aligned, owned by the caller, and
 * needs no initialisation; a call overwrites the part it uses.
 */
sd_status_t sd_workspace_bytes(sd_op_t op, int32_t B, int32_t K_max, int32_t V,
                               int32_t top_k, int32_t N, size_t* bytes);

/*
 * Chain verification [SD §1].
 *
 * T > 0 (stochastic speculative sampling). With p_i = softmax of target row i
 * and q_i = softmax of draft row i, both after dividing the logits by T and,
 * when 1 <= top_k < V, keeping only the top_k logits ordered by (logit desc,
 * id asc) (NaN never kept):
 *   position i is accepted iff p_i(y_i) > 0 and u_i * q_i(y_i) <= p_i(y_i);
 *   A = the first rejected position, or k_b when all pass;
 *   if A < k_b the next token is drawn from the normalised residual
 *   max(p_A - q_A, 0) by inverse CDF in token-id order at u_{k_b} * R
 *   (R = the residual's total mass); if A == k_b it is drawn from p_{k_b} the
 *   same way at u_{k_b}.
 * T == 0 (greedy): position i is accepted iff y_i is the lowest-id argmax of
 * the raw target row i; next_token is that argmax at row A. draft_logits and
 * uniforms may then be NULL, top_k is ignored, probs_out / resid_mass_out are
 * not written.
 *
 *   target_logits  [R_t, V] dtype          (see "Batch layout")
 *   draft_logits   [R_d, V] dtype
 *   draft_tokens   [R_d] int32             y_i
 *   uniforms       [R_t] fp32 in [0,1)
 *   cu_draft       [B+1] int32 or NULL     packed offsets (device)
 *   accepted_len   [B] int32 out           A (excludes the correction/extra token)
 *   next_token     [B] int32 out           correction if A < k_b, else extra token
 *   probs_out      [R_d, 2] fp32 out or NULL   (p_i(y_i), q_i(y_i)) for every position
 *   resid_mass_out [B] fp32 out or NULL    R (0 for an extra token)
 *   seq_status     [B] int32 out or NULL   SD_SEQ_* bits
 */
sd_status_t sd_verify_chain(const void* target_logits, const void* draft_logits,
                            sd_dtype_t dtype, const int32_t* draft_tokens,
                            const float* uniforms, const int32_t* cu_draft,
                            int32_t B, int32_t K_max, int32_t V,
                            float temperature, int32_t top_k,
                            int32_t* accepted_len, int32_t* next_token,
                            float* probs_out, float* resid_mass_out, int32_t* seq_status,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Cap-accept chain verification [SD §9 DSpark: the ragged-verify mode that
 * keeps the full verification work but limits the committed length]. The
 * batch is padded (no cu: sequence b owns target rows b*(K_max+1) ..
 * b*(K_max+1)+K_max, draft rows b*K_max .., uniforms indexed as the target
 * rows); every position of the window is evaluated, as in the "static" mode
 * (sd_verify_chain with cu_draft == NULL). The committed result is that of
 * sd_verify_chain over the first kc = clamp(k_cap[b], 0, K_max) positions
 * only (accept tests with uniforms 0..kc-1, the final token drawn with uniform
 * kc from the residual at A or, when all kc pass, from target row kc), i.e.
 * the tokens the compact mode commits with k_b = kc.
 *
 *   k_cap          [B] int32 (device)      committed-length cap per sequence
 *   accepted_len   [B] int32 out           committed A (<= kc)
 *   next_token     [B] int32 out           correction if A < kc, else extra token
 *   accepted_full  [B] int32 out or NULL   first rejection over all K_max positions
 *   probs_out      [B*K_max, 2] fp32 out or NULL  (p_i(y_i), q_i(y_i)), every position
 *   resid_mass_out, seq_status: as sd_verify_chain, for the committed decision
 * T == 0 gives the greedy rule with the same cap. Workspace as sd_verify_chain
 * (SD_OP_CHAIN). Errors as sd_verify_chain; k_cap == NULL is SD_EINVAL.
 */
sd_status_t sd_verify_chain_capped(const void* target_logits, const void* draft_logits,
                                   sd_dtype_t dtype, const int32_t* draft_tokens,
                                   const float* uniforms, const int32_t* k_cap,
                                   int32_t B, int32_t K_max, int32_t V,
                                   float temperature, int32_t top_k,
                                   int32_t* accepted_len, int32_t* next_token,
                                   int32_t* accepted_full, float* probs_out,
                                   float* resid_mass_out, int32_t* seq_status,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * sd_verify_chain without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, computation, outputs and
 * errors as sd_verify_chain, but the scratch space is a file-scope device
 * array of SD_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held
 * until the process ends). The call allocates nothing: its first use on a
 * device only looks up that device's copy of the array (hipGetSymbolAddress).
 * A call whose path needs more than SD_NOALLOC_SCRATCH_BYTES of scratch
 * (sd_workspace_bytes gives an upper bound) returns SD_EWORKSPACE with
 * nothing launched; at V = 128256, K_max = 8 the full-vocabulary path fits
 * up to B = 4999 with bf16 logits and B = 2577 with fp32 logits. Every call on one GPU shares that array, so two calls
 * that overlap in time on the same GPU (different streams, or host threads)
 * race: serialise them. The scratch needs no clearing between calls.
 */
#define SD_NOALLOC_SCRATCH_BYTES (16u << 20)
sd_status_t sd_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                    sd_dtype_t dtype, const int32_t* draft_tokens,
                                    const float* uniforms, const int32_t* cu_draft,
                                    int32_t B, int32_t K_max, int32_t V,
                                    float temperature, int32_t top_k,
                                    int32_t* accepted_len, int32_t* next_token,
                                    float* probs_out, float* resid_mass_out,
                                    int32_t* seq_status, void* hip_stream);

/*
 * Greedy chain verification [SD §1: greedy results follow the target argmax].
 * g_i = lowest-id argmax of raw target row i (NaN ignored); position i is
 * accepted iff y_i == g_i; A = first mismatch (or k_b); next_token = g_A.
 * Same layout and outputs as sd_verify_chain with T == 0.
 */
sd_status_t sd_verify_greedy(const void* target_logits, sd_dtype_t dtype,
                             const int32_t* draft_tokens, const int32_t* cu_draft,
                             int32_t B, int32_t K_max, int32_t V,
                             int32_t* accepted_len, int32_t* next_token, int32_t* seq_status,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * DDTree candidate tree [SD §5 DDTree].
 *
 *   marginals  [B, K, V] fp32 probabilities; row d is the draft marginal of
 *              depth d+1 (q_{d+1}); entries must be >= 0 and not NaN.
 * L_d = the ids of row d ordered by (q desc, id asc), cut to N-1 entries. A
 * prefix (r_1..r_m) (m <= K) names tokens L_1[r_1]..L_m[r_m] and scores
 * Q = fl32(...fl32(q_1 * q_2)... * q_m) (fp32, left to right). Prefixes are
 * ordered by (Q desc, m asc, rank tuple lexicographically asc); the tree is the
 * root (node 0: token -1, parent -1, depth 0, score 1, mask bit 0) plus the
 * first N-1 prefixes of that order, found best-first with a priority queue and
 * numbered in pop order (fewer when the whole trie is smaller).
 *
 *   node_token, node_parent, node_depth [B, N] int32 out (unused slots: -1, -1, 0)
 *   node_score   [B, N] fp32 out            Q (unused slots: 0)
 *   node_anc_mask[B, N] uint64 out          bit j set iff node j is the node or an
 *                                           ancestor of it (unused slots: 0)
 *   n_nodes      [B] int32 out
 */
sd_status_t sd_build_tree(const float* marginals, int32_t B, int32_t K, int32_t V, int32_t N,
                          int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                          float* node_score, uint64_t* node_anc_mask, int32_t* n_nodes,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * DDTree walk [SD §5 DDTree]. target_logits [B, N, V] dtype: row n is the target
 * distribution after node n (row 0 after the root/anchor). From the root, take
 * g = lowest-id argmax of the current node's row; if a child of the node carries
 * token g, move there and record it; otherwise g is next_token.
 *
 *   node_token, node_parent [B, N] int32, n_nodes [B] int32 (as built)
 *   path_nodes   [B, N] int32 out   accepted node ids in walk order (root
 *                                   excluded), -1 padded
 *   accepted_len [B] int32 out      path length
 *   next_token   [B] int32 out      the target's token after the path (-1 if
 *                                   that row is all NaN)
 * Only the rows on the walk are read, one per step. The workspace arguments
 * are unused (sd_workspace_bytes returns 0 for SD_OP_VERIFY_TREE; NULL is
 * accepted).
 */
sd_status_t sd_verify_tree(const void* target_logits, sd_dtype_t dtype,
                           const int32_t* node_token, const int32_t* node_parent,
                           const int32_t* n_nodes, int32_t B, int32_t N, int32_t V,
                           int32_t* path_nodes, int32_t* accepted_len, int32_t* next_token,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * DDTree walk under a sampling target [SD §5 DDTree: the walk follows the token
 * the target selects at each node, and the first node without a child carrying
 * it turns that token into the extra token; SD §1: temperature and truncation
 * belong inside p, and the chain's ratio test is not a rule for a tree]. At
 * node n the target selects its token by drawing from its own row: the inverse
 * CDF, in token-id order, of p_n = softmax(target row n / T) over its kept
 * set (top_k below) at uniforms[b*N + n] (the first token whose running mass
 * exceeds the uniform;
 * if rounding leaves none, the last token with positive mass). The tree's
 * nodes are fixed drafts, so no draft probability enters; a walk visits a node
 * at most once, so every draw has a fresh uniform and each committed token is
 * a draw from the target given the tokens before it. T == 0 takes the lowest-id
 * argmax instead, the walk of sd_verify_tree.
 *
 *   target_logits [B, N, V] dtype     row n: target distribution after node n
 *   node_token, node_parent [B, N] int32, n_nodes [B] int32 (as built)
 *   uniforms     [B, N] fp32 in [0, 1) (ignored and may be NULL when T == 0)
 *   temperature  T >= 0, finite
 *   top_k        0 (or >= V): no truncation; 1 .. SD_MAX_TOPK: p_n keeps the
 *                top_k ids of row n by (logit desc, id asc), as in the chain
 *   path_nodes   [B, N] int32 out     accepted node ids in walk order (root
 *                                     excluded), -1 padded
 *   accepted_len [B] int32 out; next_token [B] int32 out (-1 when the row it
 *                would be drawn from is non-finite)
 *   seq_status   [B] int32 out or NULL: SD_SEQ_NONFINITE when a visited row is
 *                non-finite (no finite maximum, or a NaN in its sum); the walk
 *                stops there
 *   workspace    unused (sd_workspace_bytes returns 0 for
 *                SD_OP_VERIFY_TREE_SAMPLED; NULL is accepted)
 *
 * Only the rows on the walk are read, one per step; with truncation the step
 * takes the exact top_k of its row on the fly.
 */
sd_status_t sd_verify_tree_sampled(const void* target_logits, sd_dtype_t dtype,
                                   const int32_t* node_token, const int32_t* node_parent,
                                   const int32_t* n_nodes, const float* uniforms, int32_t B,
                                   int32_t N, int32_t V, float temperature, int32_t top_k,
                                   int32_t* path_nodes, int32_t* accepted_len,
                                   int32_t* next_token, int32_t* seq_status, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

/*
 * EAGLE-2-style expansion step [SD §4 EAGLE-2: the candidate tree grows by
 * expanding the branches of highest cumulative path confidence; its
 * candidates are then re-ranked by sd_rerank_tree]. Per sequence b the
 * candidates sit in [B, M] arrays in topological order (the layout
 * sd_rerank_tree reads) with cand_conf, each candidate's cumulative
 * confidence (-1 for an unusable one). One call adds one layer:
 *   - n_cand[b] == 0 starts the tree: candidate 0 becomes the root (parent -1,
 *     token -1, prob 1, conf 1) and is the one node expanded. Otherwise slot
 *     w < W expands node expand_in[b, w] when 0 <= id < n_cand[b] and
 *     cand_conf[b, id] >= 0 (other slots are skipped).
 *   - The children of the node in slot w are child_token[b, w, c] with
 *     conditional draft probability child_prob[b, w, c] (c < C): the draft's
 *     proposals for that node, an input. The expanded slots' children are
 *     appended in slot order, C per slot, from n_cand[b] on, as long as the
 *     index stays below M (the rest are dropped). A child's parent is its
 *     node; its confidence is fl32(cand_conf[parent] * prob) when prob lies
 *     in [0, 1], else -1 (never expanded, and left out by sd_rerank_tree).
 *   - n_cand[b] is updated, and expand_out[b, 0..W) receives the appended
 *     candidates with confidence >= 0 ordered by (confidence desc, index asc),
 *     the first W of them, -1 padded: the nodes the next call expands.
 *
 *   cand_parent, cand_token [B, M] int32, cand_prob, cand_conf [B, M] fp32,
 *   n_cand [B] int32: read and written (only entries from the old n_cand[b]
 *   on are written, plus the root); expand_in [B, W] int32 (may be NULL when
 *   every n_cand[b] is 0; may be the same array as expand_out, which is
 *   written only after it is read); child_token [B, W, C] int32, child_prob
 *   [B, W, C] fp32. Limits 1 <= M <= SD_MAX_CANDIDATES, 1 <= W <=
 *   SD_MAX_EXPAND, 1 <= C <= SD_MAX_CANDIDATES. Needs no workspace.
 */
sd_status_t sd_expand_tree(int32_t* cand_parent, int32_t* cand_token, float* cand_prob,
                           float* cand_conf, int32_t* n_cand, const int32_t* expand_in,
                           int32_t* expand_out, const int32_t* child_token,
                           const float* child_prob, int32_t B, int32_t M, int32_t W, int32_t C,
                           void* hip_stream);

/*
 * EAGLE-2-style verification tree [SD §4 EAGLE-2: candidates expanded along
 * paths of high cumulative confidence are re-ranked and the final verification
 * tree is chosen from them]. Per sequence, an expanded candidate tree in
 * topological order: candidate 0 is the root; candidate i (1 <= i < n_cand[b])
 * has a parent in [0, i), a token and a conditional draft probability in [0, 1]
 * (a candidate with another parent or probability, or NaN, is left out with its
 * subtree). Its confidence is the fp32 product of the probabilities along its
 * path, root first. The tree is the root plus the first N-1 candidates by
 * (confidence desc, depth asc, candidate index asc) -- a child never precedes
 * its parent, so every kept node's parent is kept -- numbered in that order.
 * Outputs as sd_build_tree (node 0 the root; unused slots: token -1, parent -1,
 * depth 0, score 0, mask 0), plus node_cand[b, n], the candidate behind node n
 * (0 for the root, -1 unused; may be NULL).
 *
 *   cand_parent, cand_token [B, M] int32; cand_prob [B, M] fp32; n_cand [B] int32
 *   M <= SD_MAX_CANDIDATES, 2 <= N <= SD_MAX_TREE_N. Needs no workspace.
 */
sd_status_t sd_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token,
                           const float* cand_prob, const int32_t* n_cand, int32_t B, int32_t M,
                           int32_t N, int32_t* node_token, int32_t* node_parent,
                           int32_t* node_depth, float* node_score, uint64_t* node_anc_mask,
                           int32_t* node_cand, int32_t* n_nodes, void* hip_stream);

/*
 * Accepted-path KV compaction [SD §5 DDTree: after the walk the KV cache keeps
 * only the accepted path]. `kv` holds n_rows rows of row_bytes bytes each (one
 * token's keys and values, laid out as the caller likes; row_bytes a positive
 * multiple of 16, kv 16-byte aligned). Draft node n (1 .. N-1) of sequence b
 * wrote its row at row_base[b] + n - 1. The accepted path moves in place:
 * afterwards row row_base[b] + i holds what row row_base[b] + path_nodes[b, i]
 * - 1 held before the call, for i < accepted_len[b]; no other row changes.
 * path_nodes / accepted_len are as sd_verify_tree writes them (node ids in walk
 * order, which grow along a path: the moves rely on it). A sequence whose
 * draft region [row_base[b], row_base[b] + N - 1) is not inside [0, n_rows) is
 * left untouched; a path entry outside [1, N-1] is skipped.
 *
 *   kv            [n_rows, row_bytes] bytes (device), updated in place
 *   row_base      [B] int64 (device)
 *   path_nodes    [B, N] int32 (device)
 *   accepted_len  [B] int32 (device)
 * Needs no workspace. Bad sizes or NULL pointers are SD_EINVAL.
 */
sd_status_t sd_compact_kv(void* kv, int64_t row_bytes, int64_t n_rows, const int64_t* row_base,
                          const int32_t* path_nodes, const int32_t* accepted_len, int32_t B,
                          int32_t N, void* hip_stream);

/*
 * DSpark verify length [SD §5 DSpark]. s_0 = 1, s_j = fl32(s_{j-1} * c_j);
 * k_sel[b] = the largest k with s_j > cost_per_position for every j <= k
 * (for c in [0, 1] this is the smallest k maximising 1 + sum_{j<=k} s_j - cost*k);
 * expected_advance[b] = 1 + sum_{j <= k_sel} s_j; cu_sel = exclusive prefix sum
 * of k_sel ([B+1], usable directly as cu_draft of a packed sd_verify_chain).
 *
 *   conf [B, K_max] fp32 in [0, 1]
 *   k_sel [B] int32 out; expected_advance [B] fp32 out or NULL; cu_sel [B+1] int32 out or NULL
 * Needs no workspace.
 */
sd_status_t sd_select_len(const float* conf, int32_t B, int32_t K_max, float cost_per_position,
                          int32_t* k_sel, float* expected_advance, int32_t* cu_sel,
                          void* hip_stream);

/*
 * DSpark verify length with a per-position cost table [SD §5 DSpark: is one
 * more verified position worth what it costs]. cost_table[j-1] is the cost of
 * verifying position j (in tokens of advance, e.g. a measured per-position
 * time over the time of one decoding round). k_sel[b] = the smallest k in
 * [0, K_max] maximising f(k) = 1 + sum_{j<=k} s_j - sum_{j<=k} cost_table[j-1],
 * the two sums running in fp64 in position order over the fp32 s_j and costs
 * (a constant table gives sd_select_len's k for c in [0, 1]). Outputs as
 * sd_select_len.
 *
 *   conf [B, K_max] fp32 in [0, 1]; cost_table [K_max] fp32 (device), finite
 *   (a NaN or +inf cost makes every length that includes it lose; -inf wins)
 * Needs no workspace. conf or cost_table NULL with K_max > 0 is SD_EINVAL.
 */
sd_status_t sd_select_len_table(const float* conf, int32_t B, int32_t K_max,
                                const float* cost_table, int32_t* k_sel,
                                float* expected_advance, int32_t* cu_sel, void* hip_stream);

/*
 * Measurement support: a plain streaming read of `bytes` bytes (a multiple of
 * 16, 16-byte aligned) of device memory by n_blocks workgroups of 256 threads,
 * each reading one contiguous chunk, with the 16-byte loads the row passes use; sink [n_blocks] receives one
 * word per workgroup (a fold of what it read). It is the read ceiling the
 * verification kernels are compared with on the same device, and takes the
 * events of sd_time_next_stream_pass like the row passes.
 */
sd_status_t sd_stream_read(const void* data, size_t bytes, uint32_t* sink, int32_t n_blocks,
                           void* hip_stream);

/*
 * Measurement support: the same plain read over a row-major matrix of n_rows
 * rows of row_bytes bytes each (row r starts at data + r * row_bytes; both a
 * multiple of 16, data 16-byte aligned), each row split into chunks of
 * chunk_bytes (a multiple of 16; the last chunk of a row is shorter), one
 * 256-thread workgroup per (row, chunk): the grid the row passes use. sink
 * [n_rows * ceil(row_bytes / chunk_bytes)] receives each workgroup's fold
 * (the XOR of every 32-bit word of its chunk), row-major. SD_EINVAL for NULL
 * pointers, misalignment, zero or non-multiple-of-16 sizes, row_bytes above
 * 2^32 or more than 2^24 workgroups. Takes the events of
 * sd_time_next_stream_pass.
 */
sd_status_t sd_stream_read_rows(const void* data, size_t row_bytes, int32_t n_rows, size_t chunk_bytes,
                                uint32_t* sink, void* hip_stream);

/*
 * Measurement support. The next sd_verify_chain, sd_verify_chain_capped,
 * sd_verify_greedy, sd_build_tree, sd_verify_tree, sd_compact_kv or
 * sd_rerank_tree call made by the calling host thread binds `start_event` and
 * `stop_event` to its streaming kernel (the one pass over the logit / marginal
 * rows, which dominates its time): the kernel is launched with
 * hipExtLaunchKernel, so the events take that dispatch's own start and end
 * times and add no marker packets to the stream. The hook then clears itself.
 * Both are hipEvent_t handles created by the caller; hipEventElapsedTime of the
 * pair is that kernel's duration. A call with no such kernel (no tree rows)
 * records the two events back to back. Passing NULL, NULL clears a pending
 * hook. Returns SD_OK.
 */
sd_status_t sd_time_next_stream_pass(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* SD_H_ */
