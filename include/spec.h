/*
 * spec.h - C ABI of the tree speculative-decoding hot path for AMD MI355X
 * (gfx950): tree build, tree-masked verify attention, greedy and
 * rejection-sampled tree accept, accepted-KV compaction; the target-only
 * tree accept, the draft step, the top-k / top-p pre-pass, the FULL mask and
 * paged draft-branch planning.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "SGLang 源码完全拆解(十一):投机解码——草稿生成、批量验证与 token 接受如何接进同一条前向"
 *   [P2] "投机解码 Accept:从 Verify 行到最终输出路径"
 *   [P4] "Speculative Decoding" (sglang-internals book, execution model)
 *   [P5] "把投机采样讲透:以 SGLang 中的 EAGLE-2 为例"
 *
 * Conventions shared by every entry point
 *   - Every pointer is a device pointer on the current HIP device unless a
 *     comment says otherwise.  All tensors are dense and row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work: they never synchronise, never allocate and
 *     keep no state between calls, so they are re-entrant.
 *   - The caller owns every buffer.  Inputs are never written, except the KV
 *     pools of spec_compact_kv, which are updated in place.
 *   - Return value: SPEC_OK, or a negative SPEC_ERR_* when a host-side check
 *     fails; then nothing was launched.
 *   - `dev_status` (may be NULL) is one int32 on the device.  Kernels OR the
 *     SPEC_ST_* bits into it for data-dependent problems; the caller zeroes it
 *     and reads it whenever it likes.  This replaces the index-range guard
 *     the pages run before gathers ([P1] organize_draft_results, KV 回写).
 *   - batch == 0 is a valid no-op (the pages' idle batch returns empty
 *     results, [P1] eagle_sample 的骨架).
 *   - -1 means "none" in retrieve_* and accept_index ([P1] 邻接表:retrieve_* 三兄弟).
 *   - Tree node k of request b occupies flattened verify row b*n + k.
 *   - bf16 tensors are raw bfloat16 (16-bit) values; f32 are IEEE binary32.
 *   - Every call may be recorded into a HIP graph (stream capture).  A
 *     recorded call may later run beside other streams' kernels, and a graph
 *     does not keep a cooperative launch's co-residency guarantee, so the
 *     accepts record forms whose outputs never depend on other workgroups
 *     being scheduled: the greedy accept always runs its tree walk as a
 *     kernel of its own after the vocabulary sweep (it never waits), and
 *     so does the recorded target-only accept; the sampled walk runs its
 *     co-resident form as an ordinary kernel followed by a recovery kernel
 *     that walks again, one workgroup per request, every request whose
 *     wait gave up.  Recorded calls therefore never raise SPEC_ST_SYNC.
 *     Eager calls use the one-launch forms: a cooperative launch (sampled),
 *     or walkers fewer than the device holds at once that wait only on
 *     sweep work (target-only).
 *   - Waits between workgroups are bounded: after SPEC_POLL_LIMIT polls of
 *     one slot (environment variable read on every call, decimal, default
 *     1048576, about a second) a wait gives up; in an eager call it raises
 *     SPEC_ST_SYNC.
 */
#ifndef SPECMI_SPEC_H
#define SPECMI_SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum spec_error {
    SPEC_OK = 0,
    SPEC_ERR_NULL = -1,        /* a required pointer is NULL                      */
    SPEC_ERR_SHAPE = -2,       /* sizes inconsistent or out of the supported range */
    SPEC_ERR_DTYPE = -3,       /* dtype code not SPEC_F32 / SPEC_BF16              */
    SPEC_ERR_UNSUPPORTED = -4, /* valid request this build does not implement      */
    SPEC_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required          */
    SPEC_ERR_HIP = -6          /* a HIP launch reported an error                   */
};

enum spec_status_bits {
    SPEC_ST_RANGE = 1,          /* an index (parent, row, slot, page) out of range  */
    SPEC_ST_NOT_CLOSED = 2,     /* a kept node's parent was not kept                */
    SPEC_ST_DEPTH = 4,          /* accepted path longer than accept_width           */
    SPEC_ST_ZERO_RESIDUAL = 8,  /* residual mass exactly zero (informational)       */
    SPEC_ST_SYNC = 16           /* a wait for another workgroup's partial result
                                   timed out; that call's sampled outputs are
                                   unspecified                                      */
};

enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 };
enum spec_mask_mode { SPEC_MASK_QLEN_U8 = 1, SPEC_MASK_QLEN_BITS = 2 };

typedef void *spec_stream_t;

/* Library version (major*10000 + minor*100 + patch). */
int spec_version(void);

/* Human-readable text of a return code. */
const char *spec_status_string(int status);

/* Bytes per row of a SPEC_MASK_QLEN_BITS tree mask: 1, 2, 4 or 8, i.e. the
 * word of 8 << ceil(log2(ceil(n / 8))) bits the page gives for
 * QLEN_ONLY_BITPACKING ([P1] 三种 mask 形态).  0 if n is outside 1..64. */
int spec_mask_word_bytes(int num_draft_tokens);

/*
 * Tree build.  [P1] organize_draft_results and build_tree_kernel_efficient;
 * [P5] 4.3 (tree mask, positions); [P2] 二 (first-child / next-sibling).
 *
 * Inputs, per request b (ncand = topk + (num_steps-1)*topk*topk,
 * npar = 1 + (num_steps-1)*topk):
 *   scores   [batch, ncand] f32  path score of every draft candidate, in the
 *                                order the draft steps produced them (the
 *                                score list concatenated and flattened)
 *   tokens   [batch, ncand] i32  token id of every candidate (same order)
 *   parents  [batch, npar]  i32  the parent list of all steps but the last:
 *                                entry r is the flat candidate index whose
 *                                expansion produced score row r (entry 0 is
 *                                the root sentinel -1 and is not read)
 *   bonus    [batch]        i32  previous round's terminal token = tree root
 *   seq_lens [batch]        i32  committed history length (prefix length)
 * What is computed:
 *   the num_draft_tokens-1 candidates with the largest scores are kept
 *   (ties: lower flat index first), their flat indices sorted ascending;
 *   node 0 is the bonus token, node k >= 1 is kept candidate k-1.  A kept
 *   candidate f < topk hangs off the root; otherwise its parent is the node
 *   holding flat index parents[f / topk].
 * Outputs:
 *   draft_tokens [batch*n] i32       node tokens, root first
 *   positions    [batch*n] i32       seq_lens[b] + depth (siblings share one)
 *   tree_mask    SPEC_MASK_QLEN_U8:   [batch, n, n] u8, 1 where column node j
 *                                     is row node k itself or an ancestor
 *                SPEC_MASK_QLEN_BITS: [batch, n] words of
 *                                     spec_mask_word_bytes(n) bytes,
 *                                     little-endian, bit j = node j visible
 *   retrieve_index        [batch, n] i32  b*n + k
 *   retrieve_next_token   [batch, n] i32  smallest child index, -1 if leaf
 *   retrieve_next_sibling [batch, n] i32  next larger index with the same
 *                                         parent, -1 if none (root: -1)
 *   selected [batch, n-1] i32 (optional, NULL to skip) kept flat indices
 * Data errors: parent index outside [0, ncand) -> SPEC_ST_RANGE; parent not
 *   kept -> SPEC_ST_NOT_CLOSED; such a node is attached to the root.
 * Limits: 1 <= n <= 64, n-1 <= ncand <= 4096, topk >= 1, num_steps >= 1.
 * Scores must not be NaN.  When n - 1 = ncand every candidate is kept (the
 * chain of a topk-1 draft with n = num_steps + 1): the selection is the
 * identity, the ranking is skipped and scores are not read.
 */
int spec_build_tree(int batch, int topk, int num_steps, int num_draft_tokens, int mask_mode,
                    const float *scores, const int32_t *tokens, const int32_t *parents,
                    const int32_t *bonus, const int32_t *seq_lens,
                    int32_t *draft_tokens, int32_t *positions, void *tree_mask,
                    int32_t *retrieve_index, int32_t *retrieve_next_token,
                    int32_t *retrieve_next_sibling, int32_t *selected,
                    int32_t *dev_status, spec_stream_t stream);

/*
 * Verify attention.  [P5] 4.2-4.3 and [P1] 验证前向的组装: every tree node
 * is a query row; it attends to the request's whole cached history and to
 * the tree nodes its mask row allows (itself and its ancestors), whose K/V
 * the verify forward has written at out_cache_loc.
 *
 *   q        [batch*n, num_q_heads, head_dim]   dtype
 *   k_pool, v_pool [num_slots, num_kv_heads, head_dim]  dtype (one layer)
 *   page_table [batch, max_pages] i32  history position p of request b is
 *            slot page_table[b][p / page_size] * page_size + p % page_size
 *   seq_lens [batch] i32  history length L_b (0 allowed); positions
 *            0 .. L_b-1 are history, the tree's K/V are at out_cache_loc
 *   max_seq_len  host int, an upper bound of seq_lens (sizes the launch);
 *            a request with L_b > max_seq_len raises SPEC_ST_RANGE and its
 *            output is left unwritten
 *   out_cache_loc [batch*n] i32  slot of tree node k of request b
 *   tree_mask  [batch, n] SPEC_MASK_QLEN_BITS words (spec_mask_word_bytes)
 *   out      [batch*n, num_q_heads, head_dim]  dtype of q
 *   sm_scale   softmax scale; <= 0 selects 1/sqrt(head_dim)
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  Scores,
 * softmax and accumulation are fp32 (online softmax); bf16 operands use the
 * matrix cores.
 * workspace: at least spec_verify_attention_workspace_size(...) bytes, any
 * contents.  Slots or page ids out of range raise SPEC_ST_RANGE; the output
 * is then unspecified (no read leaves the pools).
 * Limits: 1 <= n <= 64; head_dim 64 or 128; num_q_heads % num_kv_heads == 0;
 * page_size >= 1; num_slots <= 2^31 - 1 (else SPEC_ERR_UNSUPPORTED);
 * num_slots >= 1 when batch > 0 (else SPEC_ERR_SHAPE).
 */
size_t spec_verify_attention_workspace_size(int batch, int num_draft_tokens, int num_q_heads,
                                            int num_kv_heads, int head_dim, int max_seq_len,
                                            int dtype);
int spec_verify_attention(int batch, int num_draft_tokens, int num_q_heads, int num_kv_heads,
                          int head_dim, int page_size, int dtype, float sm_scale,
                          const void *q, const void *k_pool, const void *v_pool,
                          int64_t num_slots, const int32_t *page_table, int max_pages,
                          const int32_t *seq_lens, int max_seq_len,
                          const int32_t *out_cache_loc, const void *tree_mask, void *out,
                          void *workspace, size_t workspace_bytes, int32_t *dev_status,
                          spec_stream_t stream);

/*
 * Greedy tree accept.  [P1] 三条判定路径 (argmax, then the tree walk);
 * [P2] 三 (row indices and the one-position offset); [P5] 5.3.
 *
 *   target_logits [batch*n, vocab] dtype   verify rows' logits
 *   candidates    [batch*n] i32            = draft_tokens of the tree build
 *   retrieve_*    [batch, n] i32           from spec_build_tree
 *   accept_width  = num_steps + 1 (columns of accept_index)
 * For every row the target's choice is the first index of the row maximum.
 * From the root the walk scans the children (first child, then siblings) for
 * the candidate equal to the current row's choice, descends on a match and
 * stops otherwise.  Outputs (all fully written):
 *   predict       [batch*n] i32  on the path, row(node) holds the accepted
 *                                child's token, the last node's row the
 *                                target's choice (the terminal token);
 *                                other rows 0
 *   accept_index  [batch, accept_width] i32  verify rows of root and
 *                                accepted nodes, then -1
 *   accept_length [batch] i32    accepted drafts + 1
 *   target_predict [batch*n] i32 (optional, NULL to skip) every row's choice
 * A path that would exceed accept_width raises SPEC_ST_DEPTH and stops there.
 * Two launches (the vocabulary sweep folds each chunk's best entry into its
 * row's key with an atomic max; the walk reads the keys); no workgroup
 * waits for another, so the call never raises SPEC_ST_SYNC.
 * workspace: spec_accept_workspace_size(batch, n, vocab, 0) bytes (a 64-bit
 *   key per verify row), 8-byte aligned and zero-filled before its first
 *   use; every call leaves it zero-filled again, so one workspace serves any
 *   number of calls in stream order (concurrent calls need one each).
 * Logits must not be NaN.
 */
size_t spec_accept_workspace_size(int batch, int num_draft_tokens, int64_t vocab, int sampled);
int spec_accept_greedy(int batch, int num_draft_tokens, int accept_width, int64_t vocab,
                       int dtype, const void *target_logits, const int32_t *candidates,
                       const int32_t *retrieve_index, const int32_t *retrieve_next_token,
                       const int32_t *retrieve_next_sibling, int32_t *predict,
                       int32_t *accept_index, int32_t *accept_length, int32_t *target_predict,
                       void *workspace, size_t workspace_bytes, int32_t *dev_status,
                       spec_stream_t stream);

/*
 * spec_accept_greedy without a workspace, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, outputs and errors as
 * spec_accept_greedy.  The row keys live in a fixed array inside the
 * library (256 KiB on each device the library runs on, held until the
 * process ends): a call needs batch * n <= 32768 keys, else
 * SPEC_ERR_WORKSPACE (e.g. up to 512 requests of 64 nodes).  Each call
 * first clears the keys it uses (a kernel on `stream`, no memset), then
 * runs the accept.  Every call on one device
 * shares that device's array: calls that may overlap on one device
 * (different streams, or host threads without ordering) race.  The first
 * call on a device looks the array's address up with that device current
 * (SPEC_ERR_HIP if the lookup fails).
 */
int spec_accept_greedy_noalloc(int batch, int num_draft_tokens, int accept_width, int64_t vocab,
                               int dtype, const void *target_logits, const int32_t *candidates,
                               const int32_t *retrieve_index, const int32_t *retrieve_next_token,
                               const int32_t *retrieve_next_sibling, int32_t *predict,
                               int32_t *accept_index, int32_t *accept_length,
                               int32_t *target_predict, int32_t *dev_status,
                               spec_stream_t stream);

/*
 * Rejection-sampled tree accept.  [P4] 接受/拒绝 and [P2] 四 (Classic
 * Rejection Sampling); [P5] 5.6 (same walk, other test).
 *
 *   target_logits, draft_logits [batch*n, vocab] dtype; draft_logits NULL
 *       -> SPEC_ERR_NULL (no proposal distribution, [P1] 三条判定路径)
 *   temperature  [batch] f32 > 0, applied to both distributions
 *   uniforms     [batch, n] f32 in [0,1): uniforms[b][k] tests node k
 *   final_uniforms [batch] f32 in [0,1): the terminal draw
 * At node cur the residual R starts as softmax(target_logits[row(cur)]/T);
 * q = softmax(draft_logits[row(cur)]/T).  Children are tried in sibling
 * order; child c with token t is accepted iff uniforms[b][c] < min(1,
 * R(t)/q(t)).  A rejection sets R = max(0, R - q) / sum(max(0, R - q)) (left
 * unchanged, with SPEC_ST_ZERO_RESIDUAL, if that sum is 0).  With no child
 * accepted, or at a leaf, the terminal token is the smallest x whose
 * cumulative R (vocabulary order) exceeds final_uniforms[b] * sum(R).
 * Outputs as spec_accept_greedy.  Distribution statistics are fp32 sweeps
 * with fp64 reductions; a decision closer than ~1e-6 to its threshold may
 * differ from an exact evaluation.  Only the rows the walk visits are read.
 * workspace: spec_accept_workspace_size(batch, n, vocab, 1) bytes, 16-byte
 *   aligned and zero-filled before its first use; every call leaves it
 *   zero-filled again, so one workspace serves any number of calls in
 *   stream order (concurrent calls need one each).  After a call that
 *   raised SPEC_ST_SYNC, zero it again before the next call.
 */
int spec_accept_sample(int batch, int num_draft_tokens, int accept_width, int64_t vocab,
                       int dtype, const void *target_logits, const void *draft_logits,
                       const float *temperature, const float *uniforms,
                       const float *final_uniforms, const int32_t *candidates,
                       const int32_t *retrieve_index, const int32_t *retrieve_next_token,
                       const int32_t *retrieve_next_sibling, int32_t *predict,
                       int32_t *accept_index, int32_t *accept_length, void *workspace,
                       size_t workspace_bytes, int32_t *dev_status, spec_stream_t stream);

/*
 * Target-only tree accept.  [P2] 四 (Target-only Tree Sampling) with the
 * thresholds of [P1] 三条判定路径; [P5] 5.6 (same walk, other test).  No
 * draft distribution is used.
 *
 *   target_logits [batch*n, vocab] dtype
 *   temperature  [batch] f32 > 0
 *   threshold_single, threshold_acc  host floats, threshold_acc > 0 (else
 *       SPEC_ERR_SHAPE); 1 and 1 make the output law exactly p
 *   uniforms     [batch, n] f32 in [0,1): uniforms[b][k] is the coin of
 *       node k's children
 *   final_uniforms [batch] f32 in [0,1): the terminal draw
 * At node cur, p = softmax(target_logits[row(cur)] / T).  The children are
 * tried in sibling order, each adding p(token) to a running mass that
 * starts at 0; child c is accepted iff p(token) > 0 and (uniforms[b][cur] <
 * mass / threshold_acc or p(token) >= threshold_single), and the walk
 * continues from c with c's row and coin.  With no child accepted, or at a
 * leaf, the terminal token is the smallest x whose cumulative R (vocabulary
 * order) exceeds final_uniforms[b] * sum(R), R = p with the tokens of the
 * children rejected at that node set to 0 (SPEC_ST_ZERO_RESIDUAL and x =
 * vocab - 1 if sum(R) = 0).  Outputs as spec_accept_greedy.  Statistics are
 * fp32 exponentials with fp64 sums; a decision closer than ~1e-6 to its
 * threshold may differ from an exact evaluation.  Every verify row is read
 * once (per-row softmax statistics), plus the visited children's logits and
 * one 8192-entry chunk of the terminal row.
 * workspace: spec_accept_target_only_workspace_size(batch, n, vocab) bytes
 *   (16 bytes per verify row and 8192-entry chunk), 16-byte aligned and
 *   zero-filled before its first use; every call leaves it zero-filled
 *   again, so one workspace serves any number of calls in stream order
 *   (concurrent calls need one each).  After a call that raised
 *   SPEC_ST_SYNC, zero it again before the next call.
 */
size_t spec_accept_target_only_workspace_size(int batch, int num_draft_tokens, int64_t vocab);
int spec_accept_target_only(int batch, int num_draft_tokens, int accept_width, int64_t vocab,
                            int dtype, const void *target_logits, const float *temperature,
                            float threshold_single, float threshold_acc, const float *uniforms,
                            const float *final_uniforms, const int32_t *candidates,
                            const int32_t *retrieve_index, const int32_t *retrieve_next_token,
                            const int32_t *retrieve_next_sibling, int32_t *predict,
                            int32_t *accept_index, int32_t *accept_length, void *workspace,
                            size_t workspace_bytes, int32_t *dev_status, spec_stream_t stream);

/*
 * Draft step: one call of select_top_k_tokens for a batch.  [P1]
 * organize_draft_results:三张表的归约 (_select_top_k_tokens_first /
 * _select_top_k_tokens_later and the offsets organize_draft_results reads);
 * [P5] on the accumulated path score of the EAGLE-2 dynamic tree.
 *
 *   draft_logits [batch, rows, vocab] dtype: the draft model's logits of
 *       the live branches, rows = 1 at step 0 (the root), topk later
 *   branch_scores [batch, topk] f32: the live branches' path scores (the
 *       previous call's next_scores); ignored (may be NULL) at step 0
 * p = softmax(draft_logits row), rounded to f32.  Each row's top-topk
 * entries are ranked by (p descending, token id ascending).
 *   step 0: scores / tokens get the root's top-topk p and ids at offset 0;
 *       parents gets -1, 0, .., topk-1 at offset 0.
 *   step i >= 1: scores gets the f32 products branch_scores[j] * p_j[c]
 *       (topk*topk, branch-major) and tokens their ids, at offset
 *       topk + (i-1)*topk^2; the top-topk products (value descending, lower
 *       flat index first) give parents = flat index + topk^2*(i-1) + topk at
 *       offset topk + 1 + (i-1)*topk.
 *   The parent block of step num_steps-1 is not written (it is not part of
 *   the list; parents may be NULL then).  next_scores / next_tokens
 *   [batch, topk] get the kept scores and ids (step 0: the root's top-topk),
 *   the next call's branch_scores and input tokens; next_scores may be the
 *   same buffer as branch_scores.
 * Row layouts of scores / tokens [batch, topk + (num_steps-1)*topk^2] and
 * parents [batch, 1 + (num_steps-1)*topk] are those spec_build_tree reads;
 * entries of other steps are not touched.  Normalisers are sums of f32
 * exponentials in f64, so a p may differ from the exact f64 softmax by an
 * ulp and a ranking within ~1e-6 relative of a tie may differ from an
 * exact evaluation.  topk <= 8 (else SPEC_ERR_UNSUPPORTED), vocab >= topk
 * (else SPEC_ERR_SHAPE), rows * ceil(vocab / 8192) <= 2048 (vocab <=
 * 2097152 at a later step of topk 8; else SPEC_ERR_UNSUPPORTED).
 * workspace: spec_draft_step_workspace_size(batch, topk, vocab) bytes (80
 *   bytes per branch row and 2048-entry chunk), 8-byte aligned, any
 *   contents; calls in stream order may share one (concurrent calls need
 *   one each).  Two kernels are launched on `stream`.
 */
size_t spec_draft_step_workspace_size(int batch, int topk, int64_t vocab);
int spec_draft_step(int batch, int topk, int num_steps, int step, int64_t vocab, int dtype,
                    const void *draft_logits, const float *branch_scores, float *scores,
                    int32_t *tokens, int32_t *parents, float *next_scores,
                    int32_t *next_tokens, void *workspace, size_t workspace_bytes,
                    int32_t *dev_status, spec_stream_t stream);

/*
 * Accepted-KV compaction.  [P1] KV 回写 (move_accept_tokens_to_target_kvcache)
 * and [P2] 六: the verify rows in accept_index (root plus accepted drafts;
 * the terminal token has no KV yet) move to the request's sequence positions
 * L_b .. L_b + accept_length - 1.
 *
 *   k_pool, v_pool [num_layers, num_slots, num_kv_heads, head_dim] dtype,
 *       updated in place; every source row is read before any target row
 *       of the same request is written
 *   page_table [batch, max_pages], seq_lens [batch]: as verify attention
 *   out_cache_loc [batch*n] i32, accept_index [batch, accept_width] i32,
 *   accept_length [batch] i32: as produced by the accept calls
 * Outputs:
 *   new_seq_lens [batch] i32  seq_lens + accept_length
 *   free_slots   [batch*n] i32  request b's verify slots that are not a
 *                target slot, ascending node order, from b*n; padded with -1
 *   num_free     [batch] i32
 * Entries of accept_index that are -1 are skipped; rows, slots or pages out
 * of range raise SPEC_ST_RANGE and that row is not moved.  Requests must
 * own disjoint slots.  num_draft_tokens <= 64 (else SPEC_ERR_UNSUPPORTED),
 * accept_width <= 65.
 */
int spec_compact_kv(int batch, int num_draft_tokens, int accept_width, int num_layers,
                    int num_kv_heads, int head_dim, int page_size, int dtype, void *k_pool,
                    void *v_pool, int64_t num_slots, const int32_t *page_table, int max_pages,
                    const int32_t *seq_lens, const int32_t *out_cache_loc,
                    const int32_t *accept_index, const int32_t *accept_length,
                    int32_t *new_seq_lens, int32_t *free_slots, int32_t *num_free,
                    int32_t *dev_status, spec_stream_t stream);

/*
 * Sampling-parameter pre-pass: top-k / top-p filtering of the target
 * distribution.  [P2] 四 (eagle_sample: the target softmax at the request's
 * temperature, then top-k / top-p filtering and renormalisation) and [P1]
 * 三条判定路径.
 *
 *   logits [batch*n, vocab] dtype, finite or -inf (NaN is not defined);
 *       row i belongs to request i / n
 *   temperature [batch] f32 > 0; top_k [batch] i32 (< 1 or >= vocab: off);
 *   top_p [batch] f32 (>= 1: off; <= 0 keeps nothing)
 *   out [batch*n, vocab] dtype, may be the same buffer as logits
 * p = softmax(x / T) per row; entries rank by p descending, lower index
 * first; the entry of rank r is kept iff r < top_k and the mass of the
 * entries ranked above it is < top_p.  out holds the kept logits unchanged
 * and -inf elsewhere, so softmax(out / T) is the renormalised distribution
 * that spec_accept_sample / spec_accept_target_only then read with the same
 * temperature.  A greedy request in a sampled batch is top_k = 1.  A row of
 * -inf logits has no distribution: top_p does nothing there.  Masses
 * are float32 exponentials summed in float64: a top-p decision within ~1e-6
 * of top_p may differ from an exact evaluation.  vocab <= 2^31 - 1.
 * workspace: spec_sampling_filter_workspace_size(batch, n, vocab) bytes,
 *   16-byte aligned, any contents (NULL allowed when that size is 0: vocab
 *   <= 8192 or > 524288); calls in stream order may share one.  For 8192 <
 *   vocab <= 524288 three kernels are launched on `stream` (rows x chunks of
 *   <= 8192 entries, then one workgroup per row, then rows x chunks), else
 *   one workgroup per row.  A row with top_k in [1, 64] is finished from
 *   the chunks' top entries; others may be searched whole (slower).
 */
size_t spec_sampling_filter_workspace_size(int batch, int num_draft_tokens, int64_t vocab);
int spec_sampling_filter(int batch, int num_draft_tokens, int64_t vocab, int dtype,
                         const void *logits, const float *temperature, const int32_t *top_k,
                         const float *top_p, void *out, void *workspace, size_t workspace_bytes,
                         int32_t *dev_status, spec_stream_t stream);

/*
 * FULL tree mask.  [P1] 三种 mask 形态 (FULL_MASK) and the fill_prefix_mask
 * switch: every verify row sees the whole committed prefix and, among the
 * tree nodes, its QLEN_ONLY row.
 *
 *   seq_lens [batch] i32 committed lengths L_b, 0 <= L_b <= max_seq_len
 *   tree_mask_bits [batch*n] words of spec_mask_word_bytes(n) bytes: the
 *       SPEC_MASK_QLEN_BITS mask spec_build_tree writes (word-aligned)
 *   full_mask: u8 bytes, 16-byte aligned, full_mask_bytes of them; request
 *       b's block starts at n * sum_{b' < b} (L_b' + n) and holds n rows of
 *       L_b + n bytes: L_b prefix bytes (1), then byte j of the tree part =
 *       bit j of the row's word.  The caller sizes it n * sum_b (L_b + n).
 *   fill_prefix: nonzero writes every byte; zero writes only the tree
 *       bytes (the prefix bytes keep what the buffer held)
 * Writes past full_mask_bytes are dropped and raise SPEC_ST_RANGE, as does
 * L_b outside [0, max_seq_len] (bytes past max_seq_len + n of a row are
 * then not written).  n <= 64 (else SPEC_ERR_UNSUPPORTED).
 */
int spec_full_mask(int batch, int num_draft_tokens, const int32_t *seq_lens, int max_seq_len,
                   const void *tree_mask_bits, int fill_prefix, void *full_mask,
                   int64_t full_mask_bytes, int32_t *dev_status, spec_stream_t stream);

/*
 * Paged draft-branch planning.  [P1] prepare_for_draft (KV slots of the
 * draft writes) and duplicate_prefix_tail_to_draft_branches.
 *
 * Request b has L_b committed tokens; its prefix tail is the tail = L_b mod
 * page_size tokens on its last, partial page page_table[b][L_b div
 * page_size].
 *   topk > 1: branch j owns the pages branch_pages[b][j][0 .. pages_per_branch)
 *       (caller-allocated, distinct from the request's prefix pages), a
 *       page-aligned region whose slot t is page t div page_size, offset
 *       t mod page_size.  Its first `tail` slots receive a copy of the prefix
 *       tail's K and V (every layer), so whole-page reads of the branch see
 *       its tokens; draft step s of branch j writes region slot tail + s.
 *       pages_per_branch * page_size >= page_size - 1 + num_steps (else
 *       SPEC_ERR_SHAPE).
 *   topk == 1 (the contiguous case): the branch continues the prefix in
 *       place; step s writes the slot of position L_b + s through page_table
 *       (which must hold those pages); nothing is copied; branch_pages may
 *       be NULL.
 *   k_pool, v_pool [num_layers, num_slots, num_kv_heads, head_dim] dtype,
 *       updated in place (16-byte aligned; a row's bytes a multiple of 16,
 *       else SPEC_ERR_UNSUPPORTED); page ids lie in [0, num_slots / page_size);
 *       num_slots <= 2^31 - 1 (else SPEC_ERR_UNSUPPORTED)
 *   page_table [batch, max_pages] i32
 * Output: out_cache_loc [batch, topk, num_steps] i32, the slot draft step s
 * of branch j writes (-1 and SPEC_ST_RANGE where a page id is out of
 * range; such a copy is skipped).
 */
int spec_plan_draft_branches(int batch, int topk, int num_steps, int page_size, int num_layers,
                             int num_kv_heads, int head_dim, int dtype, void *k_pool,
                             void *v_pool, int64_t num_slots, const int32_t *seq_lens,
                             const int32_t *page_table, int max_pages,
                             const int32_t *branch_pages, int pages_per_branch,
                             int32_t *out_cache_loc, int32_t *dev_status, spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECMI_SPEC_H */
