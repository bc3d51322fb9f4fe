/*
 * ddtree.h -- C ABI of libddtree.so: the DDTree tree-verify hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The stages of one speculative verify step, in the order a caller runs them:
 *   ddtree_drafter_topk        per-depth top-k log-probs of the drafter's logits
 *   ddtree_build_tree          best-first draft tree from per-depth top-k log-probs
 *   ddtree_compile_visibility  ancestor-or-self bitsets (+ positions, + dense mask)
 *   ddtree_build_tree_visibility  (or) the two above in one call
 *   ddtree_verify_attn         absorbed-MLA attention of every tree node x head
 *                              over the shared prefix plus its own ancestors
 *   ddtree_verify_attn_layers  (or) the same over several layers in one launch
 *   ddtree_accept              greedy walk along the target argmax
 *   ddtree_tree_sample         (or) stochastic acceptance against the target distribution
 *   ddtree_commit_kv           the accepted path into the KV cache (after accept)
 *   ddtree_validate_inputs     (debug) checks the index arrays a step is built from
 *   ddtree_probe_mfma_loop, ddtree_device_info  (measurement) the device's sustained
 *                              matrix-core rate and its compute units and clock
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a DEVICE pointer owned by the caller (e.g. a
 *    torch tensor's storage).  The library never allocates, frees or
 *    synchronises; each call only enqueues kernels on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns.  No call reads
 *    device memory on the host, so all calls can be captured in a HIP graph.
 *  - Requests are packed ragged: request r owns tree nodes
 *    [qo_indptr[r], qo_indptr[r+1]); its q_len Q_r = budget_r + 1 (root +
 *    budget draft nodes).  Node indices inside a request are request-local
 *    (root = 0).  qo_indptr must be computed from the budgets -- never from
 *    the drafter block size, which misaligned every offset whenever
 *    budget + 1 != block_size ("The Mask Bug That Changed Everything: A
 *    Post-Mortem on DDTree Speculative Decoding", section "The Context: A
 *    Cascade of Infrastructure and Algorithm Challenges").
 *  - Host-known scalars (bs, max_q_len, max_budget, words_per_row, ...) size
 *    the launch; device data is trusted to agree with them.  Device data that
 *    disagrees never makes a kernel read or write out of bounds, but the
 *    affected outputs are unspecified (see each call).
 *  - Return value: DDTREE_OK, or a negative ddtree_status_t when the host
 *    arguments are invalid (nothing is enqueued then) or a launch failed.
 *    ddtree_last_error() gives a message for the calling thread.
 *    Asynchronous device faults surface at the caller's next synchronisation.
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDTREE_ABI_VERSION 1

typedef enum {
  DDTREE_OK = 0,
  DDTREE_EINVAL = -1,       /* invalid host argument                          */
  DDTREE_EUNSUPPORTED = -2, /* valid but outside what this build supports     */
  DDTREE_EWORKSPACE = -3,   /* workspace missing or smaller than required     */
  DDTREE_EHIP = -4          /* a HIP runtime call or kernel launch failed     */
} ddtree_status_t;

typedef enum { DDTREE_F32 = 0, DDTREE_BF16 = 1 } ddtree_dtype_t;

/* DDTREE_ABI_VERSION of the loaded library. */
int ddtree_abi_version(void);

/* Message for the calling thread's last non-OK return ("" if none). */
const char* ddtree_last_error(void);

/*
 * ddtree_build_tree -- best-first growth of each request's draft tree.
 *
 * Defined by "The DDTree CUDA Graph Fix: Unlocking Speculative Decoding at
 * 109 tok/s on PCIe Blackwell", section "The DDTree Architecture: Confirming
 * Multiple-Path Evaluation": the candidate with the highest cumulative
 * log-prob is taken and added to the tree, its best child and next-ranked
 * sibling become candidates, until budget draft nodes are in the tree.  The
 * root (node 0) is the last verified token ("The Oracle Drafter: Validating
 * a Custom DDTree Speculative Decoding Engine", section "The Engine
 * Interface Design").
 *
 *   topk_logprobs  [bs, depth_max, topk] f32: row d holds the top-k log-probs
 *                  of draft depth d+1, non-increasing, all <= 0.
 *   topk_ids       [bs, depth_max, topk] i32: matching token ids.
 *   root_tokens    [bs] i32.
 *   qo_indptr      [bs+1] i32: budget_r = qo_indptr[r+1] - qo_indptr[r] - 1.
 *   max_budget     host bound on every budget_r; must satisfy
 *                  max_budget <= sum_{d=1..depth_max} topk^d.
 *   Outputs, packed by qo_indptr: node_tokens, node_parents (root -1,
 *   otherwise a smaller request-local index), node_depths (root 0) as i32;
 *   node_scores f32 cumulative log-prob (root 0), nullable.
 *
 * Node order is pop order.  Scores are accumulated in fp32 root to leaf as
 * f32(parent_score + lp); ties in score go to the smaller depth, then to the
 * lexicographically smaller rank path.  Results are bit-exact.
 * Errors: EINVAL (null pointer, bs < 0, max_budget < 0, depth_max/topk < 1
 * with max_budget > 0, max_budget unreachable); EUNSUPPORTED when
 * depth_max * ceil(log2(topk)) > 64 (rank paths are packed in 64 bits),
 * max_budget > 2048, or depth_max * topk > 8192 (with max_budget > 0).
 * A request whose budget exceeds max_budget gets only max_budget draft nodes;
 * its remaining node slots are written as token -1, parent -1, depth -1.
 */
int ddtree_build_tree(const float* topk_logprobs, const int32_t* topk_ids,
                      const int32_t* root_tokens, const int32_t* qo_indptr, int bs,
                      int depth_max, int topk, int max_budget, int32_t* node_tokens,
                      int32_t* node_parents, int32_t* node_depths, float* node_scores,
                      void* stream);

/*
 * ddtree_compile_visibility -- ancestor-or-self bitsets of every tree node.
 *
 * Defined by "The DDTree CUDA Graph Fix ...", section "The DDTree
 * Architecture: Confirming Multiple-Path Evaluation" (each node attends only
 * to its ancestors plus the shared prefix), "The Architecture of a
 * Speculative Decoding Engine: Designing KV Cache Semantics for DDTree
 * Inference", section "The Final Resolution: A Concrete Trace" (the root
 * sits at position = cache length and sees itself; a depth-d node sits d
 * positions later), and "The 30-Column Mask: Debugging a Structural
 * Marshaling Mismatch in Custom MLA Verification Attention", section "Mask
 * Stride Formula" (the flattened mask is [q_len, prefix_len + q_len]
 * row-major, prefix columns first).
 *
 *   node_parents, node_depths  [total_q] i32 as written by ddtree_build_tree.
 *   qo_indptr [bs+1] i32, prefix_lens [bs] i32 (P_r >= 0).
 *   words_per_row  W >= ceil(max_q_len / 32).
 *   vis_bits   [total_q, W] u32: bit (j % 32) of word j / 32 is set iff node j
 *              of the same request is the row's node or one of its ancestors.
 *   positions  nullable [total_q] i64: P_r + depth.
 *   dense_mask nullable u8, with mask_indptr [bs+1] i64 (both or neither):
 *              request r's rows start at dense_mask + mask_indptr[r], row i is
 *              P_r ones followed by the row's Q_r visibility bits as bytes
 *              (stride P_r + Q_r).
 * Errors: EINVAL (null required pointer, bs < 0, max_q_len < 1 with bs > 0,
 * W too small, only one of dense_mask / mask_indptr given).  A parent that is
 * not a smaller index ends that row's ancestor walk.
 */
int ddtree_compile_visibility(const int32_t* node_parents, const int32_t* node_depths,
                              const int32_t* qo_indptr, const int32_t* prefix_lens, int bs,
                              int max_q_len, int words_per_row, uint32_t* vis_bits,
                              int64_t* positions, uint8_t* dense_mask,
                              const int64_t* mask_indptr, void* stream);

/*
 * ddtree_build_tree_visibility -- ddtree_build_tree followed by
 * ddtree_compile_visibility (bitsets and positions, no dense mask) in one
 * call: the same outputs, bit for bit, as the two calls in sequence.
 *
 * Both operations are defined where the two calls are.  For budgets up to
 * 64 with depth_max * topk <= 256 and max_q_len <= 128 it is one launch:
 * each node's ancestor-or-self bitset is its parent's bits plus its own,
 * formed as the node is taken (a parent is always taken before its child);
 * other sizes run the two calls' kernels back to back.
 *   Arguments: those of ddtree_build_tree, then prefix_lens, max_q_len,
 *   words_per_row, vis_bits and positions as for ddtree_compile_visibility
 *   (node_depths is always written; positions nullable, needs prefix_lens).
 * Errors: those of both calls.
 */
int ddtree_build_tree_visibility(const float* topk_logprobs, const int32_t* topk_ids,
                                 const int32_t* root_tokens, const int32_t* qo_indptr,
                                 const int32_t* prefix_lens, int bs, int depth_max, int topk,
                                 int max_budget, int max_q_len, int words_per_row,
                                 int32_t* node_tokens, int32_t* node_parents,
                                 int32_t* node_depths, float* node_scores, uint32_t* vis_bits,
                                 int64_t* positions, void* stream);

/*
 * ddtree_verify_attn_workspace_size -- bytes of device workspace that
 * ddtree_verify_attn needs for these sizes on the current device (0 if none).
 * The count depends on the current device's compute-unit count when
 * num_splits == 0.  Returns 0 for invalid sizes.
 */
size_t ddtree_verify_attn_workspace_size(int bs, int num_heads, int max_q_len, int max_kv_len,
                                         int num_splits, int dtype);

/*
 * ddtree_verify_attn -- tree-verify attention, absorbed MLA.
 *
 * Defined by "The Architecture of a Speculative Decoding Engine ...",
 * section "The Forward Pass Pseudocode" (attention of the absorbed query and
 * roped query part over the cached c_kv and k_pe under a mask, output in
 * latent space), "The 30-Column Mask ...", sections "The Message: Tensor
 * Shapes as Evidence" and "The Fix: Building Combined Indices" (576-wide
 * latent rows = 512 c_kv + 64 rope in a slot pool; each request's KV list is
 * its prefix slots followed by the slots of its tree nodes; the mask stride
 * is prefix_len + q_len) and "The DDTree CUDA Graph Fix ...", section "The
 * DDTree Architecture: Confirming Multiple-Path Evaluation" (all nodes in
 * one pass; the prefix is read once for all of them).
 *
 *   q          [total_q, H, 576] dtype: cols 0..511 absorbed q_nope, 512..575
 *              roped q_pe; rows node-major, head-minor.
 *   kv_pool    [num_slots, 576] dtype: cols 0..511 c_kv, 512..575 k_pe.
 *   kv_indptr  [bs+1] i32 and kv_indices i32: request r's logical columns
 *              c = 0 .. N_r-1 (N_r = kv_indptr[r+1] - kv_indptr[r]) read pool
 *              row kv_indices[kv_indptr[r] + c].  The first P_r = N_r - Q_r
 *              are prefix slots, the last Q_r the tree nodes' own slots in
 *              node order.
 *   qo_indptr  [bs+1] i32; vis_bits [total_q, words_per_row] u32 as written
 *              by ddtree_compile_visibility.
 *   max_q_len  >= every Q_r; max_kv_len >= every N_r (host bounds).
 *   scale      softmax scale on the full 576-d dot product.
 *   out        [total_q, H, 512] dtype: sum over visible columns of
 *              softmax(scale * q . kv) * c_kv.
 *   lse        nullable [total_q, H] f32: natural-log log-sum-exp of the
 *              scaled scores.
 *   num_splits 0 = automatic (bf16: persistent work split evenly over the
 *              device's compute units, partial results merged by log-sum-exp;
 *              bf16 calls too small to fill the device that way -- at most
 *              4 units of 128 rows x 32 KV columns per compute unit by the
 *              host bounds -- take 32-row tiles with each tile's KV range cut
 *              into a fixed number of parts, see ddtree_verify_attn_plan;
 *              f32: no split); S >= 1 = each 128-row tile's KV range cut
 *              into S equal parts, then merged.  The result does not depend
 *              on the split beyond rounding.
 *   workspace  device scratch of at least ddtree_verify_attn_workspace_size()
 *              bytes (may be NULL when that is 0).
 * Arithmetic: bf16 inputs use bf16 matrix cores with fp32 accumulation, the
 * softmax weights rounded to bf16 for the value product, output rounded to
 * bf16; a split tile's partial results pass to the merge as O / l in fp16
 * (scaled per row and 128 features by a power of two into fp16's range, so
 * any finite c_kv is handled) with m and l in fp32; f32 inputs compute in fp32 throughout, on a vector-ALU kernel meant
 * for small batches and for checking the bf16 path: each of its query rows
 * reads its request's KV rows itself, so its time grows as H * Q * N (any
 * size is accepted and correct).
 * Errors: EINVAL (null required pointer, bs < 0, num_heads < 1, max_q_len < 1,
 * max_kv_len < max_q_len, words_per_row too small, non-finite scale,
 * num_slots < 1, num_splits < 0, bad dtype); EWORKSPACE.  A pool index
 * outside [0, num_slots) is clamped into range (a valid row is read); a
 * request with N_r < Q_r is skipped (its outputs are left untouched).
 */
int ddtree_verify_attn(const void* q, const void* kv_pool, int64_t num_slots,
                       const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* qo_indptr, const uint32_t* vis_bits, int words_per_row,
                       int bs, int num_heads, int max_q_len, int max_kv_len, float scale,
                       int dtype, void* out, float* lse, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * ddtree_verify_attn_plan -- the kernel and split that ddtree_verify_attn
 * (and, per layer, ddtree_verify_attn_layers) uses for these host bounds on
 * the current device, for tests and measurement.
 *   tile_rows  out: query rows per tile -- 128 (bf16 matrix-core kernel,
 *              persistent schedule or forced splits), 32 (bf16 kernel for
 *              calls too small to fill the device; see num_splits above) or
 *              4 (f32 kernel).
 *   splits     out: KV parts per tile; 0 for the persistent schedule.
 * Errors: EINVAL (null output, sizes or dtype invalid as for
 * ddtree_verify_attn); EHIP (the device's compute units cannot be read).
 */
int ddtree_verify_attn_plan(int bs, int num_heads, int max_q_len, int max_kv_len,
                            int num_splits, int dtype, int* tile_rows, int* splits);

/*
 * ddtree_verify_attn_layers -- ddtree_verify_attn over L layers in one
 * launch, sharing the step's slot lists, visibility and work schedule.
 *
 * The slot positions of a step do not change from layer to layer, only the
 * latents stored in them do, so the combined index list is built once per
 * step and serves every layer ("The 30-Column Mask ...", sections "The Fix:
 * Building Combined Indices" and "Layer-Invariant Slot Optimization").  Layer l reads q + l * q_layer_stride
 * and kv_pool + l * kv_layer_stride and writes out + l * out_layer_stride
 * and lse + l * lse_layer_stride (strides in elements of each array; a zero
 * input stride shares one array across layers); every other argument and
 * the result of each layer are exactly those of ddtree_verify_attn.  Layer
 * outputs must not overlap: with num_layers > 1, out_layer_stride (and
 * lse_layer_stride when lse is given) must be nonzero (EINVAL otherwise).  Small layers share one launch; a layer whose
 * work alone fills the device (bf16, automatic split, at least 64 KV blocks
 * of 32 columns per compute unit by the host bounds) gets a launch of its
 * own, still enqueued by this one call.  Useful where the queries of several layers are
 * at hand together; within one forward pass layer l + 1's queries need
 * layer l's output.
 *   workspace  ddtree_verify_attn_layers_workspace_size() bytes: one
 *              single-layer workspace per layer.
 * Errors: those of ddtree_verify_attn, and EINVAL for num_layers outside
 * [1, 65535] or a negative stride.
 */
size_t ddtree_verify_attn_layers_workspace_size(int num_layers, int bs, int num_heads,
                                                int max_q_len, int max_kv_len, int num_splits,
                                                int dtype);
int ddtree_verify_attn_layers(int num_layers, const void* q, int64_t q_layer_stride,
                              const void* kv_pool, int64_t kv_layer_stride, int64_t num_slots,
                              const int32_t* kv_indptr, const int32_t* kv_indices,
                              const int32_t* qo_indptr, const uint32_t* vis_bits,
                              int words_per_row, int bs, int num_heads, int max_q_len,
                              int max_kv_len, float scale, int dtype, void* out,
                              int64_t out_layer_stride, float* lse, int64_t lse_layer_stride,
                              int num_splits, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * ddtree_accept -- greedy acceptance along the target argmax.
 *
 * Defined by "The DDTree CUDA Graph Fix ...", section "The DDTree
 * Architecture: Confirming Multiple-Path Evaluation" (walk from the root,
 * stepping to the child whose token equals the target's argmax at the
 * current node, until none matches; the longest chain plus one bonus token),
 * "The Oracle Drafter ...", section "The Engine Interface Design" (outputs:
 * accepted path, accept length, proposed tokens, bonus) and "The
 * Architecture of a Speculative Decoding Engine ...", section "The Final
 * Resolution: A Concrete Trace" (the accepted nodes, root included, are
 * committed; autoregressive decoding is the budget-0 case, accept length 1).
 *
 *   node_tokens, node_parents [total_q] i32; qo_indptr [bs+1] i32;
 *   target_predict [total_q] i32: target argmax at every node.
 *   depth_max  D: the walk stops after D + 1 path nodes.
 *   accepted_nodes [bs, D+1] i32: request-local path, root first, -1 padded.
 *   accept_len     [bs] i32 in 1..D+1 (counts the root).
 *   commit_tokens  [bs, D+1] i32: the accepted draft tokens then the bonus
 *                  (accept_len tokens), -1 padded.
 *   bonus_tokens   [bs] i32: target argmax at the last accepted node.
 * If two children of one node carry the same token the smaller index wins.
 * Errors: EINVAL (null pointer, bs < 0, depth_max < 0), EUNSUPPORTED
 * (depth_max > 4096).  A request with
 * Q_r < 1 gets accept_len 0 and all -1 rows.
 */
int ddtree_accept(const int32_t* node_tokens, const int32_t* node_parents,
                  const int32_t* qo_indptr, const int32_t* target_predict, int bs, int depth_max,
                  int32_t* accepted_nodes, int32_t* accept_len, int32_t* commit_tokens,
                  int32_t* bonus_tokens, void* stream);

/*
 * ddtree_tree_sample -- stochastic (temperature) acceptance along the tree,
 * the sampling counterpart of ddtree_accept.
 *
 * Defined by "The DDTree CUDA Graph Fix ...", section "Temperature Support:
 * Already Working for Linear, Planned for DDTree" (tree-structured
 * rejection sampling against the target's filtered distribution at every
 * node, the draft being the tree's tokens).  Rule (speculative sampling for
 * a draft with all its mass on its token): at node cur the residual starts
 * as the target row, mass R; children are tried in node order; child c with
 * token t is accepted iff coins[c] * R < res[t], otherwise R -= res[t] and
 * res[t] = 0; the walk stops when no child is accepted or after
 * depth_max + 1 nodes; the bonus is the first token whose running residual
 * mass (vocabulary order) exceeds bonus_uniforms[r] times the residual's
 * mass at the last node.  Computed in fp32; decisions agree with exact
 * arithmetic except within the fp32 rounding of the sums, about
 * (ceil(vocab / 256) + 256 + nodes) * 2^-24 of the row's mass (each sum
 * runs over 256 contiguous blocks of ceil(vocab / 256) tokens, the tokens
 * of a block one by one, then the blocks one by one, so a call's result
 * does not depend on timing).  A token without mass is never accepted or
 * drawn; if rounding leaves the threshold unreached, the residual's last
 * token with mass is drawn.
 *
 *   node_tokens, node_parents [total_q] i32; qo_indptr [bs+1] i32.
 *   target_probs [total_q, vocab] f32: non-negative (temperature, top-k and
 *                top-p already applied by the caller; rows need not sum to 1).
 *   coins [total_q] f32 in [0, 1): the coin of node c, used when c is tried.
 *   bonus_uniforms [bs] f32 in [0, 1).
 *   total_q      rows of target_probs (= qo_indptr[bs]); sizes the launch.
 *   outputs as ddtree_accept: accepted_nodes [bs, D+1] (-1 padded),
 *   accept_len [bs], commit_tokens [bs, D+1] (accepted drafts then the
 *   bonus), bonus_tokens [bs] (-1 if the residual has no mass).
 *   workspace    device scratch of ddtree_tree_sample_workspace_size(total_q)
 *                bytes (the block masses of every row); contents on entry
 *                are ignored.
 * Errors: EINVAL (null pointer, bs < 0, total_q < 0, depth_max < 0,
 * vocab < 1), EUNSUPPORTED (vocab > 2^21), EWORKSPACE.  A request is walked
 * over its first 4096 nodes; a node with more than 1024 children keeps only
 * its first 1024 rejections.  Tokens outside [0, vocab) are never accepted.
 */
size_t ddtree_tree_sample_workspace_size(int total_q);
int ddtree_tree_sample(const int32_t* node_tokens, const int32_t* node_parents,
                       const int32_t* qo_indptr, const float* target_probs, const float* coins,
                       const float* bonus_uniforms, int bs, int total_q, int depth_max, int vocab,
                       int32_t* accepted_nodes, int32_t* accept_len, int32_t* commit_tokens,
                       int32_t* bonus_tokens, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * ddtree_tree_sample_noalloc -- ddtree_tree_sample without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments (less the workspace), same kernels and same results as
 * ddtree_tree_sample.  Its scratch (the block masses of every row) is a
 * static device array of the library, 8 MiB, holding up to 4096 tree nodes:
 * each GPU the call runs on keeps its own copy until the process ends.  The
 * call allocates nothing (its first call on a device looks the array's
 * address up once).  Calls that overlap on one GPU share that array and
 * race: serialise them (one stream, or events).
 * Errors: those of ddtree_tree_sample (no EWORKSPACE), EUNSUPPORTED for
 * total_q > 4096, EHIP if the array's address cannot be found.
 */
int ddtree_tree_sample_noalloc(const int32_t* node_tokens, const int32_t* node_parents,
                               const int32_t* qo_indptr, const float* target_probs,
                               const float* coins, const float* bonus_uniforms, int bs,
                               int total_q, int depth_max, int vocab, int32_t* accepted_nodes,
                               int32_t* accept_len, int32_t* commit_tokens,
                               int32_t* bonus_tokens, void* stream);

/*
 * ddtree_commit_kv -- the accepted path enters each request's KV cache.
 *
 * Defined by "The Architecture of a Speculative Decoding Engine ...",
 * sections "The First Attempt: Temporary Buffers and Post-Verify Compaction"
 * (the tree nodes' latents are appended after the prefix for verification;
 * afterwards the accepted ones are gathered from their scattered places into
 * contiguous positions), "The Off-by-One Labyrinth" (the bonus token is not
 * cached) and "The Final Resolution: A Concrete Trace" (the accepted nodes,
 * root included, are committed: the cache grows by accept_len).
 *
 *   kv_indptr [bs+1], kv_indices: request r's slot list, its P_r prefix slots
 *                then the slots of its Q_r tree nodes in node order (the
 *                ddtree_verify_attn layout).
 *   qo_indptr [bs+1]; accepted_nodes [bs, depth_max+1] and accept_len [bs]
 *                as ddtree_accept writes them (path root first).
 *   max_kv_len   >= every request's slot-list length (sizes the launch).
 *   new_kv_indptr [bs+1] i32 out: new_kv_indptr[0] = 0, request r's new list
 *                has P_r + accept_len_r entries.
 *   new_kv_indices [new_kv_capacity] i32 out: request r's new list = its
 *                prefix slots, then
 *                  index form (kv_pool NULL): the slots of the path's nodes
 *                    in path order -- no latent moves;
 *                  move form (kv_pool given): its first accept_len node slots,
 *                    after the latent row of the path's i-th node has been
 *                    copied into the i-th node slot (rows read before they
 *                    are overwritten: the compaction the page describes).
 *                Either way the new list reads the prefix latents, then the
 *                accepted nodes' latents in path order.  Entries past
 *                new_kv_capacity are not written; the old total
 *                kv_indptr[bs] - kv_indptr[0] always suffices.  Must not
 *                overlap kv_indices.
 *   kv_pool      nullable [num_slots, 576] rows of dtype (DDTREE_BF16 or
 *                DDTREE_F32), modified in place by the move form.
 * Errors: EINVAL (null required pointer, bs < 0, depth_max < 0,
 * max_kv_len < 1, new_kv_capacity < 0, bad dtype or num_slots with a pool),
 * EUNSUPPORTED (max_kv_len above 65535 * 8192).  Device data that disagrees
 * is clamped (accept_len to [0, min(Q_r, depth_max+1)], node ids to the
 * request, slots to the pool); the affected outputs are unspecified.
 */
int ddtree_commit_kv(const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* qo_indptr, const int32_t* accepted_nodes,
                     const int32_t* accept_len, int bs, int depth_max, int max_kv_len,
                     int32_t* new_kv_indptr, int32_t* new_kv_indices, long long new_kv_capacity,
                     void* kv_pool, long long num_slots, int dtype, void* stream);

/*
 * ddtree_drafter_topk -- per-depth top-k log-probabilities of the drafter's
 * logits (the input of ddtree_build_tree).
 *
 * Defined by "The DDTree CUDA Graph Fix ...", section "The DDTree
 * Architecture: Confirming Multiple-Path Evaluation" (from each depth
 * position's hidden state the vocabulary head yields the top-k candidate
 * tokens with their log-probabilities).  Reading: the log-probability is the
 * log-softmax over the whole vocabulary; the top k are the k largest in
 * descending order, equal values in ascending token id.
 *
 *   logits   [rows, vocab] of dtype (DDTREE_F32 or DDTREE_BF16), row-major;
 *            rows = bs * depth_max for a batch of drafts.  Finite or -inf,
 *            with at least one finite logit per row (a row of only -inf
 *            has no distribution; its outputs are unspecified).  Long -inf
 *            runs, e.g. a masked vocabulary tail, are fine.
 *   topk_logprobs [rows, topk] f32 out; topk_ids [rows, topk] i32 out
 *            (exactly the layout ddtree_build_tree reads).
 *   workspace of ddtree_drafter_topk_workspace_size(rows, vocab, topk)
 *            bytes (per-chunk statistics and candidates), caller-owned.
 * Computed in fp32 (hardware exp and log); the order is decided on the
 * logits themselves.  Errors: EINVAL (null pointer, rows < 0, bad dtype,
 * topk outside [1, vocab]), EUNSUPPORTED (topk > 32, or more than 1024 chunk
 * candidates: ceil(vocab / 8192) * topk > 1024), EWORKSPACE.
 */
size_t ddtree_drafter_topk_workspace_size(int rows, int vocab, int topk);
int ddtree_drafter_topk(const void* logits, int dtype, int rows, int vocab, int topk,
                        float* topk_logprobs, int32_t* topk_ids, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * ddtree_validate_inputs -- debug check of the index arrays of a verify step
 * (not needed on the hot path: the other calls trust device data).
 *
 * Looks for the marshalling mistakes "The 30-Column Mask ..." describes in
 * sections "The Fix: Building Combined Indices" and "Mistakes and Incorrect
 * Assumptions" (a KV index list holding only the prefix slots while the
 * mask expects prefix + tree columns; offsets that do not line up; slot ids
 * outside the pool) and offsets taken from the wrong length ("The Mask Bug
 * That Changed Everything ...", section "The Context: A Cascade of
 * Infrastructure and Algorithm Challenges").
 *
 *   qo_indptr [bs+1], kv_indptr [bs+1], kv_indices [num_kv_indices] i32, as
 *   for ddtree_verify_attn; total_q = the length of the node arrays;
 *   num_slots = the pool's rows.
 *   prefix_lens  nullable [bs] i32: when given, every request must have
 *                exactly P_r + Q_r KV columns.
 *   node_parents nullable [total_q] i32: when given, each request's node 0
 *                must have parent -1 and every other node c a parent in
 *                [0, c).
 *   report [2 * DDTREE_NUM_CHECKS] i32, device, written by the call: for
 *   check k, report[2k] = number of violations and report[2k+1] = the
 *   smallest offending index (-1 if none).  Checks, in order:
 *     0 QO_INDPTR  request r with qo[r] < 0, qo[r+1] < qo[r] or qo[r+1] > total_q
 *     1 KV_INDPTR  request r with kv[r] < 0, kv[r+1] < kv[r] or kv[r+1] > num_kv_indices
 *     2 KV_LEN     request r with N_r < Q_r, or N_r != P_r + Q_r (prefix_lens given)
 *     3 KV_INDEX   position j of kv_indices with a slot outside [0, num_slots)
 *     4 PARENT     node index (into the node arrays) with a bad parent
 * Every read stays inside the sizes given, whatever the arrays hold.  The
 * report is ready when the stream reaches it (the caller synchronises).
 * Errors: EINVAL (null report, negative size, null indptr with bs > 0, null
 * kv_indices with num_kv_indices > 0), EUNSUPPORTED (bs > 65534).
 */
#define DDTREE_NUM_CHECKS 5
int ddtree_validate_inputs(int bs, const int32_t* qo_indptr, int total_q,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t num_kv_indices, int64_t num_slots, const int32_t* prefix_lens,
                           const int32_t* node_parents, int32_t* report, void* stream);

/*
 * Measurement probes (not a stage of the method).  A roofline fraction is a
 * measured rate over a published peak; these give the device's own side of
 * that ratio.
 *
 * ddtree_probe_mfma_loop -- grid workgroups of 256 threads; each wave runs
 * iters rounds of 8 independent v_mfma_f32_32x32x16_bf16 (32768 flops each)
 * and writes one float per thread to out [grid * 256] (the accumulators'
 * sum, so the loop is not removed).  Flops per launch =
 * grid * 4 * iters * 8 * 32768.  Errors: EINVAL (grid < 1, iters < 1, null
 * out).
 *
 * ddtree_device_info -- the current device's compute-unit count and peak
 * shader clock in kHz, as the runtime reports them.  Errors: EINVAL (null
 * pointer), EHIP (no device or the query failed).
 */
int ddtree_probe_mfma_loop(int grid, int iters, float* out, void* stream);
int ddtree_device_info(int* compute_units, int* peak_clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */
