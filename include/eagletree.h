/*
 * eagletree.h -- C ABI of libeagletree: the data-parallel core of EAGLE-2
 * dynamic draft trees on one AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (the pages this library follows):
 *   [P1] "EAGLE-2: Faster Inference of Language Models with Dynamic Draft
 *        Trees", summary page (paperlayer.ai, arXiv 2406.16858v2):
 *        s2.1 speculative sampling, s4.1 expansion phase, s4.2 reranking
 *        phase, App. A implementation details.
 *   [P2] "EAGLE-2: Dynamic Draft Trees" explainer (stable-lab specdec
 *        notes): the path-product value equation, expand/rerank, and the
 *        "Common misconception" chain example.
 *   [P3] EAGLE notes (garden.houmin.site/infra/eagle), section "EAGLE 2 /
 *        方法": Expand stage (threshold stop) and ReRank stage (shallower
 *        node wins ties).
 *   [P4] EAGLE-3 review (xllm-io paper-review), section 五: all reported
 *        speedups are at temperature 0 (greedy decoding).
 *
 * One decode cycle of a batch of B independent sequences is:
 *     et_draft_step(step = 1 .. D)   -- expand the tree layer by layer
 *     et_rerank                      -- keep the global top-N nodes
 *     et_tree_mask                   -- flatten: ancestor mask, depth, pos
 *     et_tree_attention              -- tree-masked attention (verify)
 *     et_accept                      -- greedy longest accepted path
 *       (or et_accept_sample           -- ratio tests at temperature > 0)
 *     et_kv_commit                   -- append the accepted path's K/V
 * Fused forms with the same outputs: et_rerank_mask (rerank and mask in
 * one launch) and et_draft_step_last (the last draft step, whose merge
 * also reranks and flattens the tree).
 * A fixed-shape baseline replaces the first two with et_draft_step_static
 * x D and et_static_tree (after et_set_static_shape).
 * Between draft steps the caller runs its draft model on `next_tokens`
 * and hands the resulting vocab logits to the next step.
 *
 * Conventions
 *   - Every pointer argument named as device memory must be a device
 *     pointer (e.g. torch.empty(..., device="cuda").data_ptr()).  The
 *     library never allocates or frees device memory on these calls; the
 *     caller owns every buffer, including the workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = legacy default
 *     stream).  All calls are asynchronous and stream-ordered; none of them
 *     synchronises the host.  Host-side argument validation happens before
 *     any launch; on failure nothing is launched.
 *   - Return value: ET_OK (0) or a negative et_status; et_last_error()
 *     gives a message for the calling thread.
 *   - Device-side preconditions (not checked, documented instead): logits
 *     are finite or -inf with at least one finite entry per row; no NaN;
 *     n_kept / parent_slot / tokens are the values written by et_rerank.
 *   - Debug mode: with the environment variable ET_DEBUG set (not "0")
 *     when a plan is created, every call of that plan copies the tree and
 *     prefix-length inputs it reads to the host and checks them (as
 *     et_check_tree / et_check_prefix) before launching, returning
 *     ET_EINVAL with a message and launching nothing on a violation; then
 *     it synchronises the stream, so a failure on the device is reported
 *     (ET_EHIP) by the call that caused it, and checks the tree or
 *     frontier it wrote.  Slow: for debugging only.
 *   - T = N + 1 tree slots per sequence: slot 0 is the root (the last
 *     committed token), slots 1..n hold the kept draft tokens, slots
 *     n+1..N are padding.  W = ceil(T / 64) mask words per slot.
 *   - A plan + workspace pair carries the tree from et_draft_step(1)
 *     through et_rerank of the same cycle; use one workspace per stream
 *     that runs cycles concurrently.
 */
#ifndef EAGLETREE_H
#define EAGLETREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ET_OK = 0,
  ET_EINVAL = -1,        /* null pointer, shape, stride or range error      */
  ET_EUNSUPPORTED = -2,  /* dtype, head_dim, top-k or size outside support  */
  ET_ESTATE = -3,        /* calls out of order for this plan and workspace  */
  ET_EHIP = -4           /* a HIP launch or runtime call failed             */
} et_status;

typedef enum { ET_F32 = 0, ET_BF16 = 1 } et_dtype;

typedef void* et_stream_t;              /* a hipStream_t                    */
typedef struct et_plan_s* et_plan_t;    /* opaque, host-side metadata only  */

/* Shapes of one cycle.  Limits (ET_EUNSUPPORTED / ET_EINVAL otherwise):
 *   1 <= batch <= 65535; 2 <= vocab <= 2^18; 1 <= topk <= 16;
 *   1 <= depth <= 15; 1 <= budget_n <= 255 (so T <= 256, W <= 4);
 *   expand_threshold >= 0 (0 disables the stop rule);
 *   head_dim in {64, 128}; n_q_heads % n_kv_heads == 0;
 *   1 <= n_kv_heads, n_q_heads / n_kv_heads <= 16; prefix_cap >= 1.
 * topk is both the number of children drawn per expanded node and the
 * number of nodes expanded per layer ([P1] s4.1: the k most valuable
 * nodes of the current layer are expanded; [P3] Expand stage: each node
 * contributes its top 2 children when k = 2). */
typedef struct {
  int32_t batch;            /* B independent sequences                     */
  int32_t vocab;            /* V                                           */
  int32_t topk;             /* k                                           */
  int32_t depth;            /* D draft layers below the root               */
  int32_t budget_n;         /* N draft tokens kept by the rerank           */
  float expand_threshold;   /* nodes whose value is below it are not
                               expanded ([P3] Expand stage)                */
  int32_t logits_dtype;     /* et_dtype of draft and target logits         */
  int32_t n_q_heads;        /* Hq                                          */
  int32_t n_kv_heads;       /* Hkv (grouped-query attention, G = Hq/Hkv)   */
  int32_t head_dim;         /* d                                           */
  int32_t prefix_cap;       /* P_cap: allocated prefix length of the cache */
  int32_t qkv_dtype;        /* et_dtype of q, K/V cache, tree K/V and out  */
} et_config;

/* Validate `cfg` and create a plan (host memory only).  *out receives the
 * plan on success. */
int et_plan_create(const et_config* cfg, et_plan_t* out);
int et_plan_destroy(et_plan_t plan);

/* Bytes of device workspace the plan needs (256-byte aligned base
 * required).  The workspace holds the candidate pool, the frontier,
 * per-chunk partial results of the vocab scans and the attention split
 * partials. */
size_t et_workspace_bytes(et_plan_t plan);

/* Pool capacity per sequence: topk + (depth - 1) * topk^2 nodes. */
int32_t et_pool_capacity(et_plan_t plan);

/* Bind a freshly allocated workspace to the plan: checks its alignment
 * (256 bytes) and resets the plan's record of the call order.  Must run
 * once after the workspace is allocated and before its first use.  No
 * device memory needs clearing (every call writes what it later reads),
 * so nothing is launched on `stream`. */
int et_workspace_init(et_plan_t plan, void* ws, et_stream_t stream);

/* One expansion layer ([P1] s4.1; [P2] value equation; [P3] Expand).
 *
 * step 1 starts a new tree: the root of sequence b is root_tokens[b]
 * (device int32 [B]) with value 1; its single frontier row is row 0.
 * For step s in 1..D, frontier slot j of sequence b (j < frontier count
 * F_b, in the order of the previous call's next_tokens) reads the vocab
 * logits row at
 *     logits + b * batch_stride + j * row_stride      (elements)
 * (dtype = logits_dtype).  At steps s >= 2 all topk rows j < topk of every
 * sequence must be readable memory, whatever F_b: they are loaded before
 * F_b is known, and rows j >= F_b are then ignored (they may hold any
 * bits).  Step 1 reads row 0 only.  For each row the
 * call computes the full-vocab softmax at temperature 1, takes the topk
 * largest logits (ties: lower token id first) as children, with
 *     conf  = softmax probability of the child token,
 *     value = value(parent) * conf          (one fp32 multiply),
 * appends them to the sequence's candidate pool, and -- if s < D --
 * selects the next frontier: the topk children of this layer with the
 * largest value (ties: lower token id, then creation order), minus those
 * whose value < expand_threshold.  next_tokens (device int32 [B][topk])
 * receives the frontier's tokens in frontier order, padded with -1, and
 * next_count (device int32 [B]) its size (0 at s = D or once the tree
 * stopped).  Row alignment: 16-byte aligned rows take the vector path.
 * Errors: ET_EINVAL (null pointer, step outside 1..D, stride < vocab or
 * negative), ET_ESTATE (step != 1 and not the step after the last call on
 * this plan and workspace). */
int et_draft_step(et_plan_t plan, void* ws, int32_t step,
                  const int32_t* root_tokens, const void* logits,
                  int64_t batch_stride, int64_t row_stride,
                  int32_t* next_tokens, int32_t* next_count,
                  et_stream_t stream);

/* Rerank ([P1] s4.2; [P2] expand/rerank; [P3] ReRank stage).
 * Keeps the n = min(N, pool size) pool nodes with the largest value, with
 * ties broken by shallower depth, then lower token id, then creation
 * order, and flattens them in that rank order behind the root:
 *   tokens      device int32 [B][T]  slot 0 = root token, pads = -1
 *   parent_slot device int32 [B][T]  slot 0 = -1, pads = -1
 *   conf, value device f32   [B][T]  slot 0 = 1, pads = 0
 *   n_kept      device int32 [B]     n
 * Rank order is topological (a parent always ranks before its child), so
 * parent_slot[s] < s.  Requires et_draft_step(D) as the last call on this
 * plan and workspace (ET_ESTATE otherwise). */
int et_rerank(et_plan_t plan, void* ws, int32_t* tokens, int32_t* parent_slot,
              float* conf, float* value, int32_t* n_kept, et_stream_t stream);

/* Flatten ([P1] s4.2: the kept tokens become one sequence whose attention
 * mask keeps branches apart): for slot s <= n_kept[b]
 *   mask[b][s][w]  bit t of word w (t = 64 w + bit) is set iff slot t is
 *                  slot s or one of its ancestors; device uint64 [B][T][W]
 *   depth[b][s]    0 for the root, depth(parent) + 1 otherwise
 *   pos_ids[b][s]  prefix_len[b] + depth[b][s]
 * Pad slots get mask 0, depth -1, pos_ids -1.  prefix_len: device int32
 * [B] with 0 <= prefix_len[b] <= prefix_cap (not checked on device). */
int et_tree_mask(et_plan_t plan, const int32_t* parent_slot,
                 const int32_t* n_kept, const int32_t* prefix_len,
                 uint64_t* mask, int32_t* depth, int32_t* pos_ids,
                 et_stream_t stream);

/* Rerank and flatten in one launch ([P1] s4.2: rerank, then the flattened
 * sequence and its mask): writes every output of et_rerank and of
 * et_tree_mask, with the same values and layouts as that pair of calls
 * (et_tree_mask applied to the rerank's parent_slot and n_kept).  The
 * parent walk reads the parent slots from on-chip memory, so neither the
 * second launch nor a reread of parent_slot is needed.  Requirements and
 * errors are those of et_rerank, plus the prefix_len range of
 * et_tree_mask (checked in debug mode). */
int et_rerank_mask(et_plan_t plan, void* ws, int32_t* tokens, int32_t* parent_slot,
                   float* conf, float* value, int32_t* n_kept,
                   const int32_t* prefix_len, uint64_t* mask, int32_t* depth,
                   int32_t* pos_ids, et_stream_t stream);

/* The last draft step, reranked and flattened in its own launches ([P1]
 * s4.1 then s4.2): et_draft_step(D) (same arguments, same pool and
 * frontier outputs: the frontier of the last step is empty) whose merge
 * then writes every output of et_rerank_mask for the finished tree, with
 * the same values.  One launch fewer per cycle than et_draft_step(D)
 * followed by et_rerank_mask: the rerank runs in the merge's block, on the
 * step's children still in on-chip memory and the earlier nodes loaded
 * with the merge's inputs.  Requirements and errors are those of
 * et_draft_step at step D and of et_rerank_mask; ET_EUNSUPPORTED if the
 * pool capacity exceeds 256 nodes per draft row (no valid configuration
 * does). */
int et_draft_step_last(et_plan_t plan, void* ws, const int32_t* root_tokens,
                       const void* logits, int64_t batch_stride, int64_t row_stride,
                       int32_t* next_tokens, int32_t* next_count,
                       const int32_t* prefix_len, int32_t* tokens, int32_t* parent_slot,
                       float* conf, float* value, int32_t* n_kept, uint64_t* mask,
                       int32_t* depth, int32_t* pos_ids, et_stream_t stream);

/* Tree attention, the verify pass ([P1] s4.2; [P2]: the tree is checked
 * in one tree-attention pass; [P3]: Medusa-style tree attention).
 * For sequence b, query head h (kv head h / G) and slot s <= n_kept[b]:
 *     scores over the prefix keys k_cache[b][h/G][0 .. prefix_len[b]) and
 *     the tree keys k_tree[b][h/G][t] for every t with bit t of
 *     mask[b][s] set; p = softmax(scale * q . k); out = sum p * v.
 * Layouts (dtype = qkv_dtype, contiguous, row-major):
 *     q, out           [B][T][Hq][d]
 *     k_cache, v_cache [B][Hkv][prefix_cap][d]
 *     k_tree, v_tree   [B][Hkv][T][d]
 * Pad slots (s > n_kept[b]) get out = 0.  bf16 inputs are multiplied on
 * the matrix cores with fp32 accumulation; softmax runs in fp32. */
int et_tree_attention(et_plan_t plan, void* ws, const void* q,
                      const void* k_cache, const void* v_cache,
                      const void* k_tree, const void* v_tree,
                      const int32_t* prefix_len, const uint64_t* mask,
                      const int32_t* n_kept, float scale, void* out,
                      et_stream_t stream);

/* Greedy acceptance at temperature 0 ([P1] s2.1: tokens are accepted in
 * order along the draft; [P4] s五: greedy decoding).  Target row s of
 * sequence b is at target_logits + b * batch_stride + s * row_stride
 * (dtype = logits_dtype), for s = 0 .. n_kept[b].  All T rows s = 0 .. N
 * must be readable memory: they are loaded before n_kept[b] is known, and
 * rows past n_kept[b] are then ignored (any bits).  With a_s = argmax of
 * row s (ties: lowest id), the walk starts at slot 0 and moves to the
 * child c of the current slot whose token equals a_current, while one
 * exists.  Outputs (device int32):
 *   accept_len [B]        number of accepted draft tokens L
 *   path_slots [B][D+1]   0, then the accepted slots; -1 after L + 1
 *   out_tokens [B][D+1]   the L accepted tokens, then the bonus token
 *                         a_(last accepted slot); -1 after L + 1 */
int et_accept(et_plan_t plan, void* ws, const void* target_logits,
              int64_t batch_stride, int64_t row_stride,
              const int32_t* tokens, const int32_t* parent_slot,
              const int32_t* n_kept, int32_t* accept_len,
              int32_t* path_slots, int32_t* out_tokens, et_stream_t stream);

/* et_accept without a workspace, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the per-(row, chunk, wave) argmax keys that et_accept keeps
 * in the workspace go to a fixed device array of the library instead,
 * ET_ACCEPT_NOALLOC_SCRATCH bytes per device, held from the first call on
 * that device until the process ends.  A call needs
 *     batch * T * ceil(vocab / chunk) * 4 * 8 bytes
 * (chunk = 16384 ids for bf16 logits, 8192 for fp32); a plan needing more
 * is rejected with ET_EINVAL before anything is launched.  The call uses
 * the array of the current device (the stream must belong to it).  Every
 * call on one device shares that array: calls that overlap on one device
 * (several streams or threads) race and must not be issued; calls on one
 * stream are ordered.  No other state is kept between calls.  Arguments,
 * outputs and other errors as et_accept; it allocates nothing (no
 * hipMalloc, no hipFree). */
#define ET_ACCEPT_NOALLOC_SCRATCH (4u << 20)
int et_accept_noalloc(et_plan_t plan, const void* target_logits,
                      int64_t batch_stride, int64_t row_stride,
                      const int32_t* tokens, const int32_t* parent_slot,
                      const int32_t* n_kept, int32_t* accept_len,
                      int32_t* path_slots, int32_t* out_tokens,
                      et_stream_t stream);

/* Stochastic acceptance at temperature > 0 ([P1] s2.1: draft tokens are
 * accepted one after another by the ratio of target to draft probability;
 * [P1] s2.2: the tree lets the siblings of a rejected token be tried;
 * [P1] s1: the output keeps the target model's distribution).  The pages
 * give the chain rule only; the tree form used here: a node's children
 * are its top-k, chosen rather than sampled, so each is a point-mass
 * proposal.  With p = softmax(target row of the current slot /
 * temperature), the children of the current slot are tried in slot order
 * (highest value first); child c is accepted iff
 *     uniforms[b][c] * R < p(tokens[c]),
 * R being the target mass not yet rejected at this slot (1 before the
 * first try, minus p of each rejected sibling); the walk moves to the
 * accepted child.  When every child is rejected (or there is none, or
 * the walk reached depth D), the bonus token is drawn from the residual
 * (p without the rejected tokens) by inverse CDF in id order with
 * uniforms[b][0]: the first id whose running residual mass exceeds
 * uniforms[b][0] * R.  Every decision compares fp32-computed masses
 * (fp64 sums), so a run whose u lies within about 1e-6 of a decision
 * boundary may go either way; otherwise the result is the exact rule.
 * Inputs as et_accept (all T rows readable; rows past n_kept ignored;
 * every kept row has a finite maximum), plus:
 *   temperature  finite and > 0, with log2(e) / temperature a finite float
 *   uniforms     device fp32 [B][T], each in [0, 1); entry s is used when
 *                slot s is tried (at most once per call), entry 0 for the
 *                bonus
 * Outputs as et_accept; the bonus is never a rejected child's token.
 * Shares the accept region of the workspace with et_accept. */
int et_accept_sample(et_plan_t plan, void* ws, const void* target_logits,
                     int64_t batch_stride, int64_t row_stride,
                     const int32_t* tokens, const int32_t* parent_slot,
                     const int32_t* n_kept, float temperature,
                     const float* uniforms, int32_t* accept_len,
                     int32_t* path_slots, int32_t* out_tokens,
                     et_stream_t stream);

/* Draft step from the draft model's final hidden states: the LM head
 * (EAGLE notes, method section: the draft model reuses the target's LM
 * head) fused with the step, so the logits never reach HBM.  For row j < F
 * of sequence b,
 *     logits[v] = sum_h hidden[b][j][h] * lm_head[v][h]
 * on the matrix cores (bf16 inputs, fp32 sums in an unspecified order),
 * then exactly et_draft_step on those fp32 logits (children, conf, value,
 * next frontier; it is a dynamic-policy step and may be mixed with
 * et_draft_step steps of the same cycle).
 *   hidden     device bf16, row j of sequence b at hidden + b * batch_stride
 *              + j * row_stride (elements, multiples of 8, 16-byte aligned
 *              base); all topk rows of every sequence must be readable
 *              (rows j >= F are loaded and ignored)
 *   lm_head    device bf16 [vocab][hidden_dim], row-major, 16-byte aligned
 *   hidden_dim a multiple of 128, 128 .. 65536
 * ET_EUNSUPPORTED for another hidden_dim; other errors as et_draft_step. */
int et_draft_step_hidden(et_plan_t plan, void* ws, int32_t step,
                         const int32_t* root_tokens, const void* hidden,
                         int64_t batch_stride, int64_t row_stride,
                         const void* lm_head, int32_t hidden_dim,
                         int32_t* next_tokens, int32_t* next_count,
                         et_stream_t stream);

/* Static (fixed-shape) tree: the baseline the dynamic tree is compared
 * with ([P2] "Watch the Budget Being Spent": an EAGLE-1-style fixed shape
 * spends the same node budget on every context; [P3] EAGLE: one static
 * prior tree for every input).  Readout of either tree: the sum of the
 * kept values, the expected number of accepted tokens ([P2] value
 * equation).
 *
 * et_set_static_shape stores a shape in the plan (host only, no device
 * work): slot s = 1 .. n_nodes has parent slot parent[s - 1] (0 = root,
 * earlier slots only) and child rank rank[s - 1] in 0 .. topk - 1
 * (distinct among siblings), depth <= depth, n_nodes <= budget_n, and at
 * most topk slots of one depth have children.  ET_EINVAL otherwise (the
 * plan keeps its previous shape).
 *
 * et_draft_step_static is et_draft_step with the next frontier taken from
 * the shape instead of by value (no threshold): at step l the rows belong,
 * in slot order, to the shape's slots of depth l - 1 that have children;
 * each row's top-k children, conf and value are formed as in
 * et_draft_step.  Same arguments, layouts and call order (steps 1..D on
 * one workspace, all of the same policy); ET_ESTATE without a shape.
 *
 * et_static_tree (after step D of et_draft_step_static) writes the shape's
 * slots in the layout of et_rerank: slot 0 the root (conf = value = 1),
 * slot s the kept child, parent_slot from the shape; n_kept[b] = n_nodes;
 * pad slots token -1, parent -1, conf 0, value 0.  The result feeds
 * et_tree_mask, et_tree_attention and the accept calls unchanged. */
int et_set_static_shape(et_plan_t plan, const int32_t* parent,
                        const int32_t* rank, int32_t n_nodes);
int et_draft_step_static(et_plan_t plan, void* ws, int32_t step,
                         const int32_t* root_tokens, const void* logits,
                         int64_t batch_stride, int64_t row_stride,
                         int32_t* next_tokens, int32_t* next_count,
                         et_stream_t stream);
int et_static_tree(et_plan_t plan, void* ws, int32_t* tokens,
                   int32_t* parent_slot, float* conf, float* value,
                   int32_t* n_kept, et_stream_t stream);

/* Commit the verified path to the KV cache (the step after acceptance:
 * [P1] s2.1, the accepted tokens extend the sequence in path order; the
 * one verify pass, [P1] s4.2, computed K/V for every tree slot).  The
 * root (slot 0, the first token not yet in the cache) and the accepted
 * slots path_slots[b][1..L], L = accept_len[b], in path order, are
 * appended to the prefix cache: for every kv head, row i of the path goes
 * to cache position prefix_len[b] + i, copied bit for bit from k_tree /
 * v_tree; then prefix_len[b] += L + 1.
 * Layouts (dtype = qkv_dtype): k_cache, v_cache [B][Hkv][prefix_cap][d]
 * (in/out), k_tree, v_tree [B][Hkv][T][d], prefix_len [B] int32 (in/out),
 * path_slots [B][D+1] and accept_len [B] int32 as written by et_accept.
 * Device precondition: prefix_len[b] + accept_len[b] + 1 <= prefix_cap;
 * rows that would pass prefix_cap are not written and prefix_len[b] stops
 * at prefix_cap.  No workspace.  Errors: ET_EINVAL (null pointer, K/V
 * buffer not 16-byte aligned). */
int et_kv_commit(et_plan_t plan, void* k_cache, void* v_cache,
                 const void* k_tree, const void* v_tree, int32_t* prefix_len,
                 const int32_t* path_slots, const int32_t* accept_len,
                 et_stream_t stream);

/* Inspection: copy the workspace's candidate pool (after any draft step)
 * into caller device buffers, for tests and debugging.  Pool arrays are
 * [B][capacity] (capacity = et_pool_capacity); entries past
 * pool_count[b] are unspecified.  parent is the pool index of the
 * parent, -1 for the root.  frontier ([B][topk], pool indices) and
 * frontier_count ([B]) describe the frontier the next draft step reads.
 * Any output pointer may be NULL to skip it. */
int et_pool_export(et_plan_t plan, const void* ws, int32_t* token,
                   int32_t* parent, int32_t* depth, float* conf, float* value,
                   int32_t* pool_count, int32_t* frontier,
                   int32_t* frontier_count, et_stream_t stream);

/* Host-side checks of the device data the calls expect (what ET_DEBUG
 * runs on copies of device buffers), on HOST arrays:
 *   et_check_tree    tokens (may be NULL: not checked), parent_slot
 *                    [B][T] and n_kept [B] in the layout of et_rerank:
 *                    0 <= n_kept[b] <= N; slot 0 has parent -1; a kept slot
 *                    s <= n_kept[b] has a token in [0, vocab) and a parent
 *                    slot in [0, s) (the flattened order is topological);
 *                    pad slots have token -1 and parent -1
 *   et_check_prefix  0 <= prefix_len[b] <= prefix_cap
 * ET_OK, or ET_EINVAL with the first violation in et_last_error().
 * et_plan_debug returns 1 if the plan was created in debug mode. */
int et_check_tree(et_plan_t plan, const int32_t* tokens,
                  const int32_t* parent_slot, const int32_t* n_kept);
int et_check_prefix(et_plan_t plan, const int32_t* prefix_len);
int et_plan_debug(et_plan_t plan);

/* Message of the last failed call on this thread ("" if none). */
const char* et_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EAGLETREE_H */
