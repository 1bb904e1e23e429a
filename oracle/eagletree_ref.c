/*
 * eagletree_ref.c -- CPU oracle for the EAGLE-2 draft-tree cycle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library; the product
 * path (libeagletree) never does, and the two share no code.
 *
 * Plain loops, no intrinsics, fp64 wherever the method computes real
 * numbers; the only fp32 steps are those the method defines on fp32 data
 * (conf and value are stored as fp32; value is one fp32 multiply per
 * edge, root to leaf).  Sources:
 *   [P1] EAGLE-2 summary page (paperlayer.ai, arXiv 2406.16858v2),
 *        s2.1, s4.1 (expansion), s4.2 (reranking), App. A.
 *   [P2] "EAGLE-2: Dynamic Draft Trees" explainer: value equation
 *        (Value(v) = product of c_u over the root-to-v path),
 *        expand/rerank paragraph, "Common misconception" chain example.
 *   [P3] EAGLE notes, "EAGLE 2 / 方法": Expand stage (threshold stop),
 *        ReRank stage (keep the N most probable nodes, shallower wins
 *        ties).
 *   [P4] EAGLE-3 review, s五: temperature 0 = greedy decoding.
 * Readings where the pages are silent are listed at each function.
 *
 * State layout (owned by the caller, all arrays row-major per sequence):
 *   pool_token/parent/depth  int32 [B][cap]   parent = pool index, -1 = root
 *   pool_conf/value          f32   [B][cap]
 *   pool_count, root_token   int32 [B]
 *   frontier                 int32 [B][k]     pool indices (-1 = root)
 *   frontier_count           int32 [B]
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define REF_F32 0
#define REF_BF16 1

/* Read element i of a logits/qkv buffer exactly as a double.  bf16 is the
 * top half of an IEEE fp32 word, so widening is exact. */
static double ref_load(const void* base, int dtype, int64_t i) {
  if (dtype == REF_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------
 * Row softmax statistics ([P1] s4.1: the draft model's confidence of a
 * token stands in for its acceptance rate; [P2] "Confidence ~
 * Acceptance").  Reading: confidence is the full-vocabulary softmax at
 * temperature 1, no top-p, no renormalisation over the top-k.
 * Returns m = max x and s = sum exp(x - m), both fp64.
 * ------------------------------------------------------------------- */
static void ref_row_softmax(const void* row, int dtype, int V, double* m_out,
                            double* s_out) {
  double m = -INFINITY;
  for (int v = 0; v < V; ++v) {
    double x = ref_load(row, dtype, v);
    if (x > m) m = x;
  }
  double s = 0.0;
  for (int v = 0; v < V; ++v) s += exp(ref_load(row, dtype, v) - m);
  *m_out = m;
  *s_out = s;
}

/* Top-k of one row: k rounds, each taking the largest logit not yet taken
 * (a strict > over ascending ids keeps the lower id on equal logits).
 * Reading: children are ordered by exact logit, lower id first on ties. */
static void ref_row_topk(const void* row, int dtype, int V, int k,
                         int32_t* ids, double* xs, unsigned char* taken) {
  memset(taken, 0, (size_t)V);
  for (int r = 0; r < k; ++r) {
    int best = -1;
    double bx = 0.0;
    for (int v = 0; v < V; ++v) {
      if (taken[v]) continue;
      double x = ref_load(row, dtype, v);
      if (best < 0 || x > bx) {
        best = v;
        bx = x;
      }
    }
    taken[best] = 1;
    ids[r] = best;
    xs[r] = bx;
  }
}

/* Total order on pool nodes ([P3] ReRank: larger value first, the
 * shallower node on equal values; then lower token id, then creation
 * order -- the last two make the order total).  Returns <0 if node a
 * ranks before node b. */
typedef struct {
  const float* value;
  const int32_t* depth;
  const int32_t* token;
} ref_pool_view;
static ref_pool_view g_view; /* qsort has no context argument */

static int ref_rank_cmp(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  float va = g_view.value[a], vb = g_view.value[b];
  if (va != vb) return va > vb ? -1 : 1;
  if (g_view.depth[a] != g_view.depth[b])
    return g_view.depth[a] < g_view.depth[b] ? -1 : 1;
  if (g_view.token[a] != g_view.token[b])
    return g_view.token[a] < g_view.token[b] ? -1 : 1;
  return a < b ? -1 : (a > b);
}

/* ---------------------------------------------------------------------
 * One expansion layer, step = 1..D ([P1] s4.1; [P2] value equation and
 * expand paragraph; [P3] Expand stage).
 *   step 1: root = root_tokens[b], value 1, frontier = [root], pool empty.
 *   For frontier slot j (frontier order = order of the logits rows): read
 *   row j, take its top-k tokens as children with
 *       conf  = (float) exp(x_id - m) / s          (fp64, then rounded)
 *       value = (float) value(parent) * conf        (one fp32 multiply)
 *   appended in (frontier slot, child rank) order.
 *   If step < D the next frontier is the first k children of this layer
 *   in rank order (ref_rank_cmp), keeping only value >= threshold
 *   (reading of [P3]: a node is not expanded when its value is strictly
 *   below the threshold; 0 disables the rule; the root is always
 *   expanded).  next_tokens[b][j] = token of frontier node j (-1 pads).
 * ------------------------------------------------------------------- */
int etref_draft_step(int B, int V, int k, int D, float thr, int dtype,
                     int step, const int32_t* root_tokens, const void* logits,
                     int64_t bstride, int64_t rstride, int cap,
                     int32_t* pool_token, int32_t* pool_parent,
                     int32_t* pool_depth, float* pool_conf, float* pool_value,
                     int32_t* pool_count, int32_t* root_token,
                     int32_t* frontier, int32_t* frontier_count,
                     int32_t* next_tokens, int32_t* next_count) {
  if (step < 1 || step > D || k < 1 || V < k) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)V);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* xs = (double*)malloc(sizeof(double) * (size_t)k);
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k * k + 1));
  if (!taken || !ids || !xs || !order) return -2;

  for (int b = 0; b < B; ++b) {
    int32_t* ptok = pool_token + (int64_t)b * cap;
    int32_t* ppar = pool_parent + (int64_t)b * cap;
    int32_t* pdep = pool_depth + (int64_t)b * cap;
    float* pconf = pool_conf + (int64_t)b * cap;
    float* pval = pool_value + (int64_t)b * cap;
    int32_t* fr = frontier + (int64_t)b * k;
    if (step == 1) {
      pool_count[b] = 0;
      root_token[b] = root_tokens[b];
      fr[0] = -1;
      frontier_count[b] = 1;
    }
    int F = frontier_count[b];
    int layer_start = pool_count[b];
    for (int j = 0; j < F; ++j) {
      const char* row = (const char*)logits +
                        (b * bstride + j * rstride) * (dtype == REF_F32 ? 4 : 2);
      double m, s;
      ref_row_softmax(row, dtype, V, &m, &s);
      ref_row_topk(row, dtype, V, k, ids, xs, taken);
      int32_t par = fr[j];
      float vpar = par < 0 ? 1.0f : pval[par];
      for (int r = 0; r < k; ++r) {
        int idx = pool_count[b]++;
        if (idx >= cap) return -3;
        float conf = (float)(exp(xs[r] - m) / s);
        ptok[idx] = ids[r];
        ppar[idx] = par;
        pdep[idx] = step;
        pconf[idx] = conf;
        pval[idx] = vpar * conf;
      }
    }
    int nf = 0;
    if (step < D && F > 0) {
      int n_layer = pool_count[b] - layer_start;
      for (int i = 0; i < n_layer; ++i) order[i] = layer_start + i;
      g_view.value = pval;
      g_view.depth = pdep;
      g_view.token = ptok;
      qsort(order, (size_t)n_layer, sizeof(int32_t), ref_rank_cmp);
      for (int i = 0; i < n_layer && i < k; ++i) {
        if (thr > 0.0f && pval[order[i]] < thr) continue;
        fr[nf++] = order[i];
      }
    }
    frontier_count[b] = nf;
    next_count[b] = nf;
    for (int j = 0; j < k; ++j)
      next_tokens[(int64_t)b * k + j] = j < nf ? ptok[fr[j]] : -1;
  }
  free(taken);
  free(ids);
  free(xs);
  free(order);
  return 0;
}

/* ---------------------------------------------------------------------
 * Rerank ([P1] s4.2: all draft tokens are reranked and the top ones by
 * value are verified; [P2]: ancestors always outscore a node, so the kept
 * set is a connected tree; [P3] ReRank stage: shallower node wins ties).
 * Sort the whole pool by ref_rank_cmp, keep n = min(N, pool size), flatten
 * in rank order behind the root (slot 0).  Reading: rank order is the
 * flatten order; it is topological since a parent ranks before its child.
 * Returns -4 if a kept node's parent is not kept earlier (cannot happen
 * when conf <= 1; reported rather than assumed).
 * ------------------------------------------------------------------- */
int etref_rerank(int B, int k, int D, int N, int cap,
                 const int32_t* pool_token, const int32_t* pool_parent,
                 const int32_t* pool_depth, const float* pool_conf,
                 const float* pool_value, const int32_t* pool_count,
                 const int32_t* root_token, int32_t* tokens,
                 int32_t* parent_slot, float* conf, float* value,
                 int32_t* n_kept) {
  (void)k;
  (void)D;
  int T = N + 1;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  int32_t* slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)cap);
  if (!order || !slot_of) return -2;
  int rc = 0;
  for (int b = 0; b < B; ++b) {
    const int32_t* ptok = pool_token + (int64_t)b * cap;
    const int32_t* ppar = pool_parent + (int64_t)b * cap;
    const int32_t* pdep = pool_depth + (int64_t)b * cap;
    const float* pconf = pool_conf + (int64_t)b * cap;
    const float* pval = pool_value + (int64_t)b * cap;
    int P = pool_count[b];
    for (int i = 0; i < P; ++i) {
      order[i] = i;
      slot_of[i] = -1;
    }
    g_view.value = pval;
    g_view.depth = pdep;
    g_view.token = ptok;
    qsort(order, (size_t)P, sizeof(int32_t), ref_rank_cmp);
    int n = P < N ? P : N;
    int32_t* tk = tokens + (int64_t)b * T;
    int32_t* ps = parent_slot + (int64_t)b * T;
    float* cf = conf + (int64_t)b * T;
    float* vl = value + (int64_t)b * T;
    tk[0] = root_token[b];
    ps[0] = -1;
    cf[0] = 1.0f;
    vl[0] = 1.0f;
    for (int s = 1; s <= n; ++s) {
      int idx = order[s - 1];
      slot_of[idx] = s;
      int par = ppar[idx];
      int pslot = par < 0 ? 0 : slot_of[par];
      if (pslot < 0 || pslot >= s) rc = -4;
      tk[s] = ptok[idx];
      ps[s] = pslot;
      cf[s] = pconf[idx];
      vl[s] = pval[idx];
    }
    for (int s = n + 1; s < T; ++s) {
      tk[s] = -1;
      ps[s] = -1;
      cf[s] = 0.0f;
      vl[s] = 0.0f;
    }
    n_kept[b] = n;
  }
  free(order);
  free(slot_of);
  return rc;
}

/* ---------------------------------------------------------------------
 * Tree mask ([P1] s4.2: the kept tokens are flattened into one sequence
 * with an attention mask that keeps branches apart).  Reading: a slot
 * sees itself and its ancestors (and, in attention, the whole prefix).
 *   anc[0] = {0};  anc[s] = anc[parent_slot[s]] + {s}
 *   depth[0] = 0;  depth[s] = depth[parent_slot[s]] + 1
 *   pos[s] = prefix_len[b] + depth[s]   (reading: the standard position
 *            id of a token at that depth after the prefix)
 * Bit t of the mask row lives in word t / 64, bit t % 64.  Pad slots get
 * mask 0, depth -1, pos -1.  Requires parent_slot[s] < s.
 * ------------------------------------------------------------------- */
int etref_tree_mask(int B, int N, const int32_t* parent_slot,
                    const int32_t* n_kept, const int32_t* prefix_len,
                    uint64_t* mask, int32_t* depth, int32_t* pos) {
  int T = N + 1, W = (T + 63) / 64;
  for (int b = 0; b < B; ++b) {
    const int32_t* ps = parent_slot + (int64_t)b * T;
    uint64_t* mk = mask + (int64_t)b * T * W;
    int32_t* dp = depth + (int64_t)b * T;
    int32_t* po = pos + (int64_t)b * T;
    int n = n_kept[b];
    for (int s = 0; s < T; ++s) {
      for (int w = 0; w < W; ++w) mk[(int64_t)s * W + w] = 0;
      if (s > n) {
        dp[s] = -1;
        po[s] = -1;
        continue;
      }
      if (s == 0) {
        dp[0] = 0;
      } else {
        int p = ps[s];
        if (p < 0 || p >= s) return -4;
        for (int w = 0; w < W; ++w)
          mk[(int64_t)s * W + w] = mk[(int64_t)p * W + w];
        dp[s] = dp[p] + 1;
      }
      mk[(int64_t)s * W + s / 64] |= (uint64_t)1 << (s % 64);
      po[s] = prefix_len[b] + dp[s];
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------
 * Tree attention for one (sequence b, slot s, query head h) ([P2]: the
 * chosen tree is verified in a single tree-attention pass; [P3]: Medusa
 * style tree attention).  Reading: scaled dot-product attention with
 * scale given, kv head = h / (Hq / Hkv), over every prefix key p <
 * prefix_len[b] and every tree slot t whose mask bit is set in row s;
 * softmax and the weighted sum in fp64 on the exact input values.  Q/K
 * are taken as already position-encoded.  Writes d doubles to out.
 * ------------------------------------------------------------------- */
void etref_attention_row(int B, int T, int Hq, int Hkv, int dh, int Pcap,
                         int dtype, const void* q, const void* kc,
                         const void* vc, const void* kt, const void* vt,
                         const int32_t* prefix_len, const uint64_t* mask,
                         const int32_t* n_kept, double scale, int b, int s,
                         int h, double* out) {
  (void)B;
  int W = (T + 63) / 64, G = Hq / Hkv, kvh = h / G;
  for (int i = 0; i < dh; ++i) out[i] = 0.0;
  if (s > n_kept[b]) return;
  int P = prefix_len[b];
  int64_t qoff = (((int64_t)b * T + s) * Hq + h) * dh;
  int64_t coff = ((int64_t)b * Hkv + kvh) * Pcap * dh;
  int64_t toff = ((int64_t)b * Hkv + kvh) * T * dh;
  const uint64_t* mrow = mask + ((int64_t)b * T + s) * W;
  int nkeys = P + T;
  double* sc = (double*)malloc(sizeof(double) * (size_t)nkeys);
  char* use = (char*)malloc((size_t)nkeys);
  double mx = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    int is_tree = j >= P;
    int t = j - P;
    use[j] = is_tree ? (int)((mrow[t / 64] >> (t % 64)) & 1u) : 1;
    if (!use[j]) continue;
    double dot = 0.0;
    for (int i = 0; i < dh; ++i) {
      double kv = is_tree ? ref_load(kt, dtype, toff + (int64_t)t * dh + i)
                          : ref_load(kc, dtype, coff + (int64_t)j * dh + i);
      dot += ref_load(q, dtype, qoff + i) * kv;
    }
    sc[j] = dot * scale;
    if (sc[j] > mx) mx = sc[j];
  }
  double den = 0.0;
  for (int j = 0; j < nkeys; ++j)
    if (use[j]) {
      sc[j] = exp(sc[j] - mx);
      den += sc[j];
    }
  for (int j = 0; j < nkeys; ++j) {
    if (!use[j]) continue;
    int is_tree = j >= P;
    int t = j - P;
    double p = sc[j] / den;
    for (int i = 0; i < dh; ++i) {
      double vv = is_tree ? ref_load(vt, dtype, toff + (int64_t)t * dh + i)
                          : ref_load(vc, dtype, coff + (int64_t)j * dh + i);
      out[i] += p * vv;
    }
  }
  free(sc);
  free(use);
}

/* All rows: out is fp64 [B][T][Hq][d].  Independent (b, h) units may run
 * on several threads when built with OpenMP; each unit is the same plain
 * loop as above. */
void etref_tree_attention(int B, int T, int Hq, int Hkv, int dh, int Pcap,
                          int dtype, const void* q, const void* kc,
                          const void* vc, const void* kt, const void* vt,
                          const int32_t* prefix_len, const uint64_t* mask,
                          const int32_t* n_kept, double scale, double* out) {
  int64_t units = (int64_t)B * Hq;
#pragma omp parallel for schedule(dynamic)
  for (int64_t u = 0; u < units; ++u) {
    int b = (int)(u / Hq), h = (int)(u % Hq);
    for (int s = 0; s < T; ++s)
      etref_attention_row(B, T, Hq, Hkv, dh, Pcap, dtype, q, kc, vc, kt, vt,
                          prefix_len, mask, n_kept, scale, b, s, h,
                          out + (((int64_t)b * T + s) * Hq + h) * dh);
  }
}

/* ---------------------------------------------------------------------
 * Greedy acceptance ([P1] s2.1: draft tokens are accepted in order and
 * the first rejection ends the run; [P4] s五: greedy decoding, T = 0).
 * a_s = argmax of target row s (lowest id on ties).  From slot 0, move to
 * the child c of the current slot with tokens[c] == a_current while one
 * exists (siblings carry distinct tokens, so it is unique).  The bonus
 * token is a_(last accepted slot).  Reading: accept_len counts draft
 * tokens only; the bonus is the extra entry in out_tokens.
 * ------------------------------------------------------------------- */
int etref_accept(int B, int T, int V, int D, int dtype, const void* target,
                 int64_t bstride, int64_t rstride, const int32_t* tokens,
                 const int32_t* parent_slot, const int32_t* n_kept,
                 int32_t* accept_len, int32_t* path_slots,
                 int32_t* out_tokens) {
  int32_t* amax = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  if (!amax) return -2;
  for (int b = 0; b < B; ++b) {
    int n = n_kept[b];
    const int32_t* tk = tokens + (int64_t)b * T;
    const int32_t* ps = parent_slot + (int64_t)b * T;
    for (int s = 0; s <= n; ++s) {
      const char* row = (const char*)target +
                        (b * bstride + s * rstride) * (dtype == REF_F32 ? 4 : 2);
      int best = 0;
      double bx = ref_load(row, dtype, 0);
      for (int v = 1; v < V; ++v) {
        double x = ref_load(row, dtype, v);
        if (x > bx) {
          bx = x;
          best = v;
        }
      }
      amax[s] = best;
    }
    int32_t* pth = path_slots + (int64_t)b * (D + 1);
    int32_t* ot = out_tokens + (int64_t)b * (D + 1);
    for (int i = 0; i <= D; ++i) {
      pth[i] = -1;
      ot[i] = -1;
    }
    int cur = 0, len = 0;
    pth[0] = 0;
    for (;;) {
      int next = -1;
      for (int c = 1; c <= n; ++c)
        if (ps[c] == cur && tk[c] == amax[cur]) {
          next = c;
          break;
        }
      if (next < 0 || len >= D) break;
      ot[len] = tk[next];
      ++len;
      pth[len] = next;
      cur = next;
    }
    ot[len] = amax[cur];
    accept_len[b] = len;
  }
  free(amax);
  return 0;
}

/* -------------------------------------------------------------------
 * Commit the verified path to the KV cache: the step after acceptance.
 * [P1] s2.1: the accepted draft tokens extend the sequence in path order;
 * [P1] s4.2: the one verify pass computed K/V for every tree slot.
 * Readings: the root (slot 0) is the first token not yet in the cache, so
 * the committed tokens are slot 0 and the accepted slots path[1..L]; for
 * every kv head they become cache positions P_b .. P_b + L, row i being
 * the K (and V) row of path[i]; P_b becomes P_b + L + 1.  Rows that would
 * pass prefix_cap are dropped and P_b stops at prefix_cap.  Rows are
 * copied as raw elements of esz bytes (2 for bf16, 4 for fp32).
 * ------------------------------------------------------------------- */
void etref_kv_commit(int B, int T, int Hkv, int dh, int Pcap, int D, int esz,
                     void* k_cache, void* v_cache, const void* k_tree,
                     const void* v_tree, int32_t* prefix_len,
                     const int32_t* path_slots, const int32_t* accept_len) {
  const size_t row = (size_t)dh * (size_t)esz;
  for (int b = 0; b < B; ++b) {
    const int P = prefix_len[b];
    const int L = accept_len[b];
    int rows = L + 1;
    if (P + rows > Pcap) rows = Pcap - P;
    if (rows < 0) rows = 0;
    for (int h = 0; h < Hkv; ++h) {
      for (int i = 0; i < rows; ++i) {
        const int slot = path_slots[(int64_t)b * (D + 1) + i];
        const size_t src = (((size_t)b * Hkv + h) * T + slot) * row;
        const size_t dst = (((size_t)b * Hkv + h) * Pcap + P + i) * row;
        memcpy((char*)k_cache + dst, (const char*)k_tree + src, row);
        memcpy((char*)v_cache + dst, (const char*)v_tree + src, row);
      }
    }
    prefix_len[b] = P + rows;
  }
}

/* ---------------------------------------------------------------------
 * Stochastic acceptance at temperature tau > 0 ([P1] s2.1: draft tokens
 * are accepted one after another by the ratio of target to draft
 * probability; [P1] s2.2: on a rejection the tree lets a sibling branch be
 * tried; [P1] s1: the output distribution stays the target's).
 * Readings, since the pages give only the chain rule:
 *  - the draft tokens of a node are its top-k (chosen, not sampled), so
 *    as a proposal each is a point mass: the ratio for child token t is
 *    p(t) / 1, and rejecting t leaves the residual max(p - delta_t, 0),
 *    i.e. p with t removed and renormalised;
 *  - p = softmax(target row / tau) over the whole vocabulary;
 *  - a node's children are tried in slot order (highest value first);
 *    child c is accepted iff u[c] * R < p(token c), R being the target
 *    mass not yet rejected at this node (unnormalised weights below);
 *  - when every child of the final node is rejected (or it has none), the
 *    bonus token is drawn from the residual by inverse CDF in token-id
 *    order with u[0]: the first id whose running residual mass exceeds
 *    u[0] * R (no such id: the last id of positive residual mass; none
 *    of those either: the lowest id not rejected).
 * uniforms: fp32 [B][T] in [0, 1); u[b][s] is used when slot s is tried
 * (each slot at most once per cycle), u[b][0] for the bonus draw.
 * margin[b]: the smallest |u*R - p| (ratio tests) or distance of u[0]*R
 * to the chosen id's mass interval (bonus), over every decision taken,
 * relative to the row's total mass; a run with a small margin may flip
 * under a different rounding order of the same sums.
 * ------------------------------------------------------------------- */
int etref_accept_sample(int B, int T, int V, int D, int dtype,
                        const void* target, int64_t bstride, int64_t rstride,
                        const int32_t* tokens, const int32_t* parent_slot,
                        const int32_t* n_kept, double tau,
                        const float* uniforms, int32_t* accept_len,
                        int32_t* path_slots, int32_t* out_tokens,
                        double* margin) {
  double* wgt = (double*)malloc(sizeof(double) * (size_t)V);
  char* rejected = (char*)malloc((size_t)V);
  if (!wgt || !rejected) {
    free(wgt);
    free(rejected);
    return -2;
  }
  for (int b = 0; b < B; ++b) {
    const int n = n_kept[b];
    const int32_t* tk = tokens + (int64_t)b * T;
    const int32_t* ps = parent_slot + (int64_t)b * T;
    const float* u = uniforms + (int64_t)b * T;
    int32_t* pth = path_slots + (int64_t)b * (D + 1);
    int32_t* ot = out_tokens + (int64_t)b * (D + 1);
    for (int i = 0; i <= D; ++i) {
      pth[i] = -1;
      ot[i] = -1;
    }
    pth[0] = 0;
    int cur = 0, len = 0;
    double mg = INFINITY;
    for (;;) {
      /* target weights exp((x - max) / tau) of the current slot's row */
      const char* row = (const char*)target +
                        (b * bstride + cur * rstride) * (dtype == REF_F32 ? 4 : 2);
      double m = -INFINITY;
      for (int v = 0; v < V; ++v) {
        double x = ref_load(row, dtype, v);
        if (x > m) m = x;
      }
      double Z = 0.0;
      for (int v = 0; v < V; ++v) {
        wgt[v] = exp((ref_load(row, dtype, v) - m) / tau);
        Z += wgt[v];
      }
      memset(rejected, 0, (size_t)V);
      /* ratio tests of the children, in slot order */
      double R = Z;
      int next = -1;
      if (len < D) {
        for (int c = 1; c <= n; ++c) {
          if (ps[c] != cur) continue;
          const double p = wgt[tk[c]];
          const double lhs = (double)u[c] * R;
          const double d = fabs(lhs - p) / Z;
          if (d < mg) mg = d;
          if (lhs < p) {
            next = c;
            break;
          }
          R -= p;
          rejected[tk[c]] = 1;
        }
      }
      if (next >= 0) {
        ot[len] = tk[next];
        ++len;
        pth[len] = next;
        cur = next;
        continue;
      }
      /* bonus: inverse CDF of the residual in id order */
      const double t = (double)u[0] * R;
      double C = 0.0;
      int pick = -1, last = -1;
      for (int v = 0; v < V; ++v) {
        if (rejected[v] || !(wgt[v] > 0.0)) continue;
        const double Cn = C + wgt[v];
        last = v;
        if (Cn > t) {
          const double d = fmin(t - C, Cn - t) / Z;
          if (d < mg) mg = d;
          pick = v;
          break;
        }
        C = Cn;
      }
      if (pick < 0 && last >= 0) {
        const double d = fabs(t - C) / Z;
        if (d < mg) mg = d;
        pick = last;
      }
      if (pick < 0) {
        pick = 0;
        while (pick < V - 1 && rejected[pick]) ++pick;
        mg = 0.0;
      }
      ot[len] = pick;
      break;
    }
    accept_len[b] = len;
    margin[b] = mg;
  }
  free(wgt);
  free(rejected);
  return 0;
}

/* ---------------------------------------------------------------------
 * Static draft tree: the fixed-shape baseline the dynamic tree is compared
 * with ([P2] "Watch the Budget Being Spent": an EAGLE-1-style fixed shape
 * spends the same node budget; [P3] EAGLE: one static prior tree is used
 * for every input).  The shape: nodes s = 1..M, parent sp[s] in [0, s)
 * (0 = root), child rank sr[s] in [0, k), distinct among siblings,
 * depth <= D.  Readings: at step l, row j of layer l-1 belongs to the j-th
 * slot, in slot order, of depth l-1 with a child in the shape (at most k
 * such slots); a node's children are its row's top-k by (logit desc, id
 * asc) with conf and value exactly as in the draft step, and the shape
 * keeps the child of rank sr[s].  Slot order is the shape's order.
 * logits: element (b, l, j, v) at b*bstride + l*lstride + j*rstride + v.
 * Outputs as etref_rerank (slot 0 the root; pad slots -1/-1/0/0), with
 * n_kept[b] = M.  Returns -1 for a shape that breaks the rules above.
 * ------------------------------------------------------------------- */
int etref_static_tree(int B, int V, int k, int D, int T, int dtype,
                      const int32_t* root_tokens, const void* logits,
                      int64_t bstride, int64_t lstride, int64_t rstride,
                      int M, const int32_t* sp, const int32_t* sr,
                      int32_t* tokens, int32_t* parent_slot, float* conf,
                      float* value, int32_t* n_kept) {
  if (M < 0 || M > T - 1 || k < 1 || V < k) return -1;
  int32_t* dep = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
  int32_t* row = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* xs = (double*)malloc(sizeof(double) * (size_t)k);
  unsigned char* taken = (unsigned char*)malloc((size_t)V);
  if (!dep || !row || !ids || !xs || !taken) return -2;
  int rc = 0;
  /* depths, rank rules, and the row each expanded slot reads */
  dep[0] = 0;
  for (int s = 1; s <= M && rc == 0; ++s) {
    if (sp[s] < 0 || sp[s] >= s || sr[s] < 0 || sr[s] >= k) rc = -1;
    else dep[s] = dep[sp[s]] + 1;
    if (rc == 0 && dep[s] > D) rc = -1;
    for (int t = 1; t < s && rc == 0; ++t)
      if (sp[t] == sp[s] && sr[t] == sr[s]) rc = -1;
  }
  for (int l = 0; l < D && rc == 0; ++l) {
    int j = 0;
    for (int s = 0; s <= M; ++s) {
      if (dep[s] != l) continue;
      int has_child = 0;
      for (int c = s + 1; c <= M; ++c) has_child |= sp[c] == s;
      row[s] = has_child ? j++ : -1;
    }
    if (j > k) rc = -1;
  }
  for (int b = 0; b < B && rc == 0; ++b) {
    int32_t* tk = tokens + (int64_t)b * T;
    int32_t* ps = parent_slot + (int64_t)b * T;
    float* cf = conf + (int64_t)b * T;
    float* vl = value + (int64_t)b * T;
    tk[0] = root_tokens[b];
    ps[0] = -1;
    cf[0] = 1.0f;
    vl[0] = 1.0f;
    for (int s = 1; s <= M; ++s) {
      const int p = sp[s];
      const char* x = (const char*)logits +
                      (b * bstride + dep[p] * lstride + row[p] * rstride) *
                          (dtype == REF_F32 ? 4 : 2);
      double m, sum;
      ref_row_softmax(x, dtype, V, &m, &sum);
      ref_row_topk(x, dtype, V, k, ids, xs, taken);
      const float c = (float)(exp(xs[sr[s]] - m) / sum);
      tk[s] = ids[sr[s]];
      ps[s] = p;
      cf[s] = c;
      vl[s] = vl[p] * c;
    }
    for (int s = M + 1; s < T; ++s) {
      tk[s] = -1;
      ps[s] = -1;
      cf[s] = 0.0f;
      vl[s] = 0.0f;
    }
    n_kept[b] = M;
  }
  free(dep);
  free(row);
  free(ids);
  free(xs);
  free(taken);
  return rc;
}

/* Cap the threads of the OpenMP loop above (no effect without OpenMP);
 * the single-threaded baseline of the benchmark uses 1. */
void etref_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads the OpenMP loop above may use (1 without OpenMP). */
int etref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
