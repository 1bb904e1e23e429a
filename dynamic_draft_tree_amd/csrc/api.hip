// api.hip -- the extern "C" boundary of libeagletree: argument validation,
// plan creation, workspace layout and kernel launches.  Every check runs
// on the host before anything is launched; kernels never allocate.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ET_OK;
  return fail(ET_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define CHECK_PTR(p)                                                  \
  do {                                                                \
    if (!(p)) return fail(ET_EINVAL, "%s: %s is NULL", fn, #p);        \
  } while (0)

et::Plan* as_plan(et_plan_t p) { return reinterpret_cast<et::Plan*>(p); }

// Region indices of Plan::off.
enum {
  R_POOL_TOKEN, R_POOL_PARENT, R_POOL_DEPTH, R_POOL_CONF, R_POOL_VALUE,
  R_POOL_COUNT, R_ROOT, R_FRONTIER, R_FRONTIER_VAL, R_FRONTIER_COUNT, R_PART_M, R_PART_S,
  R_PART_KEYS, R_LM_M, R_LM_S, R_LM_KEYS, R_ACC_PART,
  R_ATT_O, R_ATT_M, R_ATT_L, R_ATT_ORDER, R_COUNT
};

void layout(et::Plan& p) {
  const size_t B = p.B, k = p.k, S = p.s_draft, T = p.T, cap = p.cap;
  const size_t units = (size_t)p.B * p.Hkv * p.attn_nqb * p.attn_splits;
  const size_t att_rows = p.attn_splits > 1 ? units * 64 * p.attn_wr : 0;
  size_t sz[R_COUNT] = {};
  sz[R_POOL_TOKEN] = sz[R_POOL_PARENT] = sz[R_POOL_DEPTH] = B * cap * 4;
  sz[R_POOL_CONF] = sz[R_POOL_VALUE] = B * cap * 4;
  sz[R_POOL_COUNT] = sz[R_ROOT] = B * 4;
  sz[R_FRONTIER] = 2 * B * k * 4;
  sz[R_FRONTIER_VAL] = 2 * B * k * 4;
  sz[R_FRONTIER_COUNT] = 2 * B * 4;
  // draft partials: one per (row, chunk, wave of the scan block)
  const size_t W4 = et::kScanThreads / 64;
  sz[R_PART_M] = sz[R_PART_S] = B * k * S * W4 * 4;
  sz[R_PART_KEYS] = B * k * S * W4 * et::kMaxTopk * 8;
  // LM-head lists: per (row, 512-id vocab block)
  const size_t L1 = et::lm_lists1(p.V);
  sz[R_LM_M] = sz[R_LM_S] = B * k * L1 * 4;
  sz[R_LM_KEYS] = B * k * L1 * et::kMaxTopk * 8;
  // accept partials: per (slot row, chunk, wave) an 8-byte argmax key
  // (greedy) or a 16-byte (max, fp64 mass) pair (sampled)
  sz[R_ACC_PART] = B * T * p.s_accept * W4 * 16;
  sz[R_ATT_O] = att_rows * p.HD * 4;
  sz[R_ATT_M] = sz[R_ATT_L] = att_rows * 4;
  sz[R_ATT_ORDER] = B * 4;
  size_t off = 0;
  for (int r = 0; r < R_COUNT; ++r) {
    p.off[r] = off;
    off += align256(sz[r]);
  }
  p.ws_bytes = off;
}

// Chunks per scan block for `rows` rows of S chunks: 1 unless rows * S
// blocks would be many times what the chip holds; then spread evenly
// over each row's blocks.
int chunks_per_block(long long rows, int S) {
  long long cpb = (rows * S + et::kScanTargetBlocks - 1) / et::kScanTargetBlocks;
  if (cpb > S) cpb = S;
  const long long per_row = (S + cpb - 1) / cpb;
  return (int)((S + per_row - 1) / per_row);
}

template <typename T>
T* at(void* ws, const et::Plan& p, int r) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + p.off[r]);
}

// ---- checks of documented device preconditions (ET_DEBUG) ---------------
// The calls document what they expect of device data (n_kept, parent_slot,
// tokens as et_rerank writes them; prefix lengths within the cache) rather
// than checking it on every launch.  With ET_DEBUG set when a plan is
// created, every call of that plan copies those inputs to the host and
// checks them before launching, synchronises after launching (a kernel
// fault is reported by the call that caused it) and checks the tree and
// frontier outputs it wrote.  The same checks are exported for host
// arrays (et_check_tree, et_check_prefix).

bool env_debug() {
  const char* e = std::getenv("ET_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}

// The tree layout of et_rerank: 0 <= n_kept <= N; slot 0 the root (parent
// -1, a token); slots 1..n a token in [0, V) and a parent slot in [0, s);
// pad slots token -1 and parent -1.  tokens may be NULL (not checked).
int check_tree_host(const et::Plan& p, const char* fn, const int32_t* tokens,
                    const int32_t* parent, const int32_t* n_kept) {
  for (int b = 0; b < p.B; ++b) {
    const int n = n_kept[b];
    if (n < 0 || n > p.N)
      return fail(ET_EINVAL, "%s: n_kept[%d] = %d outside 0..%d", fn, b, n, p.N);
    for (int s = 0; s < p.T; ++s) {
      const int64_t o = (int64_t)b * p.T + s;
      const int par = parent[o];
      const int tok = tokens ? tokens[o] : 0;
      const bool kept = s <= n;
      const bool par_ok = s == 0 || !kept ? par == -1 : (par >= 0 && par < s);
      if (!par_ok)
        return fail(ET_EINVAL, "%s: parent_slot[%d][%d] = %d (n_kept %d)", fn, b, s, par, n);
      if (tokens && (kept ? (tok < 0 || tok >= p.V) : tok != -1))
        return fail(ET_EINVAL, "%s: tokens[%d][%d] = %d (n_kept %d, vocab %d)", fn, b, s,
                    tok, n, p.V);
    }
  }
  return ET_OK;
}

int check_prefix_host(const et::Plan& p, const char* fn, const int32_t* prefix_len) {
  for (int b = 0; b < p.B; ++b)
    if (prefix_len[b] < 0 || prefix_len[b] > p.Pcap)
      return fail(ET_EINVAL, "%s: prefix_len[%d] = %d outside 0..%d", fn, b, prefix_len[b],
                  p.Pcap);
  return ET_OK;
}

// Copy n int32 values from the device (stream-ordered) and wait.
int d2h(const char* fn, std::vector<int32_t>& h, const int32_t* d, size_t n, hipStream_t s) {
  h.resize(n);
  hipError_t e = hipMemcpyAsync(h.data(), d, n * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(ET_EHIP, "%s (ET_DEBUG): device read: %s", fn, hipGetErrorString(e));
  return ET_OK;
}

// tokens may be NULL; n_kept only (parent == NULL) checks n_kept's range.
int debug_tree(const et::Plan& p, const char* fn, const int32_t* tokens, const int32_t* parent,
               const int32_t* n_kept, hipStream_t s) {
  std::vector<int32_t> tk, ps, nk;
  int rc = d2h(fn, nk, n_kept, p.B, s);
  if (rc == ET_OK && tokens) rc = d2h(fn, tk, tokens, (size_t)p.B * p.T, s);
  if (rc == ET_OK && parent) rc = d2h(fn, ps, parent, (size_t)p.B * p.T, s);
  if (rc != ET_OK) return rc;
  if (!parent) {
    for (int b = 0; b < p.B; ++b)
      if (nk[b] < 0 || nk[b] > p.N)
        return fail(ET_EINVAL, "%s: n_kept[%d] = %d outside 0..%d", fn, b, nk[b], p.N);
    return ET_OK;
  }
  return check_tree_host(p, fn, tokens ? tk.data() : nullptr, ps.data(), nk.data());
}

int debug_prefix(const et::Plan& p, const char* fn, const int32_t* prefix_len, hipStream_t s) {
  std::vector<int32_t> pl;
  const int rc = d2h(fn, pl, prefix_len, p.B, s);
  return rc != ET_OK ? rc : check_prefix_host(p, fn, pl.data());
}

// After a launch: wait for it and report a failure on the device.
int debug_sync(const char* fn, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(ET_EHIP, "%s (ET_DEBUG): failed on the device: %s", fn,
                                   hipGetErrorString(e));
  return ET_OK;
}

// After a draft step: 0 <= next_count <= k, next_tokens in [0, V) for the
// first next_count entries and -1 after.
int debug_frontier(const et::Plan& p, const char* fn, const int32_t* next_tokens,
                   const int32_t* next_count, hipStream_t s) {
  std::vector<int32_t> nt, nc;
  int rc = debug_sync(fn, s);
  if (rc == ET_OK) rc = d2h(fn, nc, next_count, p.B, s);
  if (rc == ET_OK) rc = d2h(fn, nt, next_tokens, (size_t)p.B * p.k, s);
  if (rc != ET_OK) return rc;
  for (int b = 0; b < p.B; ++b) {
    if (nc[b] < 0 || nc[b] > p.k)
      return fail(ET_EINVAL, "%s: next_count[%d] = %d outside 0..%d", fn, b, nc[b], p.k);
    for (int j = 0; j < p.k; ++j) {
      const int t = nt[(size_t)b * p.k + j];
      if (j < nc[b] ? (t < 0 || t >= p.V) : t != -1)
        return fail(ET_EINVAL, "%s: next_tokens[%d][%d] = %d (next_count %d)", fn, b, j, t,
                    nc[b]);
    }
  }
  return ET_OK;
}

}  // namespace

namespace et {

DraftWs draft_ws(const Plan& p, void* ws) {
  DraftWs w;
  w.pool_token = at<int32_t>(ws, p, R_POOL_TOKEN);
  w.pool_parent = at<int32_t>(ws, p, R_POOL_PARENT);
  w.pool_depth = at<int32_t>(ws, p, R_POOL_DEPTH);
  w.pool_conf = at<float>(ws, p, R_POOL_CONF);
  w.pool_value = at<float>(ws, p, R_POOL_VALUE);
  w.pool_count = at<int32_t>(ws, p, R_POOL_COUNT);
  w.root_token = at<int32_t>(ws, p, R_ROOT);
  w.frontier = at<int32_t>(ws, p, R_FRONTIER);
  w.frontier_val = at<float>(ws, p, R_FRONTIER_VAL);
  w.frontier_count = at<int32_t>(ws, p, R_FRONTIER_COUNT);
  w.part_m = at<float>(ws, p, R_PART_M);
  w.part_s = at<float>(ws, p, R_PART_S);
  w.part_keys = at<uint64_t>(ws, p, R_PART_KEYS);
  return w;
}

LmWs lm_ws(const Plan& p, void* ws) {
  LmWs w;
  w.m = at<float>(ws, p, R_LM_M);
  w.s = at<float>(ws, p, R_LM_S);
  w.keys = at<uint64_t>(ws, p, R_LM_KEYS);
  return w;
}

AcceptWs accept_ws(const Plan& p, void* ws) {
  AcceptWs w;
  w.part = at<uint64_t>(ws, p, R_ACC_PART);
  return w;
}

AttnWs attn_ws(const Plan& p, void* ws) {
  AttnWs w;
  w.o = at<float>(ws, p, R_ATT_O);
  w.m = at<float>(ws, p, R_ATT_M);
  w.l = at<float>(ws, p, R_ATT_L);
  w.order = at<int32_t>(ws, p, R_ATT_ORDER);
  return w;
}

}  // namespace et

extern "C" {

const char* et_last_error(void) { return g_err; }

int et_check_tree(et_plan_t plan, const int32_t* tokens, const int32_t* parent_slot,
                  const int32_t* n_kept) {
  const char* fn = "et_check_tree";
  CHECK_PTR(plan);
  CHECK_PTR(parent_slot);
  CHECK_PTR(n_kept);
  return check_tree_host(*as_plan(plan), fn, tokens, parent_slot, n_kept);
}

int et_check_prefix(et_plan_t plan, const int32_t* prefix_len) {
  const char* fn = "et_check_prefix";
  CHECK_PTR(plan);
  CHECK_PTR(prefix_len);
  return check_prefix_host(*as_plan(plan), fn, prefix_len);
}

int et_plan_debug(et_plan_t plan) { return plan && as_plan(plan)->debug ? 1 : 0; }

int et_plan_create(const et_config* cfg, et_plan_t* out) {
  const char* fn = "et_plan_create";
  CHECK_PTR(cfg);
  CHECK_PTR(out);
  const et_config& c = *cfg;
  if (c.logits_dtype != ET_F32 && c.logits_dtype != ET_BF16)
    return fail(ET_EUNSUPPORTED, "%s: logits_dtype %d", fn, c.logits_dtype);
  if (c.qkv_dtype != ET_F32 && c.qkv_dtype != ET_BF16)
    return fail(ET_EUNSUPPORTED, "%s: qkv_dtype %d", fn, c.qkv_dtype);
  if (c.batch < 1 || c.batch > 65535)
    return fail(ET_EINVAL, "%s: batch %d outside 1..65535", fn, c.batch);
  if (c.vocab < 2 || c.vocab > et::kMaxVocab)
    return fail(ET_EUNSUPPORTED, "%s: vocab %d outside 2..%d", fn, c.vocab,
                et::kMaxVocab);
  if (c.topk < 1 || c.topk > et::kMaxTopk)
    return fail(ET_EUNSUPPORTED, "%s: topk %d outside 1..%d", fn, c.topk,
                et::kMaxTopk);
  if (c.topk > c.vocab)
    return fail(ET_EINVAL, "%s: topk %d > vocab %d", fn, c.topk, c.vocab);
  if (c.depth < 1 || c.depth > et::kMaxDepth)
    return fail(ET_EUNSUPPORTED, "%s: depth %d outside 1..%d", fn, c.depth,
                et::kMaxDepth);
  if (c.budget_n < 1 || c.budget_n > et::kMaxBudget)
    return fail(ET_EUNSUPPORTED, "%s: budget_n %d outside 1..%d", fn,
                c.budget_n, et::kMaxBudget);
  if (!(c.expand_threshold >= 0.0f) || c.expand_threshold > 1.0f)
    return fail(ET_EINVAL, "%s: expand_threshold outside [0, 1]", fn);
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(ET_EUNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn,
                c.head_dim);
  if (c.n_kv_heads < 1 || c.n_q_heads < c.n_kv_heads ||
      c.n_q_heads % c.n_kv_heads != 0)
    return fail(ET_EINVAL, "%s: heads %d / %d not grouped", fn, c.n_q_heads,
                c.n_kv_heads);
  if (c.n_q_heads / c.n_kv_heads > 16)
    return fail(ET_EUNSUPPORTED, "%s: group size %d > 16", fn,
                c.n_q_heads / c.n_kv_heads);
  if (c.prefix_cap < 1)
    return fail(ET_EINVAL, "%s: prefix_cap %d < 1", fn, c.prefix_cap);
  const long long cap = c.topk + (long long)(c.depth - 1) * c.topk * c.topk;
  if (cap > et::kMaxPool)
    return fail(ET_EUNSUPPORTED, "%s: pool capacity %lld > %d", fn, cap,
                et::kMaxPool);

  et::Plan* p = new (std::nothrow) et::Plan();
  if (!p) return fail(ET_EINVAL, "%s: out of host memory", fn);
  p->cfg = c;
  p->static_m = -1;
  p->B = c.batch;
  p->V = c.vocab;
  p->k = c.topk;
  p->D = c.depth;
  p->N = c.budget_n;
  p->T = c.budget_n + 1;
  p->W = (p->T + 63) / 64;
  p->cap = (int)cap;
  p->Hq = c.n_q_heads;
  p->Hkv = c.n_kv_heads;
  p->G = c.n_q_heads / c.n_kv_heads;
  p->HD = c.head_dim;
  p->Pcap = c.prefix_cap;
  p->ldt = c.logits_dtype;
  p->qdt = c.qkv_dtype;
  {
    const int narrow = (p->V + et::chunk_elems(p->ldt, false) - 1) / et::chunk_elems(p->ldt, false);
    p->draft_wide = (long long)p->B * p->k * narrow > et::kScanWideBlocks;
    const int ce = et::chunk_elems(p->ldt, p->draft_wide);
    p->s_draft = (p->V + ce - 1) / ce;
  }
  p->s_accept = (p->V + et::accept_chunk_elems(p->ldt) - 1) / et::accept_chunk_elems(p->ldt);
  p->draft_cpb = chunks_per_block((long long)p->B * p->k, p->s_draft);
  p->accept_cpb = chunks_per_block((long long)p->B * p->T, p->s_accept);
  // Attention: the G*T query rows of one kv head are cut into blocks of
  // 64 or 128 rows.  When the kv heads alone leave most compute units idle
  // (keys must be split, and every split writes partials of its block's
  // rows), 64-row blocks keep the partials small; otherwise 128 rows when
  // that adds no padding rows (each K/V tile then serves twice the rows).
  // The keys are split until the grid has about one block per compute
  // unit.
  {
    const int R = p->T * p->G;
    const int q1 = (R + 63) / 64, q2 = (R + 127) / 128;
    const bool split_keys = (long long)p->B * p->Hkv * q1 < et::kAttnTargetBlocks;
    p->attn_wr = !split_keys && q2 * 128 <= q1 * 64 ? 2 : 1;
    p->attn_nqb = p->attn_wr == 2 ? q2 : q1;
  }
  const long long units = (long long)p->B * p->Hkv * p->attn_nqb;
  const int max_tiles = (p->Pcap + p->T + et::kAttnTile - 1) / et::kAttnTile;
  long long splits = (et::kAttnTargetBlocks + units - 1) / units;
  if (splits > max_tiles) splits = max_tiles;
  if (splits > et::kAttnMaxSplits) splits = et::kAttnMaxSplits;
  if (splits < 1) splits = 1;
  p->attn_splits = p->qdt == ET_F32 ? 1 : (int)splits;
  p->last_ws = nullptr;
  p->last_step = 0;
  p->debug = env_debug();
  layout(*p);
  *out = reinterpret_cast<et_plan_t>(p);
  g_err[0] = 0;
  return ET_OK;
}

int et_plan_destroy(et_plan_t plan) {
  delete as_plan(plan);
  return ET_OK;
}

size_t et_workspace_bytes(et_plan_t plan) {
  return plan ? as_plan(plan)->ws_bytes : 0;
}

int32_t et_pool_capacity(et_plan_t plan) {
  return plan ? as_plan(plan)->cap : 0;
}

int et_workspace_init(et_plan_t plan, void* ws, et_stream_t stream) {
  const char* fn = "et_workspace_init";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  (void)stream;  // no device state needs clearing
  et::Plan& p = *as_plan(plan);
  p.last_ws = nullptr;
  p.last_step = 0;
  return ET_OK;
}

namespace {

int draft_step(const char* fn, et_plan_t plan, void* ws, int32_t step,
               const int32_t* root_tokens, const void* logits,
               int64_t batch_stride, int64_t row_stride, int32_t* next_tokens,
               int32_t* next_count, et_stream_t stream, bool fixed,
               const et::RerankOut* last = nullptr) {
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(logits);
  CHECK_PTR(next_tokens);
  CHECK_PTR(next_count);
  et::Plan& p = *as_plan(plan);
  if (step < 1 || step > p.D)
    return fail(ET_EINVAL, "%s: step %d outside 1..%d", fn, step, p.D);
  if (step == 1) CHECK_PTR(root_tokens);
  if (row_stride < p.V)
    return fail(ET_EINVAL, "%s: row_stride %lld < vocab %d", fn,
                (long long)row_stride, p.V);
  if (batch_stride < 0)
    return fail(ET_EINVAL, "%s: negative batch_stride", fn);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  if (step != 1 && (p.last_ws != ws || p.last_step != step - 1 || p.last_fixed != fixed))
    return fail(ET_ESTATE, "%s: step %d does not follow step %d of the same "
                "policy on this workspace", fn, step, p.last_step);
  if (fixed && p.static_m < 0)
    return fail(ET_ESTATE, "%s: no fixed shape set (et_set_static_shape)", fn);
  et::FixedFrontier ff;
  if (fixed) {
    ff.n = step < p.D ? p.static_nf[step + 1] : 0;
    for (int i = 0; i < et::kMaxTopk; ++i) ff.ci[i] = p.static_next[step][i];
  }
  const int per = p.ldt == ET_BF16 ? 8 : 4;
  const bool vec = aligned16(logits) && batch_stride % per == 0 &&
                   row_stride % per == 0 && p.V >= per;
  int rc = hip_status(
      et::launch_draft_step(p, et::draft_ws(p, ws), step, root_tokens, logits,
                            batch_stride, row_stride, vec, fixed ? &ff : nullptr,
                            next_tokens, next_count, (hipStream_t)stream, last),
      fn);
  if (rc == ET_OK && p.debug)
    rc = debug_frontier(p, fn, next_tokens, next_count, (hipStream_t)stream);
  if (rc == ET_OK && p.debug && last)
    rc = debug_tree(p, fn, last->tokens, last->parent_slot, last->n_kept, (hipStream_t)stream);
  if (rc == ET_OK) {
    p.last_ws = ws;
    p.last_step = step;
    p.last_fixed = fixed;
  }
  return rc;
}

}  // namespace

int et_draft_step(et_plan_t plan, void* ws, int32_t step,
                  const int32_t* root_tokens, const void* logits,
                  int64_t batch_stride, int64_t row_stride,
                  int32_t* next_tokens, int32_t* next_count,
                  et_stream_t stream) {
  return draft_step("et_draft_step", plan, ws, step, root_tokens, logits,
                    batch_stride, row_stride, next_tokens, next_count, stream,
                    false);
}

int et_draft_step_last(et_plan_t plan, void* ws, const int32_t* root_tokens,
                       const void* logits, int64_t batch_stride, int64_t row_stride,
                       int32_t* next_tokens, int32_t* next_count,
                       const int32_t* prefix_len, int32_t* tokens, int32_t* parent_slot,
                       float* conf, float* value, int32_t* n_kept, uint64_t* mask,
                       int32_t* depth, int32_t* pos_ids, et_stream_t stream) {
  const char* fn = "et_draft_step_last";
  CHECK_PTR(plan);
  CHECK_PTR(prefix_len);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(conf);
  CHECK_PTR(value);
  CHECK_PTR(n_kept);
  CHECK_PTR(mask);
  CHECK_PTR(depth);
  CHECK_PTR(pos_ids);
  et::Plan& p = *as_plan(plan);
  // the merge block (64 k threads) holds at most kRerankPer pool nodes per
  // thread; every valid configuration fits (capacity <= 1 + k + 14 k^2)
  if (p.cap > 4 * 64 * p.k)
    return fail(ET_EUNSUPPORTED, "%s: pool capacity %d above %d", fn, p.cap, 4 * 64 * p.k);
  if (p.debug) {
    const int rc = debug_prefix(p, fn, prefix_len, (hipStream_t)stream);
    if (rc != ET_OK) return rc;
  }
  et::RerankOut o;
  o.tokens = tokens;
  o.parent_slot = parent_slot;
  o.conf = conf;
  o.value = value;
  o.n_kept = n_kept;
  o.prefix_len = prefix_len;
  o.mask = mask;
  o.depth = depth;
  o.pos = pos_ids;
  o.N = p.N;
  o.T = p.T;
  o.W = p.W;
  return draft_step(fn, plan, ws, p.D, root_tokens, logits, batch_stride, row_stride,
                    next_tokens, next_count, stream, false, &o);
}

int et_draft_step_static(et_plan_t plan, void* ws, int32_t step,
                         const int32_t* root_tokens, const void* logits,
                         int64_t batch_stride, int64_t row_stride,
                         int32_t* next_tokens, int32_t* next_count,
                         et_stream_t stream) {
  return draft_step("et_draft_step_static", plan, ws, step, root_tokens,
                    logits, batch_stride, row_stride, next_tokens, next_count,
                    stream, true);
}

int et_draft_step_hidden(et_plan_t plan, void* ws, int32_t step,
                         const int32_t* root_tokens, const void* hidden,
                         int64_t batch_stride, int64_t row_stride,
                         const void* lm_head, int32_t hidden_dim,
                         int32_t* next_tokens, int32_t* next_count,
                         et_stream_t stream) {
  const char* fn = "et_draft_step_hidden";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(hidden);
  CHECK_PTR(lm_head);
  CHECK_PTR(next_tokens);
  CHECK_PTR(next_count);
  et::Plan& p = *as_plan(plan);
  if (step < 1 || step > p.D)
    return fail(ET_EINVAL, "%s: step %d outside 1..%d", fn, step, p.D);
  if (step == 1) CHECK_PTR(root_tokens);
  if (hidden_dim < 128 || hidden_dim > 65536 || hidden_dim % 128 != 0)
    return fail(ET_EUNSUPPORTED, "%s: hidden_dim %d not a multiple of 128 in 128..65536",
                fn, hidden_dim);
  if (row_stride < hidden_dim || batch_stride < 0 || row_stride % 8 != 0 ||
      batch_stride % 8 != 0)
    return fail(ET_EINVAL, "%s: strides %lld, %lld (elements) must be multiples of 8, "
                "row_stride >= hidden_dim", fn, (long long)batch_stride,
                (long long)row_stride);
  if (!aligned16(hidden) || !aligned16(lm_head))
    return fail(ET_EINVAL, "%s: hidden and lm_head must be 16-byte aligned", fn);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  if (step != 1 && (p.last_ws != ws || p.last_step != step - 1 || p.last_fixed))
    return fail(ET_ESTATE, "%s: step %d does not follow step %d of the same "
                "policy on this workspace", fn, step, p.last_step);
  int rc = hip_status(
      et::launch_draft_step_hidden(p, et::draft_ws(p, ws), et::lm_ws(p, ws), step,
                                   root_tokens, hidden, batch_stride, row_stride,
                                   lm_head, hidden_dim, next_tokens, next_count,
                                   (hipStream_t)stream),
      fn);
  if (rc == ET_OK && p.debug)
    rc = debug_frontier(p, fn, next_tokens, next_count, (hipStream_t)stream);
  if (rc == ET_OK) {
    p.last_ws = ws;
    p.last_step = step;
    p.last_fixed = false;
  }
  return rc;
}

int et_set_static_shape(et_plan_t plan, const int32_t* parent,
                        const int32_t* rank, int32_t n_nodes) {
  const char* fn = "et_set_static_shape";
  CHECK_PTR(plan);
  et::Plan& p = *as_plan(plan);
  if (n_nodes < 0 || n_nodes > p.N)
    return fail(ET_EINVAL, "%s: %d nodes outside 0..%d", fn, n_nodes, p.N);
  if (n_nodes > 0) {
    CHECK_PTR(parent);
    CHECK_PTR(rank);
  }
  // slot s = node s - 1 of the arrays; slot 0 is the root
  int dep[et::kMaxBudget + 1], row[et::kMaxBudget + 1];
  bool has_child[et::kMaxBudget + 1] = {};
  dep[0] = 0;
  for (int s = 1; s <= n_nodes; ++s) {
    const int ps = parent[s - 1], r = rank[s - 1];
    if (ps < 0 || ps >= s)
      return fail(ET_EINVAL, "%s: slot %d: parent %d not an earlier slot", fn, s, ps);
    if (r < 0 || r >= p.k)
      return fail(ET_EINVAL, "%s: slot %d: rank %d outside 0..%d", fn, s, r, p.k - 1);
    dep[s] = dep[ps] + 1;
    if (dep[s] > p.D)
      return fail(ET_EINVAL, "%s: slot %d: depth %d > %d", fn, s, dep[s], p.D);
    for (int t = 1; t < s; ++t)
      if (parent[t - 1] == ps && rank[t - 1] == r)
        return fail(ET_EINVAL, "%s: slots %d and %d: same rank under one parent", fn, t, s);
    has_child[ps] = true;
  }
  // rows of each step: the slots of the layer above with a child, in slot
  // order (at most k)
  int nf[et::kMaxDepth + 2] = {};
  for (int s = 0; s <= n_nodes; ++s) {
    row[s] = -1;
    if (!has_child[s]) continue;
    const int l = dep[s] + 1;
    if (nf[l] == p.k)
      return fail(ET_EINVAL, "%s: more than %d slots of depth %d have children", fn,
                  p.k, dep[s]);
    row[s] = nf[l]++;
  }
  int base[et::kMaxDepth + 2] = {};
  for (int l = 2; l <= p.D; ++l) base[l] = base[l - 1] + nf[l - 1] * p.k;
  for (int l = 0; l <= p.D; ++l)
    for (int i = 0; i < et::kMaxTopk; ++i) p.static_next[l][i] = -1;
  for (int s = 1; s <= n_nodes; ++s) {
    const int ps = parent[s - 1], l = dep[s];
    const int ci = row[ps] * p.k + rank[s - 1];  // child index within step l
    p.static_slot[s] = (base[l] + ci) | (ps << 16);
    if (has_child[s]) p.static_next[l][row[s]] = ci;
  }
  for (int l = 0; l <= p.D + 1; ++l) p.static_nf[l] = nf[l];
  p.static_m = n_nodes;
  return ET_OK;
}

int et_static_tree(et_plan_t plan, void* ws, int32_t* tokens,
                   int32_t* parent_slot, float* conf, float* value,
                   int32_t* n_kept, et_stream_t stream) {
  const char* fn = "et_static_tree";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(conf);
  CHECK_PTR(value);
  CHECK_PTR(n_kept);
  et::Plan& p = *as_plan(plan);
  if (p.static_m < 0)
    return fail(ET_ESTATE, "%s: no fixed shape set (et_set_static_shape)", fn);
  if (p.last_ws != ws || p.last_step != p.D || !p.last_fixed)
    return fail(ET_ESTATE, "%s: the fixed-shape tree is not complete (last "
                "step %d of %d on this workspace)", fn, p.last_step, p.D);
  et::FixedSlots fs;
  fs.m = p.static_m;
  for (int s = 0; s <= et::kMaxBudget; ++s) fs.slot[s] = s <= p.static_m ? p.static_slot[s] : 0;
  int rc = hip_status(et::launch_static_tree(p, et::draft_ws(p, ws), fs, tokens,
                                             parent_slot, conf, value, n_kept,
                                             (hipStream_t)stream),
                      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, (hipStream_t)stream);
  if (rc == ET_OK && p.debug)
    rc = debug_tree(p, fn, tokens, parent_slot, n_kept, (hipStream_t)stream);
  return rc;
}

int et_rerank(et_plan_t plan, void* ws, int32_t* tokens, int32_t* parent_slot,
              float* conf, float* value, int32_t* n_kept,
              et_stream_t stream) {
  const char* fn = "et_rerank";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(conf);
  CHECK_PTR(value);
  CHECK_PTR(n_kept);
  et::Plan& p = *as_plan(plan);
  if (p.last_ws != ws || p.last_step != p.D)
    return fail(ET_ESTATE, "%s: the tree is not complete (last step %d of "
                "%d on this workspace)", fn, p.last_step, p.D);
  int rc = hip_status(et::launch_rerank(p, et::draft_ws(p, ws), tokens,
                                        parent_slot, conf, value, n_kept,
                                        (hipStream_t)stream),
                      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, (hipStream_t)stream);
  if (rc == ET_OK && p.debug)
    rc = debug_tree(p, fn, tokens, parent_slot, n_kept, (hipStream_t)stream);
  return rc;
}

int et_rerank_mask(et_plan_t plan, void* ws, int32_t* tokens, int32_t* parent_slot,
                   float* conf, float* value, int32_t* n_kept,
                   const int32_t* prefix_len, uint64_t* mask, int32_t* depth,
                   int32_t* pos_ids, et_stream_t stream) {
  const char* fn = "et_rerank_mask";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(conf);
  CHECK_PTR(value);
  CHECK_PTR(n_kept);
  CHECK_PTR(prefix_len);
  CHECK_PTR(mask);
  CHECK_PTR(depth);
  CHECK_PTR(pos_ids);
  et::Plan& p = *as_plan(plan);
  const hipStream_t st = (hipStream_t)stream;
  if (p.last_ws != ws || p.last_step != p.D)
    return fail(ET_ESTATE, "%s: the tree is not complete (last step %d of "
                "%d on this workspace)", fn, p.last_step, p.D);
  if (p.debug) {
    const int rc = debug_prefix(p, fn, prefix_len, st);
    if (rc != ET_OK) return rc;
  }
  int rc = hip_status(et::launch_rerank_mask(p, et::draft_ws(p, ws), tokens, parent_slot,
                                             conf, value, n_kept, prefix_len, mask,
                                             depth, pos_ids, st),
                      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  if (rc == ET_OK && p.debug) rc = debug_tree(p, fn, tokens, parent_slot, n_kept, st);
  return rc;
}

int et_tree_mask(et_plan_t plan, const int32_t* parent_slot,
                 const int32_t* n_kept, const int32_t* prefix_len,
                 uint64_t* mask, int32_t* depth, int32_t* pos_ids,
                 et_stream_t stream) {
  const char* fn = "et_tree_mask";
  CHECK_PTR(plan);
  CHECK_PTR(parent_slot);
  CHECK_PTR(n_kept);
  CHECK_PTR(prefix_len);
  CHECK_PTR(mask);
  CHECK_PTR(depth);
  CHECK_PTR(pos_ids);
  et::Plan& p = *as_plan(plan);
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    int rc = debug_tree(p, fn, nullptr, parent_slot, n_kept, st);
    if (rc == ET_OK) rc = debug_prefix(p, fn, prefix_len, st);
    if (rc != ET_OK) return rc;
  }
  int rc = hip_status(et::launch_tree_mask(p, parent_slot, n_kept, prefix_len,
                                           mask, depth, pos_ids, st),
                      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

int et_tree_attention(et_plan_t plan, void* ws, const void* q,
                      const void* k_cache, const void* v_cache,
                      const void* k_tree, const void* v_tree,
                      const int32_t* prefix_len, const uint64_t* mask,
                      const int32_t* n_kept, float scale, void* out,
                      et_stream_t stream) {
  const char* fn = "et_tree_attention";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(q);
  CHECK_PTR(k_cache);
  CHECK_PTR(v_cache);
  CHECK_PTR(k_tree);
  CHECK_PTR(v_tree);
  CHECK_PTR(prefix_len);
  CHECK_PTR(mask);
  CHECK_PTR(n_kept);
  CHECK_PTR(out);
  et::Plan& p = *as_plan(plan);
  if (!(scale > 0.0f) || scale != scale)
    return fail(ET_EINVAL, "%s: scale must be positive", fn);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  if (p.qdt == ET_BF16 &&
      !(aligned16(q) && aligned16(k_cache) && aligned16(v_cache) &&
        aligned16(k_tree) && aligned16(v_tree) && aligned16(out)))
    return fail(ET_EINVAL, "%s: bf16 q/k/v/out must be 16-byte aligned", fn);
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    int rc = debug_tree(p, fn, nullptr, nullptr, n_kept, st);
    if (rc == ET_OK) rc = debug_prefix(p, fn, prefix_len, st);
    if (rc != ET_OK) return rc;
  }
  int rc = hip_status(et::launch_tree_attention(
                          p, et::attn_ws(p, ws), q, k_cache, v_cache, k_tree,
                          v_tree, prefix_len, mask, n_kept, scale, out, st),
                      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

int et_accept(et_plan_t plan, void* ws, const void* target_logits,
              int64_t batch_stride, int64_t row_stride, const int32_t* tokens,
              const int32_t* parent_slot, const int32_t* n_kept,
              int32_t* accept_len, int32_t* path_slots, int32_t* out_tokens,
              et_stream_t stream) {
  const char* fn = "et_accept";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(target_logits);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(n_kept);
  CHECK_PTR(accept_len);
  CHECK_PTR(path_slots);
  CHECK_PTR(out_tokens);
  et::Plan& p = *as_plan(plan);
  if (row_stride < p.V)
    return fail(ET_EINVAL, "%s: row_stride %lld < vocab %d", fn,
                (long long)row_stride, p.V);
  if (batch_stride < 0)
    return fail(ET_EINVAL, "%s: negative batch_stride", fn);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  const int per = p.ldt == ET_BF16 ? 8 : 4;
  const bool vec = aligned16(target_logits) && batch_stride % per == 0 &&
                   row_stride % per == 0 && p.V >= per;
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    const int rc = debug_tree(p, fn, tokens, parent_slot, n_kept, st);
    if (rc != ET_OK) return rc;
  }
  int rc = hip_status(
      et::launch_accept(p, et::accept_ws(p, ws), target_logits, batch_stride,
                        row_stride, vec, tokens, parent_slot, n_kept,
                        accept_len, path_slots, out_tokens, st),
      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

}  // extern "C"

// Scratch of et_accept_noalloc: the accept partial keys of one call.  Each
// device the library runs on holds its own copy, at its own address.
static __device__ __align__(256) unsigned char scratch[ET_ACCEPT_NOALLOC_SCRATCH];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, resolved with
// hipGetSymbolAddress on the first call there and kept per device.  (In
// host code the array's name stands for no device address.)
int scratch_on_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ET_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ET_EUNSUPPORTED, "%s: device %d outside 0..%d", fn, dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ET_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ET_OK;
}

}  // namespace

extern "C" {

int et_accept_noalloc(et_plan_t plan, const void* target_logits,
                      int64_t batch_stride, int64_t row_stride,
                      const int32_t* tokens, const int32_t* parent_slot,
                      const int32_t* n_kept, int32_t* accept_len,
                      int32_t* path_slots, int32_t* out_tokens,
                      et_stream_t stream) {
  const char* fn = "et_accept_noalloc";
  CHECK_PTR(plan);
  CHECK_PTR(target_logits);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(n_kept);
  CHECK_PTR(accept_len);
  CHECK_PTR(path_slots);
  CHECK_PTR(out_tokens);
  et::Plan& p = *as_plan(plan);
  if (row_stride < p.V)
    return fail(ET_EINVAL, "%s: row_stride %lld < vocab %d", fn,
                (long long)row_stride, p.V);
  if (batch_stride < 0)
    return fail(ET_EINVAL, "%s: negative batch_stride", fn);
  // one 8-byte key per (target row, chunk, wave)
  const size_t need = (size_t)p.B * p.T * p.s_accept * (et::kScanThreads / 64) * 8;
  if (need > ET_ACCEPT_NOALLOC_SCRATCH)
    return fail(ET_EINVAL, "%s: this plan needs %zu bytes of scratch, the maximum is %u "
                "(use et_accept with a workspace)", fn, need, ET_ACCEPT_NOALLOC_SCRATCH);
  void* sp = nullptr;
  int rc = scratch_on_device(fn, &sp);
  if (rc != ET_OK) return rc;
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    rc = debug_tree(p, fn, tokens, parent_slot, n_kept, st);
    if (rc != ET_OK) return rc;
  }
  et::AcceptWs w;
  w.part = static_cast<uint64_t*>(sp);
  const int per = p.ldt == ET_BF16 ? 8 : 4;
  const bool vec = aligned16(target_logits) && batch_stride % per == 0 &&
                   row_stride % per == 0 && p.V >= per;
  rc = hip_status(
      et::launch_accept(p, w, target_logits, batch_stride, row_stride, vec, tokens,
                        parent_slot, n_kept, accept_len, path_slots, out_tokens, st),
      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

int et_accept_sample(et_plan_t plan, void* ws, const void* target_logits,
                     int64_t batch_stride, int64_t row_stride,
                     const int32_t* tokens, const int32_t* parent_slot,
                     const int32_t* n_kept, float temperature,
                     const float* uniforms, int32_t* accept_len,
                     int32_t* path_slots, int32_t* out_tokens,
                     et_stream_t stream) {
  const char* fn = "et_accept_sample";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  CHECK_PTR(target_logits);
  CHECK_PTR(tokens);
  CHECK_PTR(parent_slot);
  CHECK_PTR(n_kept);
  CHECK_PTR(uniforms);
  CHECK_PTR(accept_len);
  CHECK_PTR(path_slots);
  CHECK_PTR(out_tokens);
  et::Plan& p = *as_plan(plan);
  if (row_stride < p.V)
    return fail(ET_EINVAL, "%s: row_stride %lld < vocab %d", fn,
                (long long)row_stride, p.V);
  if (batch_stride < 0)
    return fail(ET_EINVAL, "%s: negative batch_stride", fn);
  if (((uintptr_t)ws & 255u) != 0)
    return fail(ET_EINVAL, "%s: workspace not 256-byte aligned", fn);
  // weights are exp2((x - max) * c); c must be a finite positive float
  const double c = 1.4426950408889634 / (double)temperature;
  if (!(temperature > 0.0f) || !std::isfinite(temperature) || !std::isfinite((float)c))
    return fail(ET_EINVAL, "%s: temperature %g out of range", fn, (double)temperature);
  const int per = p.ldt == ET_BF16 ? 8 : 4;
  const bool vec = aligned16(target_logits) && batch_stride % per == 0 &&
                   row_stride % per == 0 && p.V >= per;
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    const int rc = debug_tree(p, fn, tokens, parent_slot, n_kept, st);
    if (rc != ET_OK) return rc;
  }
  int rc = hip_status(
      et::launch_accept_sample(p, et::accept_ws(p, ws), target_logits,
                               batch_stride, row_stride, vec, tokens,
                               parent_slot, n_kept, c, uniforms, accept_len,
                               path_slots, out_tokens, st),
      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

int et_kv_commit(et_plan_t plan, void* k_cache, void* v_cache,
                 const void* k_tree, const void* v_tree, int32_t* prefix_len,
                 const int32_t* path_slots, const int32_t* accept_len,
                 et_stream_t stream) {
  const char* fn = "et_kv_commit";
  CHECK_PTR(plan);
  CHECK_PTR(k_cache);
  CHECK_PTR(v_cache);
  CHECK_PTR(k_tree);
  CHECK_PTR(v_tree);
  CHECK_PTR(prefix_len);
  CHECK_PTR(path_slots);
  CHECK_PTR(accept_len);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_tree) ||
      !aligned16(v_tree))
    return fail(ET_EINVAL, "%s: K/V buffers must be 16-byte aligned", fn);
  et::Plan& p = *as_plan(plan);
  const hipStream_t st = (hipStream_t)stream;
  if (p.debug) {
    std::vector<int32_t> al;
    int rc = debug_prefix(p, fn, prefix_len, st);
    if (rc == ET_OK) rc = d2h(fn, al, accept_len, p.B, st);
    if (rc != ET_OK) return rc;
    for (int b = 0; b < p.B; ++b)
      if (al[b] < 0 || al[b] > p.D)
        return fail(ET_EINVAL, "%s: accept_len[%d] = %d outside 0..%d", fn, b, al[b], p.D);
  }
  int rc = hip_status(
      et::launch_kv_commit(p, k_cache, v_cache, k_tree, v_tree, prefix_len,
                           path_slots, accept_len, st),
      fn);
  if (rc == ET_OK && p.debug) rc = debug_sync(fn, st);
  return rc;
}

int et_pool_export(et_plan_t plan, const void* ws, int32_t* token,
                   int32_t* parent, int32_t* depth, float* conf, float* value,
                   int32_t* pool_count, int32_t* frontier,
                   int32_t* frontier_count, et_stream_t stream) {
  const char* fn = "et_pool_export";
  CHECK_PTR(plan);
  CHECK_PTR(ws);
  et::Plan& p = *as_plan(plan);
  return hip_status(
      et::launch_pool_export(p, et::draft_ws(p, const_cast<void*>(ws)), token,
                             parent, depth, conf, value, pool_count, frontier,
                             frontier_count, (hipStream_t)stream),
      fn);
}

}  // extern "C"
