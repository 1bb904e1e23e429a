// tree.hip -- rerank (global top-N of the pool) and the flattened tree mask.
//
// Rerank: EAGLE-2 summary page, s4.2 (reranking phase): after expansion
// all draft tokens are reranked and the top ones by value are verified;
// explainer "EAGLE-2: Dynamic Draft Trees": a node's ancestors always
// outscore it, so the kept set is a connected tree; EAGLE notes,
// "EAGLE 2 / 方法", ReRank stage: on equal values the shallower node is
// kept first.  Lower token id and then creation order complete the order.
//
// Mask: summary page s4.2: the kept tokens are flattened into one
// sequence whose attention mask keeps branches apart.  A slot sees itself
// and its ancestors.
#include "device.h"
#include "internal.h"
#include "rerank.h"

namespace et {

constexpr int kRerankThreads = 1024;

struct RerankArgs {
  DraftWs ws;
  int cap;
};

// One block per sequence.  MASK: also flatten the kept tree (the
// tree-mask outputs), from the parent slots held in LDS, in the same launch.
template <bool MASK>
__global__ __launch_bounds__(kRerankThreads) void rerank_kernel(RerankArgs a, RerankOut o) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ RerankLds L;
  const int64_t pb = (int64_t)b * a.cap;
  const int P = a.ws.pool_count[b];
  const int n = P < o.N ? P : o.N;
  const int pre = MASK ? o.prefix_len[b] : 0;
  // Each thread keeps its nodes' fields in registers: the kept ones are
  // written out by their owner once the ranks are known, with no second
  // round of pool loads.  The loads cover the whole capacity (cap <=
  // kRerankMaxPool, all of it readable) and go out together with the pool
  // size's; entries at or past the size are dropped once it arrives.
  // (Loads in rounds of the block size, as many as the capacity needs; the
  // index is clamped rather than guarded so that no branch splits them,
  // and the values pass through an empty asm after the last load is
  // issued, so that nothing computed from them is scheduled between the
  // loads, each such use being a wait for the memory round trip.)
  uint64_t key[kRerankPer];
  int par[kRerankPer], dep[kRerankPer], tok[kRerankPer];
  float cnf[kRerankPer], val[kRerankPer];
  const int root = a.ws.root_token[b];
  const int rounds = (a.cap + kRerankThreads - 1) / kRerankThreads;
#pragma unroll
  for (int i = 0; i < kRerankPer; ++i) {
    const int idx = tid + kRerankThreads * i;
    val[i] = cnf[i] = 0.f;
    par[i] = dep[i] = tok[i] = -1;
    if (i < rounds) {  // uniform
      const int64_t g = pb + min(idx, a.cap - 1);
      val[i] = a.ws.pool_value[g];
      dep[i] = a.ws.pool_depth[g];
      tok[i] = a.ws.pool_token[g];
      par[i] = a.ws.pool_parent[g];
      cnf[i] = a.ws.pool_conf[g];
    }
  }
#pragma unroll
  for (int i = 0; i < kRerankPer; ++i) {
    asm volatile("" : "+v"(val[i]), "+v"(dep[i]), "+v"(tok[i]), "+v"(par[i]), "+v"(cnf[i]));
    const int idx = tid + kRerankThreads * i;
    key[i] = idx < P ? pool_key(val[i], dep[i], tok[i], idx) : 0;
  }
  rerank_block<MASK, kRerankPer>(o, L, b, kRerankThreads, key, par, cnf, n, root, pre);
}

RerankOut rerank_out(const Plan& p, int32_t* tokens, int32_t* parent_slot, float* conf,
                     float* value, int32_t* n_kept, const int32_t* prefix_len, uint64_t* mask,
                     int32_t* depth, int32_t* pos) {
  RerankOut o;
  o.tokens = tokens;
  o.parent_slot = parent_slot;
  o.conf = conf;
  o.value = value;
  o.n_kept = n_kept;
  o.prefix_len = prefix_len;
  o.mask = mask;
  o.depth = depth;
  o.pos = pos;
  o.N = p.N;
  o.T = p.T;
  o.W = p.W;
  return o;
}

hipError_t launch_rerank(const Plan& p, const DraftWs& w, int32_t* tokens,
                         int32_t* parent_slot, float* conf, float* value,
                         int32_t* n_kept, hipStream_t s) {
  RerankArgs a;
  a.ws = w;
  a.cap = p.cap;
  rerank_kernel<false><<<p.B, kRerankThreads, 0, s>>>(
      a, rerank_out(p, tokens, parent_slot, conf, value, n_kept, nullptr, nullptr, nullptr,
                    nullptr));
  return hipGetLastError();
}

hipError_t launch_rerank_mask(const Plan& p, const DraftWs& w, int32_t* tokens,
                              int32_t* parent_slot, float* conf, float* value,
                              int32_t* n_kept, const int32_t* prefix_len,
                              uint64_t* mask, int32_t* depth, int32_t* pos,
                              hipStream_t s) {
  RerankArgs a;
  a.ws = w;
  a.cap = p.cap;
  rerank_kernel<true><<<p.B, kRerankThreads, 0, s>>>(
      a, rerank_out(p, tokens, parent_slot, conf, value, n_kept, prefix_len, mask, depth, pos));
  return hipGetLastError();
}

// Fixed-shape tree (the static baseline): slot s >= 1 is a given pool
// node with a given parent slot; one thread per slot gathers the node.
// Slot 0 is the root (value 1); slots past the shape are pads, as rerank
// writes them.
__global__ __launch_bounds__(256) void static_tree_kernel(
    DraftWs ws, FixedSlots fs, int32_t* tokens, int32_t* parent_slot,
    float* conf, float* value, int32_t* n_kept, int T, int cap) {
  const int b = blockIdx.x;
  for (int s = threadIdx.x; s < T; s += blockDim.x) {
    int tok = -1, par = -1;
    float c = 0.0f, v = 0.0f;
    if (s == 0) {
      tok = ws.root_token[b];
      c = v = 1.0f;
    } else if (s <= fs.m) {
      const int e = fs.slot[s];
      const int pi = min(e & 0xFFFF, cap - 1);
      const int64_t g = (int64_t)b * cap + pi;
      tok = ws.pool_token[g];
      par = e >> 16;
      c = ws.pool_conf[g];
      v = ws.pool_value[g];
    }
    const int64_t o = (int64_t)b * T + s;
    tokens[o] = tok;
    parent_slot[o] = par;
    conf[o] = c;
    value[o] = v;
  }
  if (threadIdx.x == 0) n_kept[b] = fs.m;
}

hipError_t launch_static_tree(const Plan& p, const DraftWs& w, const FixedSlots& fs,
                              int32_t* tokens, int32_t* parent_slot, float* conf,
                              float* value, int32_t* n_kept, hipStream_t s) {
  static_tree_kernel<<<p.B, 256, 0, s>>>(w, fs, tokens, parent_slot, conf, value,
                                         n_kept, p.T, p.cap);
  return hipGetLastError();
}

// One thread per slot: walk the parent pointers (staged in LDS) to the root.
__global__ __launch_bounds__(256) void tree_mask_kernel(
    const int32_t* parent_slot, const int32_t* n_kept,
    const int32_t* prefix_len, uint64_t* mask, int32_t* depth, int32_t* pos,
    int T, int W) {
  __shared__ int16_t s_par[256];
  const int b = blockIdx.x, s = threadIdx.x;
  const int n = n_kept[b];
  const int pre = prefix_len[b];
  if (s < T) s_par[s] = (int16_t)parent_slot[(int64_t)b * T + s];
  __syncthreads();
  if (s >= T) return;
  const int64_t o = (int64_t)b * T + s;
  uint64_t bits[4] = {0, 0, 0, 0};
  int d = -1, p = -1;
  if (s <= n) {
    int cur = s;
    d = 0;
    for (int guard = 0; guard < T; ++guard) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if ((cur >> 6) == w) bits[w] |= 1ull << (cur & 63);
      if (cur <= 0) break;
      cur = s_par[cur];
      ++d;
    }
    p = pre + d;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w < W) mask[o * W + w] = bits[w];
  depth[o] = d;
  pos[o] = p;
}

hipError_t launch_tree_mask(const Plan& p, const int32_t* parent_slot,
                            const int32_t* n_kept, const int32_t* prefix_len,
                            uint64_t* mask, int32_t* depth, int32_t* pos,
                            hipStream_t s) {
  tree_mask_kernel<<<p.B, 256, 0, s>>>(parent_slot, n_kept, prefix_len, mask,
                                       depth, pos, p.T, p.W);
  return hipGetLastError();
}

// Inspection copy of the pool and the frontier the next step reads.
__global__ void pool_export_kernel(DraftWs w, int B, int cap, int k,
                                   int parity, int32_t* token, int32_t* parent,
                                   int32_t* depth, float* conf, float* value,
                                   int32_t* pool_count, int32_t* frontier,
                                   int32_t* frontier_count) {
  const int64_t n = (int64_t)B * cap;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (token) token[i] = w.pool_token[i];
    if (parent) parent[i] = w.pool_parent[i];
    if (depth) depth[i] = w.pool_depth[i];
    if (conf) conf[i] = w.pool_conf[i];
    if (value) value[i] = w.pool_value[i];
    if (i < B) {
      if (pool_count) pool_count[i] = w.pool_count[i];
      if (frontier_count) frontier_count[i] = w.frontier_count[parity * B + i];
    }
    if (i < (int64_t)B * k && frontier) frontier[i] = w.frontier[parity * B * k + i];
  }
}

hipError_t launch_pool_export(const Plan& p, const DraftWs& w, int32_t* token,
                              int32_t* parent, int32_t* depth, float* conf,
                              float* value, int32_t* pool_count,
                              int32_t* frontier, int32_t* frontier_count,
                              hipStream_t s) {
  int parity = p.last_step & 1;
  int64_t n = (int64_t)p.B * p.cap;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  pool_export_kernel<<<blocks, 256, 0, s>>>(w, p.B, p.cap, p.k, parity, token,
                                            parent, depth, conf, value,
                                            pool_count, frontier,
                                            frontier_count);
  return hipGetLastError();
}

}  // namespace et
