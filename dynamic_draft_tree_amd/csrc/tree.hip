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

namespace et {

constexpr int kRerankThreads = 1024;
constexpr int kRerankMaxPool = 4096;

struct RerankArgs {
  DraftWs ws;
  int32_t* tokens;
  int32_t* parent_slot;
  float* conf;
  float* value;
  int32_t* n_kept;
  int B, N, T, cap;
};

// One block per sequence.  Pool keys (value, -depth, -token, -index) are
// sorted descending in LDS with a bitonic network; the first n = min(N,
// pool) ranks become slots 1..n.  A parent's key exceeds its child's key
// (value(child) = value(parent) * conf <= value(parent), and equal values
// fall back to the shallower depth), so rank order is topological.
__global__ __launch_bounds__(kRerankThreads) void rerank_kernel(RerankArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ uint64_t s_key[kRerankMaxPool];
  __shared__ int16_t s_slot[kRerankMaxPool];
  const int64_t pb = (int64_t)b * a.cap;
  const int P = a.ws.pool_count[b];
  int Pp = 2;
  while (Pp < P) Pp <<= 1;
  for (int i = tid; i < Pp; i += kRerankThreads) {
    uint64_t key = 0;
    if (i < P)
      key = pool_key(a.ws.pool_value[pb + i], a.ws.pool_depth[pb + i],
                     a.ws.pool_token[pb + i], i);
    s_key[i] = key;
    s_slot[i] = -1;
  }
  __syncthreads();
  for (int k = 2; k <= Pp; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < Pp; i += kRerankThreads) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = s_key[i], y = s_key[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            s_key[i] = y;
            s_key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  const int n = P < a.N ? P : a.N;
  for (int r = tid; r < n; r += kRerankThreads)
    s_slot[pool_index_of(s_key[r])] = (int16_t)(r + 1);
  __syncthreads();
  const int64_t ob = (int64_t)b * a.T;
  for (int s = tid; s < a.T; s += kRerankThreads) {
    int tok = -1, ps = -1;
    float cf = 0.f, vl = 0.f;
    if (s == 0) {
      tok = a.ws.root_token[b];
      cf = 1.f;
      vl = 1.f;
    } else if (s <= n) {
      int idx = pool_index_of(s_key[s - 1]);
      int par = a.ws.pool_parent[pb + idx];
      tok = a.ws.pool_token[pb + idx];
      ps = par < 0 ? 0 : s_slot[par];
      cf = a.ws.pool_conf[pb + idx];
      vl = a.ws.pool_value[pb + idx];
    }
    a.tokens[ob + s] = tok;
    a.parent_slot[ob + s] = ps;
    a.conf[ob + s] = cf;
    a.value[ob + s] = vl;
  }
  if (tid == 0) a.n_kept[b] = n;
}

hipError_t launch_rerank(const Plan& p, const DraftWs& w, int32_t* tokens,
                         int32_t* parent_slot, float* conf, float* value,
                         int32_t* n_kept, hipStream_t s) {
  RerankArgs a;
  a.ws = w;
  a.tokens = tokens;
  a.parent_slot = parent_slot;
  a.conf = conf;
  a.value = value;
  a.n_kept = n_kept;
  a.B = p.B;
  a.N = p.N;
  a.T = p.T;
  a.cap = p.cap;
  rerank_kernel<<<p.B, kRerankThreads, 0, s>>>(a);
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

__global__ void clear_u32_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_clear_u32(uint32_t* p, size_t n, hipStream_t s) {
  int blocks = (int)((n + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  clear_u32_kernel<<<blocks, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace et
