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
  // flatten outputs (the fused form only)
  const int32_t* prefix_len;
  uint64_t* mask;
  int32_t* depth;
  int32_t* pos;
  int B, N, T, W, cap;
};

// One block per sequence.  Pool keys (value, -depth, -token, -index) order
// the nodes totally.  A parent's key exceeds its child's key (value(child)
// = value(parent) * conf <= value(parent), and equal values fall back to
// the shallower depth), so rank order is topological.
//
// Selection of the n = min(N, pool) largest keys is a radix select from
// the top: a 256-bucket histogram of the next 8 key bits, restricted to
// the keys that share the prefix chosen so far, picks the bucket where the
// count from the top first reaches n.  Levels continue until at most
// max(128, n + 64) keys lie at or above the prefix (usually two: value
// exponent, then leading mantissa bits).  Keys are distinct (the index
// field), so the eighth level leaves exactly n.  The survivors are ranked
// by counting in LDS, each by a group of lanes that split the list.
constexpr int kRerankCand = 512;  // >= max(128, n + 64) for n <= 255

// Wave 0: find the largest bucket c of hist[0..255] whose suffix count
// (sum of hist[c..255]) reaches `need`; returns c and the count above c.
__device__ __forceinline__ void suffix_pick(const uint32_t* hist, int need,
                                            int* bucket, int* above) {
  const int lane = threadIdx.x & 63;
  uint32_t h[4];
  // lane l holds buckets 255 - 4l - q (q = 0..3): descending order
#pragma unroll
  for (int q = 0; q < 4; ++q) h[q] = hist[255 - 4 * lane - q];
  const uint32_t mine = h[0] + h[1] + h[2] + h[3];
  // inclusive prefix over lanes (lane 0 = highest buckets)
  uint32_t inc = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  uint32_t run = inc - mine;  // count strictly above this lane's buckets
  int found = -1, ab = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (found < 0 && run + h[q] >= (uint32_t)need) {
      found = 255 - 4 * lane - q;
      ab = (int)run;
    }
    run += h[q];
  }
  // the first lane (highest buckets) that reaches `need` holds the answer
  const uint64_t bal = __ballot(found >= 0);
  const int src = bal ? (int)__ffsll((unsigned long long)bal) - 1 : 0;
  *bucket = __shfl(found, src);
  *above = __shfl(ab, src);
}

// MASK: also flatten the kept tree (the tree-mask outputs), from the
// parent slots held in LDS, in the same launch.
template <bool MASK>
__global__ __launch_bounds__(kRerankThreads) void rerank_kernel(RerankArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ uint64_t s_cand[kRerankCand];
  __shared__ int16_t s_slot[kRerankMaxPool];
  __shared__ int16_t s_ps[MASK ? 256 : 1];  // parent slot of each slot
  __shared__ uint32_t s_hist[256];
  __shared__ int s_pick, s_above, s_count;
  const int64_t pb = (int64_t)b * a.cap;
  const int P = a.ws.pool_count[b];
  const int n = P < a.N ? P : a.N;
  const int pre = MASK ? a.prefix_len[b] : 0;
  constexpr int PER = kRerankMaxPool / kRerankThreads;
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
  uint64_t key[PER];
  int par[PER], dep[PER], tok[PER];
  float cnf[PER], val[PER];
  const int root = a.ws.root_token[b];
  const int rounds = (a.cap + kRerankThreads - 1) / kRerankThreads;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
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
    s_slot[idx] = -1;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    asm volatile("" : "+v"(val[i]), "+v"(dep[i]), "+v"(tok[i]), "+v"(par[i]), "+v"(cnf[i]));
    const int idx = tid + kRerankThreads * i;
    key[i] = idx < P ? pool_key(val[i], dep[i], tok[i], idx) : 0;
  }
  if (tid == 0) s_count = 0;
  uint64_t prefix = 0;  // chosen high key bits, right-aligned
  int above = 0;        // keys strictly above the chosen prefix
  int cnt = 0;          // keys at or above it
  int shift = 64;
  for (int level = 0; level < 8 && n > 0; ++level) {
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
    const int sh = shift - 8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = key[i] != 0 && (level == 0 || (key[i] >> shift) == prefix);
      if (in) atomicAdd(&s_hist[(key[i] >> sh) & 0xFFu], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      int c, ab;
      suffix_pick(s_hist, n - above, &c, &ab);
      if (tid == 0) {
        s_pick = c;
        s_above = ab;
      }
    }
    __syncthreads();
    const int c = s_pick;
    prefix = (prefix << 8) | (uint64_t)c;
    above += s_above;
    cnt = above + (int)s_hist[c];
    shift = sh;
    __syncthreads();  // s_hist and s_pick are rewritten by the next level
    if (cnt <= max(128, n + 64)) break;
  }
  const uint64_t T = prefix << shift;
  const int64_t ob = (int64_t)b * a.T;
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (key[i] != 0 && key[i] >= T) s_cand[atomicAdd(&s_count, 1)] = key[i];
    __syncthreads();
    // g consecutive lanes rank one candidate, each counting every g-th key
    // of the list; a butterfly over the group adds the counts.  The group
    // shares its loop trip count, so all its lanes take part in the sums.
    const int g = cnt <= 64 ? 16 : cnt <= 128 ? 8 : cnt <= 256 ? 4 : 2;
    const int part = tid & (g - 1);
    for (int t = tid / g; t < cnt; t += kRerankThreads / g) {
      const uint64_t me = s_cand[t];
      int rank = 0;
      for (int j = part; j < cnt; j += g) rank += s_cand[j] > me ? 1 : 0;
      for (int o = 1; o < g; o <<= 1) rank += __shfl_xor(rank, o);
      if (part == 0 && rank < n) s_slot[pool_index_of(me)] = (int16_t)(rank + 1);
    }
  }
  __syncthreads();
  // kept nodes: slot = rank + 1, written by the thread that holds the node
  // (token and value come back out of the key, which holds both exactly)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + kRerankThreads * i;
    const int s = key[i] != 0 ? s_slot[idx] : -1;
    if (s > 0) {
      const int ps = par[i] < 0 ? 0 : s_slot[par[i]];
      a.tokens[ob + s] = pool_token_of(key[i]);
      a.parent_slot[ob + s] = ps;
      a.conf[ob + s] = cnf[i];
      a.value[ob + s] = pool_value_of(key[i]);
      if (MASK) s_ps[s] = (int16_t)ps;
    }
  }
  // the root and the pad slots
  for (int s = tid; s < a.T; s += kRerankThreads) {
    if (s != 0 && s <= n) continue;
    a.tokens[ob + s] = s == 0 ? root : -1;
    a.parent_slot[ob + s] = -1;
    a.conf[ob + s] = s == 0 ? 1.f : 0.f;
    a.value[ob + s] = s == 0 ? 1.f : 0.f;
  }
  if (tid == 0) a.n_kept[b] = n;
  if constexpr (MASK) {
    // Flatten: slot s <= n walks its parent slots (each smaller than its
    // own, so the walk ends at the root within s steps), setting one mask
    // bit per slot on its path.
    if (tid == 0) s_ps[0] = -1;
    __syncthreads();
    const int s = tid;
    if (s < a.T) {
      const int64_t o = ob + s;
      uint64_t bits[4] = {0, 0, 0, 0};
      int d = -1, p = -1;
      if (s <= n) {
        int cur = s;
        d = 0;
        for (int guard = 0; guard < a.T; ++guard) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if ((cur >> 6) == w) bits[w] |= 1ull << (cur & 63);
          if (cur <= 0) break;
          cur = s_ps[cur];
          ++d;
        }
        p = pre + d;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < a.W) a.mask[o * a.W + w] = bits[w];
      a.depth[o] = d;
      a.pos[o] = p;
    }
  }
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
  a.prefix_len = nullptr;
  a.mask = nullptr;
  a.depth = a.pos = nullptr;
  a.B = p.B;
  a.N = p.N;
  a.T = p.T;
  a.W = p.W;
  a.cap = p.cap;
  rerank_kernel<false><<<p.B, kRerankThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_rerank_mask(const Plan& p, const DraftWs& w, int32_t* tokens,
                              int32_t* parent_slot, float* conf, float* value,
                              int32_t* n_kept, const int32_t* prefix_len,
                              uint64_t* mask, int32_t* depth, int32_t* pos,
                              hipStream_t s) {
  RerankArgs a;
  a.ws = w;
  a.tokens = tokens;
  a.parent_slot = parent_slot;
  a.conf = conf;
  a.value = value;
  a.n_kept = n_kept;
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.depth = depth;
  a.pos = pos;
  a.B = p.B;
  a.N = p.N;
  a.T = p.T;
  a.W = p.W;
  a.cap = p.cap;
  rerank_kernel<true><<<p.B, kRerankThreads, 0, s>>>(a);
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
