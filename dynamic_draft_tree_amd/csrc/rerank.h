// rerank.h -- the selection, output and flatten stages of the rerank,
// shared by the rerank kernel and the last draft step's merge.
//
// EAGLE-2 summary page, s4.2 (reranking phase): after expansion all draft
// tokens are reranked and the top ones by value are verified, flattened
// into one sequence whose attention mask keeps branches apart; explainer
// "EAGLE-2: Dynamic Draft Trees": a node's ancestors always outscore it, so
// the kept set is a connected tree; EAGLE notes, "EAGLE 2 / 方法", ReRank
// stage: on equal values the shallower node is kept first.
//
// Pool keys (value, -depth, -token, -index) order the nodes totally.  A
// parent's key exceeds its child's key (value(child) = value(parent) * conf
// <= value(parent), and equal values fall back to the shallower depth), so
// rank order is topological.  Selection of the n = min(N, pool) largest
// keys is a radix select from the top: a 256-bucket histogram of the next
// 8 key bits, restricted to the keys that share the prefix chosen so far,
// picks the bucket where the count from the top first reaches n.  Levels
// continue until at most max(128, n + 64) keys lie at or above the prefix
// (usually two: value exponent, then leading mantissa bits).  Keys are
// distinct (the index field), so the eighth level leaves exactly n.  The
// survivors are ranked by counting in LDS, each by a group of lanes that
// split the list.
#pragma once

#include "device.h"
#include "internal.h"

namespace et {

constexpr int kRerankMaxPool = 4096;
constexpr int kRerankPer = 4;     // pool nodes per thread (nt * 4 >= capacity)
constexpr int kRerankCand = 512;  // >= max(128, n + 64) for n <= 255

// LDS of one rerank (declared by the calling kernel).
struct RerankLds {
  uint64_t cand[kRerankCand];
  int16_t slot[kRerankMaxPool];
  int16_t ps[256];  // parent slot of each slot
  uint32_t hist[256];
  int pick, above, count;
};

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

// The rerank of sequence b by a block of nt threads (nt a multiple of 64,
// nt * RP >= every pool index, RP <= kRerankPer).  Thread tid holds pool nodes
// tid + nt * i: their keys (0 for no node), parent pool indexes and conf.
// Writes the kept tree (slot 0 the root token, slots 1..n in rank order,
// pads) and, with MASK, each slot's ancestor mask, depth and position id
// (pre + depth).  Every thread of the block calls it.  Its barriers order
// LDS data only (lds_barrier: no wait for the block's global stores, such
// as a merge's pool stores before it or the output stores before the
// flatten).
template <bool MASK, int RP>
__device__ __forceinline__ void rerank_block(const RerankOut& o, RerankLds& L, int b, int nt,
                                             const uint64_t (&key)[RP], const int (&par)[RP],
                                             const float (&cnf)[RP], int n, int root,
                                             int pre) {
  static_assert(RP >= 1 && RP <= kRerankPer, "pool nodes per thread");
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < RP; ++i)
    if (tid + nt * i < kRerankMaxPool) L.slot[tid + nt * i] = -1;
  if (tid == 0) L.count = 0;
  uint64_t prefix = 0;  // chosen high key bits, right-aligned
  int above = 0;        // keys strictly above the chosen prefix
  int cnt = 0;          // keys at or above it
  int shift = 64;
  for (int level = 0; level < 8 && n > 0; ++level) {
    for (int h = tid; h < 256; h += nt) L.hist[h] = 0;
    lds_barrier();
    const int sh = shift - 8;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const bool in = key[i] != 0 && (level == 0 || (key[i] >> shift) == prefix);
      if (in) atomicAdd(&L.hist[(key[i] >> sh) & 0xFFu], 1u);
    }
    lds_barrier();
    if (tid < 64) {
      int c, ab;
      suffix_pick(L.hist, n - above, &c, &ab);
      if (tid == 0) {
        L.pick = c;
        L.above = ab;
      }
    }
    lds_barrier();
    const int c = L.pick;
    prefix = (prefix << 8) | (uint64_t)c;
    above += L.above;
    cnt = above + (int)L.hist[c];
    shift = sh;
    lds_barrier();  // hist and pick are rewritten by the next level
    if (cnt <= max(128, n + 64)) break;
  }
  const uint64_t T = prefix << shift;
  const int64_t ob = (int64_t)b * o.T;
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < RP; ++i)
      if (key[i] != 0 && key[i] >= T) L.cand[atomicAdd(&L.count, 1)] = key[i];
    lds_barrier();
    // g consecutive lanes rank one candidate, each counting every g-th key
    // of the list; a butterfly over the group adds the counts.  The group
    // shares its loop trip count, so all its lanes take part in the sums.
    const int g = cnt <= 64 ? 16 : cnt <= 128 ? 8 : cnt <= 256 ? 4 : 2;
    const int part = tid & (g - 1);
    for (int t = tid / g; t < cnt; t += nt / g) {
      const uint64_t me = L.cand[t];
      int rank = 0;
      for (int j = part; j < cnt; j += g) rank += L.cand[j] > me ? 1 : 0;
      for (int q = 1; q < g; q <<= 1) rank += __shfl_xor(rank, q);
      if (part == 0 && rank < n) L.slot[pool_index_of(me)] = (int16_t)(rank + 1);
    }
  }
  lds_barrier();
  // kept nodes: slot = rank + 1, written by the thread that holds the node
  // (token and value come back out of the key, which holds both exactly)
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const int s = key[i] != 0 ? L.slot[tid + nt * i] : -1;
    if (s > 0) {
      const int ps = par[i] < 0 ? 0 : L.slot[par[i]];
      o.tokens[ob + s] = pool_token_of(key[i]);
      o.parent_slot[ob + s] = ps;
      o.conf[ob + s] = cnf[i];
      o.value[ob + s] = pool_value_of(key[i]);
      if (MASK) L.ps[s] = (int16_t)ps;
    }
  }
  // the root and the pad slots
  for (int s = tid; s < o.T; s += nt) {
    if (s != 0 && s <= n) continue;
    o.tokens[ob + s] = s == 0 ? root : -1;
    o.parent_slot[ob + s] = -1;
    o.conf[ob + s] = s == 0 ? 1.f : 0.f;
    o.value[ob + s] = s == 0 ? 1.f : 0.f;
  }
  if (tid == 0) o.n_kept[b] = n;
  if constexpr (MASK) {
    // Flatten: slot s <= n walks its parent slots (each smaller than its
    // own, so the walk ends at the root within s steps), setting one mask
    // bit per slot on its path.
    if (tid == 0) L.ps[0] = -1;
    lds_barrier();
    for (int s = tid; s < o.T; s += nt) {
      const int64_t oo = ob + s;
      uint64_t bits[4] = {0, 0, 0, 0};
      int d = -1, p = -1;
      if (s <= n) {
        int cur = s;
        d = 0;
        for (int guard = 0; guard < o.T; ++guard) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if ((cur >> 6) == w) bits[w] |= 1ull << (cur & 63);
          if (cur <= 0) break;
          cur = L.ps[cur];
          ++d;
        }
        p = pre + d;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < o.W) o.mask[oo * o.W + w] = bits[w];
      o.depth[oo] = d;
      o.pos[oo] = p;
    }
  }
}

}  // namespace et
