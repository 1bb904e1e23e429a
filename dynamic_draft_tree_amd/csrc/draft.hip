// draft.hip -- one expansion layer of the dynamic draft tree.
//
// EAGLE-2 summary page, s4.1 (expansion phase): the draft model's softmax
// confidence stands in for a token's acceptance rate, a node's value is
// the product of confidences on its root path, and the k most valuable
// nodes of the current layer are expanded.  Explainer "EAGLE-2: Dynamic
// Draft Trees", value equation.  EAGLE notes, "EAGLE 2 / 方法", Expand
// stage: nodes whose value is below the threshold are not expanded.
//
// One launch per step.  Grid (S chunks, k frontier rows, B sequences),
// 256 threads.  Each block streams one chunk of one logits row with
// 16-byte loads and publishes the chunk's (max, sum of exp) and its top-k
// logit keys.  The last block of a sequence to finish (one arrival
// ticket over all F x S blocks) merges every row of that sequence, turns
// the rows into children (conf, value), appends them to the pool and
// selects the next frontier.  No host sync, no second launch.
#include "device.h"
#include "internal.h"

namespace et {

struct DraftArgs {
  DraftWs ws;
  const void* logits;
  int64_t bstride, rstride;
  const int32_t* root_tokens;
  int32_t* next_tokens;
  int32_t* next_count;
  int B, V, k, D, S, step, cap;
  float thr;
};

constexpr int kWaves = kScanThreads / 64;  // waves per scan block
constexpr int kWaveCap = 64;             // candidate slots per wave
constexpr int kStage = 4;                // keys per chunk list read up front
constexpr int kRowCap = 64;              // merge candidates per row

// The k-th largest of the wave's 64 keys (k <= 64): the largest T whose
// count of keys >= T is at least k, built bit by bit from the top (bits
// below `lo` are known to be zero in every key).  One compare and one
// ballot per bit, no data exchange.
__device__ __forceinline__ uint32_t wave_kth_largest_u32(uint32_t key, int k, int lo) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    if (bit < lo) break;
    const uint32_t cand = t | (1u << bit);
    if (__popcll(__ballot(key >= cand)) >= k) t = cand;
  }
  return t;
}
// The same over float values through their order-preserving image; values
// from bf16 have 16 significant bits.  (For negative bf16 values the image
// has ones in its low bits, so the result can sit slightly below the exact
// k-th largest: still a lower bound.)
template <bool BF16>
__device__ __forceinline__ float wave_kth_largest(float v, int k) {
  return unordered_f32(wave_kth_largest_u32(ordered_f32(v), k, BF16 ? 16 : 0));
}

// Smallest logit key whose logit is >= x.
__device__ __forceinline__ uint64_t key_floor(float x) {
  return (uint64_t)ordered_f32(x) << 32;
}

template <bool BF16, bool VEC, int E>
__global__ __launch_bounds__(256) void draft_step_kernel(DraftArgs a) {
  constexpr int NT = kScanThreads;
  constexpr int kChunkE = NT * E;
  constexpr float kLog2e = 1.4426950408889634f;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k, S = a.S;
  __shared__ __attribute__((aligned(16))) float s_x[kScanThreads * E];  // lane values
  __shared__ uint64_t s_wl[kWaves * kWaveCap];  // wave candidate lists
  __shared__ uint64_t s_bc[kWaves * kWaveCap];  // block candidates
  __shared__ float s_wf[3][kWaves];             // wave bound, max, sum
  __shared__ int s_wcnt[kWaves];
  __shared__ int s_count;
  __shared__ int s_flag;
  // merge (last block of the sequence)
  __shared__ uint64_t s_rc[kMaxTopk * kRowCap];   // row candidates
  __shared__ uint64_t s_rk[kMaxTopk * kMaxTopk];  // row top-k keys
  __shared__ uint64_t s_aux[256];

  const int prev = (a.step - 1) & 1, cur = a.step & 1;
  if (a.step == 1 && j > 0) return;  // the root is the only row of step 1
  // The chunk's loads are issued before the frontier count arrives (every
  // row j < topk is readable memory by contract; rows j >= F are dropped
  // below), so the count's latency hides behind the logits'.
  const int64_t esz = BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + (b * a.bstride + j * a.rstride) * esz;
  const int base = c * kChunkE;
  float x[E];
  load_chunk<BF16, VEC, E>(row, base, a.V, tid, x);
  const int F = a.step == 1 ? 1 : a.ws.frontier_count[prev * a.B + b];
  // phase: frontier count read
  if (F == 0) {
    // The tree stopped growing earlier: no rows, empty next frontier.
    if (c == 0 && j == 0) {
      if (tid < k) a.next_tokens[(int64_t)b * k + tid] = -1;
      if (tid == 0) {
        a.next_count[b] = 0;
        a.ws.frontier_count[cur * a.B + b] = 0;
      }
    }
    return;
  }
  if (j >= F) return;

  // ---- one chunk: per wave max, sum of exp and candidates ----------------
  if (tid == 0) s_count = 0;
  // phase: chunk loaded

  // Lane max as a pairwise tree (short dependency chain).
  float mx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) mx[e] = x[e];
#pragma unroll
  for (int w = E / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < w; ++e) mx[e] = fmaxf(mx[e], mx[e + w]);
  const float lmax = mx[0];
  const float mw = wave_max_f32(lmax);
  float sl = 0.f;
  if (mw > -INFINITY) {
    // exp(x - m) = 2^(x log2 e - m log2 e): one FMA and v_exp_f32; four
    // accumulators keep the add chain short.
    const float off = mw * kLog2e;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < E; ++e)
      acc[e & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2e, -off));
    sl = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  const float sw = wave_sum_f32(sl);
  // phase: max and sum of exp
  // The wave's k-th largest lane maximum Lw bounds its k-th largest
  // element from below (those k maxima are k distinct elements), so every
  // element of the wave's top-k is >= Lw.  Each lane marks its elements
  // >= Lw in a bit mask; a wave prefix sum of the counts gives each lane
  // its slots, and the lane writes its (usually zero to two) candidates.
  const float Lw = wave_kth_largest<BF16>(lmax, k);
  // phase: wave threshold
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int id = base + elem_off<BF16>(e, tid);
    bits |= (id < a.V && x[e] >= Lw) ? (1u << e) : 0u;
  }
  int wtot;
  int o = wave_excl_prefix_small(__popc(bits), &wtot);
  uint64_t* wl = &s_wl[wave * kWaveCap];
  if (wtot <= kWaveCap) {
    // The lane's values are staged in LDS so that each candidate is read
    // by index (a register array cannot be indexed at run time cheaply).
    // Layout: 16-byte group q of every lane in one contiguous row of the
    // block, so each group's store is free of bank conflicts.
#pragma unroll
    for (int q = 0; q < E / 4; ++q)
      *(float4*)&s_x[(q * kScanThreads + tid) * 4] =
          make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
    while (bits) {
      const int e = __ffs(bits) - 1;
      bits &= bits - 1;
      wl[o++] = logit_key(s_x[((e >> 2) * kScanThreads + tid) * 4 + (e & 3)],
                          (uint32_t)(base + elem_off<BF16>(e, tid)));
    }
  } else {
    // Many equal logits: the wave's exact top-k, by k rounds of maximum.
    uint64_t prevk = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int id = base + elem_off<BF16>(e, tid);
        const uint64_t key = id < a.V ? logit_key(x[e], (uint32_t)id) : 0;
        if (key < prevk && key > best) best = key;
      }
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) wl[r] = w;
      prevk = w;
    }
    wtot = k;
  }
  if (lane == 0) {
    s_wcnt[wave] = wtot;
    s_wf[0][wave] = Lw;
    s_wf[1][wave] = mw;
    s_wf[2][wave] = sw;
  }
  __syncthreads();
  // phase: wave candidates
  // Block: the largest wave bound bounds the block's k-th largest element
  // from below; the candidates at or above it are ranked by counting.
  float Lb = s_wf[0][0], mb = s_wf[1][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    Lb = fmaxf(Lb, s_wf[0][w]);
    mb = fmaxf(mb, s_wf[1][w]);
  }
  {
    const int w = tid / kWaveCap, i = tid - w * kWaveCap;
    if (i < s_wcnt[w]) {
      const uint64_t v = s_wl[tid];
      if (v != 0 && v >= key_floor(Lb)) s_bc[atomicAdd(&s_count, 1)] = v;
    }
  }
  __syncthreads();
  const int nb = s_count;
  const int64_t rowid = (int64_t)b * k + j;
  const int64_t pe = rowid * S + c;  // this block's partial entry
  uint64_t* dst = &a.ws.part_keys[pe * kMaxTopk];
  for (int t = tid; t < nb; t += NT) {
    const uint64_t me = s_bc[t];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < nb; ++q) rank += s_bc[q] > me;
    if (rank < k) st_agent(&dst[rank], me);
  }
  if (tid >= nb && tid < k) st_agent(&dst[tid], (uint64_t)0);
  if (tid == 0) {
    float sb = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      sb += s_wf[1][w] > -INFINITY ? s_wf[2][w] * expf(s_wf[1][w] - mb) : 0.f;
    st_agent(&a.ws.part_m[pe], mb);
    st_agent(&a.ws.part_s[pe], sb);
  }
  // phase: partial published

  // ---- last block of this sequence: merge every row ---------------------
  if (!block_arrive_last(&a.ws.seq_ticket[b], (uint32_t)(F * S), &s_flag)) return;
  // phase: sequence ticket won
  // ---- row merges: a segment of SP lanes per row ------------------------
  // SP is the power of two >= S, so a wave merges 64 / SP rows at once and
  // lane q of a segment holds chunk q's (max, sum) and the first kStage
  // keys of its sorted list.  The row's max and sum of exp are segment
  // reductions.  Bound: with at least k chunks the k-th largest chunk head
  // bounds the row's k-th largest key from below, so only keys at or above
  // it (a prefix of every chunk's list) are ranked.
  const int64_t e0 = (int64_t)b * k * S;  // first partial of the sequence
  int SP = 1;
  while (SP < S) SP <<= 1;
  const int RW = 64 / SP;                 // rows per wave
  const int seg = lane / SP, q = lane - seg * SP;
  const uint64_t segmask = SP == 64 ? ~0ull : ((1ull << SP) - 1ull) << (seg * SP);
  const uint64_t below = segmask & ((1ull << lane) - 1ull);
  const int64_t pb = (int64_t)b * a.cap;
  const int P0 = a.step == 1 ? 0 : a.ws.pool_count[b];
  for (int r0 = 0; r0 < F; r0 += kWaves * RW) {
    const int jr = r0 + wave * RW + seg;
    const bool on = jr < F && q < S;
    // the row's parent: its frontier slot's pool index and value, both
    // stored by the previous step (no dependent load)
    const int64_t fs = ((int64_t)prev * a.B + b) * k + jr;
    const bool hp = a.step > 1 && jr < F;
    const int par = hp ? a.ws.frontier[fs] : -1;
    const float vpar = hp ? a.ws.frontier_val[fs] : 1.0f;
    const int64_t e = e0 + (int64_t)jr * S + q;
    const float pm = on ? ld_agent(&a.ws.part_m[e]) : -INFINITY;
    const float ps = on ? ld_agent(&a.ws.part_s[e]) : 0.f;
    uint64_t pk[kMaxTopk];
#pragma unroll
    for (int r = 0; r < kMaxTopk; ++r)
      pk[r] = (on && r < kStage && r < k) ? ld_agent(&a.ws.part_keys[e * kMaxTopk + r]) : 0;
    // phase: partials read
    float m = pm;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
      if (d < SP) m = fmaxf(m, xor_lane_rt(m, d));
    float sum = pm > -INFINITY ? ps * __builtin_amdgcn_exp2f((pm - m) * kLog2e) : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
      if (d < SP) sum += xor_lane_rt(sum, d);
    // phase: row max and sum
    // k-th largest head of the segment, bit by bit on the ordered logit
    uint64_t Lk = 0;
    if (S >= k) {
      const uint32_t hk = on && pk[0] != 0 ? (uint32_t)(pk[0] >> 32) : 0u;
      uint32_t t = 0;
#pragma unroll
      for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
        const uint32_t cand = t | (1u << bit);
        if (__popcll(__ballot(hk >= cand) & segmask) >= k) t = cand;
      }
      Lk = (uint64_t)t << 32;
    }
    // phase: row bound
    int cq = 0;
#pragma unroll
    for (int r = 0; r < kStage; ++r) cq += (pk[r] != 0 && pk[r] >= Lk) ? 1 : 0;
    if (__ballot(cq == kStage && k > kStage) != 0ull) {
      // rare: a list qualifies beyond its staged keys
      if (cq == kStage) {
#pragma unroll
        for (int r = kStage; r < kMaxTopk; ++r)
          if (r < k) pk[r] = ld_agent(&a.ws.part_keys[e * kMaxTopk + r]);
#pragma unroll
        for (int r = kStage; r < kMaxTopk; ++r)
          cq += (r < k && pk[r] != 0 && pk[r] >= Lk) ? 1 : 0;
      }
    }
    // segment prefix sum and total of cq (<= 16), one ballot per bit
    int off = 0, n = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
      const uint64_t bm = __ballot((cq >> bit) & 1);
      off += __popcll(bm & below) << bit;
      n += __popcll(bm & segmask) << bit;
    }
    // phase: row prefix
    const bool fits = n <= kRowCap;
    if (jr < F) {
      uint64_t* lst = &s_rc[jr * kRowCap];
      if (fits) {
#pragma unroll
        for (int r = 0; r < kMaxTopk; ++r)
          if (r < cq) lst[off + r] = pk[r];
      }
    }
    wave_lds_sync();
    // phase: row list written
    if (jr < F && fits) {
      const uint64_t* lst = &s_rc[jr * kRowCap];
      for (int i = q; i < n; i += SP) {
        const uint64_t me = lst[i];
        int rank = 0;
#pragma unroll 8
        for (int t = 0; t < n; ++t) rank += lst[t] > me;
        if (rank < k) s_rk[jr * kMaxTopk + rank] = me;
      }
    }
    // phase: row ranked
    // Many equal logits overflow a row's list: that row takes k rounds of
    // maximum over all of its chunk lists, with the whole wave.
    for (int sg = 0; sg < RW; ++sg) {
      const int jo = r0 + wave * RW + sg;
      if (jo >= F) break;
      if ((__ballot(!fits) & (SP == 64 ? ~0ull : ((1ull << SP) - 1ull) << (sg * SP))) == 0ull)
        continue;
      uint64_t prevk = ~0ull;
      for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
        for (int t = lane; t < S * k; t += 64) {
          const uint64_t v = ld_agent(&a.ws.part_keys[(e0 + (int64_t)jo * S + t / k) * kMaxTopk + t % k]);
          if (v < prevk && v > best) best = v;
        }
        const uint64_t w = wave_max_u64(best);
        if (lane == 0) s_rk[jo * kMaxTopk + r] = w;
        prevk = w;
      }
    }
    wave_lds_sync();
    // phase: row merged
    // Children of the row, in rank order (conf decreasing): child r of row
    // jr is pool node P0 + jr * k + r.
    if (jr < F) {
      for (int r = q; r < k; r += SP) {
        const uint64_t key = s_rk[jr * kMaxTopk + r];
        const int tok = (int)id_of(key);
        const float conf = __builtin_amdgcn_exp2f((logit_of(key) - m) * kLog2e) / sum;
        const float val = __fmul_rn(vpar, conf);
        const int ci = jr * k + r, pi = P0 + ci;
        a.ws.pool_token[pb + pi] = tok;
        a.ws.pool_parent[pb + pi] = par;
        a.ws.pool_depth[pb + pi] = a.step;
        a.ws.pool_conf[pb + pi] = conf;
        a.ws.pool_value[pb + pi] = val;
        s_aux[ci] = pool_key(val, a.step, tok, pi);
      }
    }
  }
  const int n_new = F * k;  // <= 256 = NT
  if (tid == 0) {
    a.ws.pool_count[b] = P0 + n_new;
    if (a.step == 1) a.ws.root_token[b] = a.root_tokens[b];
  }
  __syncthreads();
  // phase: children appended
  if (wave != 0) return;
  // ---- next frontier (wave 0): the k most valuable children ---------------
  // Lane l holds children l, l+64, l+128, l+192.  The k-th largest lane
  // maximum of the keys' top 32 bits bounds the top 32 bits of the k-th
  // largest key from below; the keys at or above it are ranked by counting
  // and the top k, in value order, become the frontier (those below the
  // expansion threshold, a suffix, stay unexpanded).
  int nf = 0;
  if (a.step < a.D) {
    uint64_t ck[4];
    uint32_t hmax = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = lane + 64 * u;
      ck[u] = t < n_new ? s_aux[t] : 0;
      const uint32_t hi = (uint32_t)(ck[u] >> 32);
      hmax = hi > hmax ? hi : hmax;
    }
    const uint32_t T = wave_kth_largest_u32(hmax, k, 0);
    int cq = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) cq += (ck[u] != 0 && (uint32_t)(ck[u] >> 32) >= T) ? 1 : 0;
    int n;
    const int off = wave_excl_prefix_small(cq, &n);
    uint64_t* wbuf = &s_bc[0];
    const int fb = (cur * a.B + b) * k;
    if (n <= kWaveCap) {
      int o = off;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ck[u] != 0 && (uint32_t)(ck[u] >> 32) >= T) wbuf[o++] = ck[u];
      wave_lds_sync();
      bool kept = false;
      if (lane < n) {
        const uint64_t me = wbuf[lane];
        int rank = 0;
#pragma unroll 8
        for (int q = 0; q < n; ++q) rank += wbuf[q] > me;
        if (rank < k) {
          kept = !(pool_value_of(me) < a.thr);
          a.ws.frontier[fb + rank] = kept ? pool_index_of(me) : -1;
          a.ws.frontier_val[fb + rank] = pool_value_of(me);
          // token field of the pool key: bits 12..29 hold 2^18 - 1 - token
          a.next_tokens[(int64_t)b * k + rank] =
              kept ? (int)((1u << 18) - 1u - (uint32_t)((me >> 12) & 0x3FFFFu)) : -1;
        }
      }
      nf = __popcll(__ballot(kept));
    } else {
      // Many equal values: k rounds of wave maximum.
      uint64_t prevk = ~0ull;
      for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (ck[u] < prevk && ck[u] > best) best = ck[u];
        const uint64_t w = wave_max_u64(best);
        const bool kept = w != 0 && !(pool_value_of(w) < a.thr);
        if (lane == 0) {
          a.ws.frontier[fb + r] = kept ? pool_index_of(w) : -1;
          a.ws.frontier_val[fb + r] = pool_value_of(w);
          a.next_tokens[(int64_t)b * k + r] =
              kept ? (int)((1u << 18) - 1u - (uint32_t)((w >> 12) & 0x3FFFFu)) : -1;
        }
        nf += kept ? 1 : 0;
        prevk = w;
      }
    }
  } else if (lane < k) {
    a.ws.frontier[(cur * a.B + b) * k + lane] = -1;
    a.next_tokens[(int64_t)b * k + lane] = -1;
  }
  if (lane == 0) {
    a.ws.frontier_count[cur * a.B + b] = nf;
    a.next_count[b] = nf;
  }
  // phase: frontier written
}

hipError_t launch_draft_step(const Plan& p, const DraftWs& w, int step,
                             const int32_t* root_tokens, const void* logits,
                             int64_t bstride, int64_t rstride, bool vec,
                             int32_t* next_tokens, int32_t* next_count,
                             hipStream_t s) {
  DraftArgs a;
  a.ws = w;
  a.logits = logits;
  a.bstride = bstride;
  a.rstride = rstride;
  a.root_tokens = root_tokens;
  a.next_tokens = next_tokens;
  a.next_count = next_count;
  a.B = p.B;
  a.V = p.V;
  a.k = p.k;
  a.D = p.D;
  a.S = p.s_draft;
  a.step = step;
  a.cap = p.cap;
  a.thr = p.cfg.expand_threshold;
  dim3 grid(p.s_draft, p.k, p.B);
  const bool bf = p.ldt == ET_BF16;
  if (bf && vec) draft_step_kernel<true, true, kElemsBf16><<<grid, kScanThreads, 0, s>>>(a);
  else if (bf) draft_step_kernel<true, false, kElemsBf16><<<grid, kScanThreads, 0, s>>>(a);
  else if (vec) draft_step_kernel<false, true, kElemsF32><<<grid, kScanThreads, 0, s>>>(a);
  else draft_step_kernel<false, false, kElemsF32><<<grid, kScanThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace et
