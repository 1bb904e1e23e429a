// draft.hip -- one expansion layer of the dynamic draft tree.
//
// EAGLE-2 summary page, s4.1 (expansion phase): the draft model's softmax
// confidence stands in for a token's acceptance rate, a node's value is
// the product of confidences on its root path, and the k most valuable
// nodes of the current layer are expanded.  Explainer "EAGLE-2: Dynamic
// Draft Trees", value equation.  EAGLE notes, "EAGLE 2 / 方法", Expand
// stage: nodes whose value is below the threshold are not expanded.
//
// Two launches per step.  Scan: grid (chunk groups, k frontier rows, B
// sequences), 256 threads; each block streams cpb consecutive 8K-element
// chunks of one logits row with 16-byte loads (the next chunk's loads in
// flight while the current one is reduced) and publishes, per chunk and
// wave, the wave's (max, sum of exp) and its top-k logit keys.  cpb is 1
// unless the grid would be many times what the chip holds at once.
// Merge: one block per sequence combines every row's partials into the
// row's softmax statistics and top-k, turns the rows into children (conf,
// value), appends them to the pool and selects the next frontier.  (A
// single launch in which the last scan block to arrive does the merge was
// slower: every block then waits for its stores and an arrival ticket.)
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "rerank.h"

namespace et {

struct DraftArgs {
  DraftWs ws;
  const void* logits;
  int64_t bstride, rstride;
  const int32_t* root_tokens;
  int32_t* next_tokens;
  int32_t* next_count;
  int B, V, k, D, S, cpb, parts, step, cap;
  float thr;
};

constexpr int kWaves = kScanThreads / 64;  // waves per scan block
constexpr int kWaveCap = 64;             // candidate slots per wave

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
// The same over float values through their order-preserving image.  Values
// from bf16 have 16 significant bits: the search fixes the image's top 16
// bits, and the low 16 are those every bf16 image has (zeros for a
// non-negative value, ones for a negative one), so the result is the exact
// k-th largest.  (Left at zero for a negative value, they would make an
// image below that of -inf, i.e. a NaN, against which every comparison
// fails: a wave with fewer than k finite values would lose its top ones.)
template <bool BF16>
__device__ __forceinline__ float wave_kth_largest(float v, int k) {
  uint32_t t = wave_kth_largest_u32(ordered_f32(v), k, BF16 ? 16 : 0);
  if (BF16 && !(t & 0x80000000u)) t |= 0xFFFFu;
  return unordered_f32(t);
}

// Smallest logit key whose logit is >= x.
__device__ __forceinline__ uint64_t key_floor(float x) {
  return (uint64_t)ordered_f32(x) << 32;
}

typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));
// Number of keys in base[lo, hi) (LDS) greater than me, read 16 keys at a
// time with 16-byte loads issued together (one wait per 16 keys, not one
// per key).  base must be 16-byte aligned and lo even; reads reach below
// lo + 16 * ceil((hi - lo) / 16), which the caller's array must hold.
__device__ __forceinline__ int count_greater(const uint64_t* base, int lo, int hi, uint64_t me) {
  int cnt = 0;
  for (int j0 = lo; j0 < hi; j0 += 16) {
    u64x2_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const u64x2_t*)&base[j0 + 2 * u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      cnt += (j0 + 2 * u < hi && v[u].x > me) ? 1 : 0;
      cnt += (j0 + 2 * u + 1 < hi && v[u].y > me) ? 1 : 0;
    }
  }
  return cnt;
}

// Chunks [c0, c0 + nch) of row j of sequence b: per chunk, the block's
// (max, sum of exp) and its top-k logit keys, stored for the merge launch;
// with WAVE, each wave publishes its own 1/4 of the chunk instead
// (no block-level step, the waves never wait for one another).  The caller has issued the first chunk's loads (raw, or x on
// the element-wise path); the next chunk's loads are issued once the
// current chunk's values are staged in LDS.  On the vector path the
// values stay in their loaded form (bf16 pairs) and are widened where
// used, which keeps the register count down.
template <bool BF16, bool VEC, int E, bool WAVE>
__device__ __forceinline__ void scan_chunks(const DraftArgs& a, const char* row, int j, int b,
                                            int c0, int nch, float (&x)[E],
                                            u32x4_t (&raw)[VEC ? chunk_vectors<BF16, E>() : 1]) {
  constexpr int NT = kScanThreads;
  constexpr int kChunkE = NT * E;
  constexpr float kLog2e = 1.4426950408889634f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k, S = a.S;
  constexpr int NV = chunk_vectors<BF16, E>();
  constexpr int kE2Bits = E < 32 ? 5 : E < 64 ? 6 : 7;  // bit planes of a count <= E
  // lane values as loaded (vector path) or as fp32 (element-wise path)
  __shared__ u32x4_t s_x[kScanThreads * (VEC ? NV : E / 4)];
  __shared__ __attribute__((aligned(16))) uint64_t s_wl[kWaves * kWaveCap];  // wave candidate lists
  __shared__ uint64_t s_bc[kWaves * kWaveCap];  // block candidates
  __shared__ float s_wf[3][kWaves];             // wave bound, max, sum
  __shared__ int s_wcnt[kWaves];
  __shared__ int s_count;
  // ---- chunks: per wave max, sum of exp and candidates --------------------
  for (int ci = 0; ci < nch; ++ci) {
  const int c = c0 + ci;
  const int base = c * kChunkE;
  if constexpr (VEC) fix_chunk_tail<BF16, E>(row, base, a.V, tid, raw);
  if (tid == 0) s_count = 0;
  // phase: chunk loaded
  // element e of the lane (e a compile-time index)
  auto xv = [&](int e) -> float {
    if constexpr (VEC && BF16) {
      const uint32_t w = raw[e >> 3][(e >> 1) & 3];
      return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else if constexpr (VEC) {
      return __uint_as_float(raw[e >> 2][e & 3]);
    } else {
      return x[e];
    }
  };
  // element e of the lane from its LDS copy (e may be a run-time index)
  auto xs = [&](int e) -> float {
    if constexpr (VEC && BF16)
      return __uint_as_float((uint32_t)((const uint16_t*)s_x)[((e >> 3) * NT + tid) * 8 + (e & 7)] << 16);
    else
      return ((const float*)s_x)[((e >> 2) * NT + tid) * 4 + (e & 3)];
  };

  // Lane max as a ternary tree (three-input maxima, short chain).
  float mx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) mx[e] = xv(e);
#pragma unroll
  for (int n = E; n > 1; n = (n + 2) / 3)
#pragma unroll
    for (int i = 0; i < (n + 2) / 3; ++i) {
      float m = mx[3 * i];
      if (3 * i + 1 < n) m = fmaxf(m, mx[3 * i + 1]);
      if (3 * i + 2 < n) m = fmaxf(m, mx[3 * i + 2]);
      mx[i] = m;
    }
  const float lmax = mx[0];
  // exp(x - m) = 2^(x log2 e - m log2 e): one FMA and v_exp_f32; four
  // accumulators keep the add chain short.  The lane sums against its own
  // maximum (offset a), so the exps need not wait for the wave's maximum
  // (offset b): the lane's share of the wave sum is that sum times
  // 2^(a - b), and with x log2 e - a exact inside the FMA the product
  // differs from the direct 2^(x log2 e - b) by the rounding of a - b.
  const float offa = lmax > -INFINITY ? lmax * kLog2e : 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < E; ++e)
    acc[e & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(xv(e), kLog2e, -offa));
  const float ls = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  const float mw = wave_max_f32(lmax);
  const float sl = lmax > -INFINITY ? ls * __builtin_amdgcn_exp2f(offa - mw * kLog2e) : 0.f;
  const float sw = wave_sum_f32(sl);
  // phase: max and sum of exp
  // The wave's k-th largest lane maximum Lw bounds its k-th largest
  // element from below (those k maxima are k distinct elements), so every
  // element of the wave's top-k is >= Lw.  Each lane marks its elements
  // >= Lw in a bit mask; a wave prefix sum of the counts gives each lane
  // its slots, and the lane writes its (usually zero to two) candidates.
  const float Lw = wave_kth_largest<BF16>(lmax, k);
  // phase: wave threshold
  // element e's vocab id is lid + (its offset from the lane's first
  // element, a constant); ids at or past V are padding
  constexpr int per = BF16 ? 8 : 4;
  const int lid = base + tid * per;
  const int lim = a.V - lid;
  // Ids past V read -inf, so with a finite Lw no bound check is needed;
  // Lw = -inf (fewer than k lanes of the wave inside the row) takes it.
  static_assert(E <= 64, "one mask bit per element");
  using mask_t = typename std::conditional<(E > 32), uint64_t, uint32_t>::type;
  mask_t bits = 0u;
  if (Lw > -INFINITY) {
    // x >= Lw exactly when x - Lw has a clear sign bit: x - Lw is +0 for
    // x == Lw and -inf for x = -inf (inputs hold no NaN or +inf), and a
    // zero bound is taken as -0 so that an element -0, equal to it, gives
    // +0.  Each sign bit is shifted into a register with one alignbit
    // ((neg << 1) | (d >> 31)), elements 32 h .. 32 h + 31 into word h,
    // element e ending at bit n_h - 1 - (e - 32 h) of it (n_h elements);
    // one bit reversal per word then puts element e at bit e - 32 h.
    const float Lz = Lw == 0.f ? -0.f : Lw;
    uint32_t neg[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e)
      neg[e >> 5] = __builtin_amdgcn_alignbit(neg[e >> 5], __float_as_uint(xv(e) - Lz), 31);
    bits = (mask_t)(__brev(~neg[0]) >> (32 - (E < 32 ? E : 32)));
    if constexpr (E > 32) bits |= (mask_t)(__brev(~neg[1]) >> (64 - E)) << 32;
  } else {
    // (one is opaque to the compiler: written as cond ? 1 << e : 0 the
    // masks would be hoisted out of the chunk loop into registers)
    mask_t one = 1u;
    asm volatile("" : "+v"(one));
#pragma unroll
    for (int e = 0; e < E; ++e)
      bits |= (elem_off<BF16>(e, 0) < lim && xv(e) >= Lw ? one : 0u) << e;
  }
  // The lane's values are staged in LDS so that each candidate is read by
  // index (a register array cannot be indexed at run time cheaply).
  // Layout: 16-byte group q of every lane in one contiguous row of the
  // block, so each group's store is free of bank conflicts.
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < NV; ++q) s_x[q * kScanThreads + tid] = raw[q];
  } else {
#pragma unroll
    for (int q = 0; q < E / 4; ++q)
      s_x[q * kScanThreads + tid] = u32x4_t{__float_as_uint(x[4 * q]), __float_as_uint(x[4 * q + 1]),
                                            __float_as_uint(x[4 * q + 2]), __float_as_uint(x[4 * q + 3])};
  }
  // The registers are free from here on: the next chunk's loads go out
  // and land while this chunk's candidates are ranked and published.
  if constexpr (VEC)
    if (ci + 1 < nch) issue_chunk<BF16, E>(row, base + kChunkE, a.V, tid, raw);
  int wtot;
  int o = wave_excl_prefix_small<kE2Bits>(__popcll((uint64_t)bits), &wtot);  // <= E
  uint64_t* wl = &s_wl[wave * kWaveCap];
  if (wtot <= kWaveCap) {
    while (bits) {
      const int e = __ffsll((unsigned long long)bits) - 1;
      bits &= bits - 1;
      wl[o++] = logit_key(xs(e), (uint32_t)(lid + elem_off<BF16>(e, 0)));
    }
  } else {
    // Many equal logits: the wave's exact top-k, by k rounds of maximum.
    uint64_t prevk = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      // (a rare path, rolled: unrolled, its per-element keys took registers
      // from the common path, 167 against 102 per lane, and the step was
      // 9% slower at 64 sequences)
#pragma unroll 2
      for (int e = 0; e < E; ++e) {
        const int id = lid + elem_off<BF16>(e, 0);
        const uint64_t key = id < a.V ? logit_key(xs(e), (uint32_t)id) : 0;
        if (key < prevk && key > best) best = key;
      }
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) wl[r] = w;
      prevk = w;
    }
    wtot = k;
  }
  if constexpr (WAVE) {
    // The wave's list, ranked by counting; its entry is partial
    // (row, chunk, wave).
    wave_lds_fence();
    const int64_t rowid = (int64_t)b * k + j;
    const int li = c * kWaves + wave;  // list index within the row
    const int64_t pe = rowid * a.parts + li;
    uint64_t* dst = &a.ws.part_keys[rowid * kMaxTopk * a.parts + li];  // rank r at r * parts
    if (lane < wtot) {
      const uint64_t me = wl[lane];
      const int rank = count_greater(wl, 0, wtot, me);  // wtot <= 64: reads within the list
      if (rank < k) dst[(int64_t)rank * a.parts] = me;
    }
    if (lane >= wtot && lane < k) dst[(int64_t)lane * a.parts] = 0;
    if (lane == 0) {
      a.ws.part_m[pe] = mw;
      a.ws.part_s[pe] = sw;
    }
    // phase: wave published
    if constexpr (!VEC)
      if (ci + 1 < nch) load_chunk<BF16, false, E>(row, base + kChunkE, a.V, tid, x);
    continue;
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
  uint64_t* dst = &a.ws.part_keys[rowid * kMaxTopk * S + c];  // rank r at r * S
  for (int t = tid; t < nb; t += NT) {
    const uint64_t me = s_bc[t];
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < nb; ++q) rank += s_bc[q] > me;
    if (rank < k) dst[(int64_t)rank * S] = me;
  }
  if (tid >= nb && tid < k) dst[(int64_t)tid * S] = 0;
  if (tid == 0) {
    float sb = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      sb += s_wf[1][w] > -INFINITY ? s_wf[2][w] * expf(s_wf[1][w] - mb) : 0.f;
    a.ws.part_m[pe] = mb;
    a.ws.part_s[pe] = sb;
  }
  if (ci + 1 < nch) {
    if constexpr (!VEC) load_chunk<BF16, false, E>(row, base + kChunkE, a.V, tid, x);
    __syncthreads();  // the LDS lists are reused by the next chunk
  }
  }
}

// A sequence whose tree stopped growing: no rows, empty next frontier.
__device__ __forceinline__ void empty_frontier(const DraftArgs& a, int b) {
  const int tid = threadIdx.x, cur = a.step & 1;
  if (tid < a.k) a.next_tokens[(int64_t)b * a.k + tid] = -1;
  if (tid == 0) {
    a.next_count[b] = 0;
    a.ws.frontier_count[cur * a.B + b] = 0;
  }
}

// Merge launch: one block of k waves per sequence; wave j merges frontier
// row j, one partial list per lane (a row has at most 64 lists).  The
// row's max and sum of exp are wave reductions.  Bound: with at least k
// lists the k-th largest list head bounds the row's k-th largest key from
// below, so only keys at or above it (a prefix of every sorted list) are
// ranked; each lane stages the first KST keys of its list.  A row whose
// candidates do not fit the staged keys (many equal or clustered logits)
// takes an exact path: k rounds of wave maximum over all of its keys.
// The children (conf, value) go to the pool; the next frontier is the k
// largest children keys, ranked by counting with four threads per child
// across the whole block.
// FIXED: the next frontier comes from a fixed shape (fx) instead of the
// children's values.
// What the last step's merge leaves for the rerank in the same block: the
// pool size before the step, the children appended, and the children's
// pool keys, parent pool indexes and conf in LDS (child c at index c).
struct LastChildren {
  int P0, n_new;
  const uint64_t* key;
  const int* par;
  const float* conf;
};

template <bool BF16, int KST, bool FIXED, bool LAST = false>
__device__ __forceinline__ void merge_rows(const DraftArgs& a, const FixedFrontier* fx, int b,
                                           LastChildren* lc = nullptr) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int tid = threadIdx.x, lane = tid & 63, jr = tid >> 6;  // jr: this wave's row
  const int k = a.k, S = a.parts;  // partial lists per row (<= 64)
  const int prev = (a.step - 1) & 1, cur = a.step & 1;
  __shared__ __attribute__((aligned(16))) uint64_t s_rc[kMaxTopk * 64];  // row candidates
  __shared__ uint64_t s_rk[kMaxTopk * kMaxTopk];  // row top-k keys
  // children's pool keys; the padding covers count_greater's last reads
  __shared__ __attribute__((aligned(16))) uint64_t s_aux[kMaxTopk * kMaxTopk + 32];
  __shared__ int s_cpar[LAST ? kMaxTopk * kMaxTopk : 1];    // children's parents (LAST)
  __shared__ float s_cconf[LAST ? kMaxTopk * kMaxTopk : 1];  // and conf (LAST)
  __shared__ int s_nf;
  // Every load is issued before the frontier count F arrives: rows j < k
  // of the workspace are always readable, rows j >= F are dropped.
  const int64_t rowid = (int64_t)b * k + jr;
  const int li = lane < S ? lane : S - 1;
  const int64_t fs = ((int64_t)prev * a.B + b) * k + jr;
  const int par0 = a.ws.frontier[fs];
  const float vpar0 = a.ws.frontier_val[fs];
  float pm = a.ws.part_m[rowid * S + li];
  float ps = a.ws.part_s[rowid * S + li];
  uint64_t pk[KST];
#pragma unroll
  for (int r = 0; r < KST; ++r)
    pk[r] = a.ws.part_keys[(rowid * kMaxTopk + min(r, k - 1)) * S + li];
  const int P0 = a.step == 1 ? 0 : a.ws.pool_count[b];
  const int F = a.step == 1 ? 1 : a.ws.frontier_count[prev * a.B + b];
  if constexpr (LAST) *lc = LastChildren{P0, 0, s_aux, s_cpar, s_cconf};
  if (F == 0) {
    empty_frontier(a, b);
    return;
  }
  if (tid == 0) s_nf = 0;
  // phase: partials read
  const bool on_row = jr < F;
  if (!on_row || lane >= S) {
    pm = -INFINITY;
    ps = 0.f;
  }
#pragma unroll
  for (int r = 0; r < KST; ++r)
    if (!on_row || lane >= S || r >= k) pk[r] = 0;
  const int par = a.step > 1 ? par0 : -1;
  const float vpar = a.step > 1 ? vpar0 : 1.0f;
  const float m = wave_max_f32(pm);
  const float sum =
      wave_sum_f32(pm > -INFINITY ? ps * __builtin_amdgcn_exp2f((pm - m) * kLog2e) : 0.f);
  // phase: row max and sum
  // k-th largest list head, bit by bit on the ordered logit
  uint64_t Lk = 0;
  if (S >= k) {
    const uint32_t hk = (uint32_t)(pk[0] >> 32);  // 0 for no key
    uint32_t t = 0;
#pragma unroll
    for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
      const uint32_t cand = t | (1u << bit);
      if (__popcll(__ballot(hk >= cand)) >= k) t = cand;
    }
    Lk = (uint64_t)t << 32;
  }
  // phase: row bound
  // keys at or above the bound: a prefix of each list; a list whose staged
  // keys all qualify may hold more (then the row takes the exact path)
  int cl = 0;
#pragma unroll
  for (int r = 0; r < KST; ++r) cl += (pk[r] != 0 && pk[r] >= Lk) ? 1 : 0;
  const bool more = cl == KST && k > KST;
  int n;
  const int off = wave_excl_prefix_small<KST == 4 ? 3 : 4>(cl, &n);  // cl <= KST
  const bool fits = n <= 64 && __ballot(more) == 0ull;
  uint64_t* lst = &s_rc[jr * 64];
  if (on_row && fits) {
#pragma unroll
    for (int r = 0; r < KST; ++r)
      if (r < cl) lst[off + r] = pk[r];
  }
  wave_lds_fence();
  // phase: row list written
  // The row's top-k keys: the candidate of rank r (r < k) becomes child r,
  // formed by the lane that ranked it (fast path), or by lane r from the
  // exact path's list.
  uint64_t ckey = 0;
  int crank = -1;
  if (on_row && fits) {
    if (lane < n) {  // n <= 64: reads stay within the row's 64 entries
      ckey = lst[lane];
      crank = count_greater(lst, 0, n, ckey);
      if (crank >= k) crank = -1;
    }
  } else if (on_row) {
    // every key of the row, at most 64 lists x 16 ranks (16 per lane)
    const uint64_t* rk = &a.ws.part_keys[rowid * kMaxTopk * S];  // [rank][list]
    uint64_t v[kMaxTopk];
#pragma unroll
    for (int i = 0; i < kMaxTopk; ++i) {
      const int t = lane + 64 * i;  // rank t / S of list t % S
      v[i] = t < S * k ? rk[t] : 0;
    }
    uint64_t prevk = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kMaxTopk; ++i)
        if (v[i] < prevk && v[i] > best) best = v[i];
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) s_rk[jr * kMaxTopk + r] = w;
      prevk = w;
    }
    wave_lds_fence();
    if (lane < k) {
      ckey = s_rk[jr * kMaxTopk + lane];
      crank = lane;
    }
  }
  // phase: row ranked
  // Children of the row, in rank order (conf decreasing): child r of row
  // jr is pool node P0 + jr * k + r.
  // The child's pool fields stay in registers: every global store of the
  // merge is issued at its end, so no later step waits for a store to land
  // (the compiler waits for pending stores before reusing their registers).
  const int64_t pb = (int64_t)b * a.cap;
  const bool mine = crank >= 0;  // on_row is implied
  const float rsum = __builtin_amdgcn_rcpf(sum);
  int c_tok = 0, c_pi = 0;
  float c_conf = 0.f, c_val = 0.f;
  if (mine) {
    c_tok = (int)id_of(ckey);
    c_conf = __builtin_amdgcn_exp2f((logit_of(ckey) - m) * kLog2e) * rsum;
    c_val = __fmul_rn(vpar, c_conf);
    const int ci = jr * k + crank;
    c_pi = P0 + ci;
    s_aux[ci] = pool_key(c_val, a.step, c_tok, c_pi);
    if constexpr (LAST) {
      s_cpar[ci] = par;
      s_cconf[ci] = c_conf;
    }
  }
  const int n_new = F * k;  // <= k * k: four threads per child fit the k waves
  if constexpr (LAST) lc->n_new = n_new;
  lds_barrier();
  // phase: children appended
  const int fb = (cur * a.B + b) * k;
  // the frontier entry this thread writes at the end (slot f_at, or none)
  int f_at = -1, f_idx = -1, f_tok = -1;
  float f_val = 0.f;
  if constexpr (FIXED) {
    // Fixed shape: next-frontier node i is child fx->ci[i] of this step.
    if (tid < k) {
      int ci = -1;
#pragma unroll
      for (int i = 0; i < kMaxTopk; ++i)
        if (tid == i && i < fx->n) ci = fx->ci[i];
      const bool kept = ci >= 0 && ci < n_new;
      const uint64_t key = kept ? s_aux[ci] : 0;
      f_at = tid;
      f_idx = kept ? pool_index_of(key) : -1;
      f_val = kept ? pool_value_of(key) : 0.0f;
      f_tok = kept ? pool_token_of(key) : -1;
      if (kept) atomicAdd(&s_nf, 1);
    }
  } else if (a.step < a.D) {
    // The k largest children keys: child c's rank is the number of larger
    // keys, counted by its four threads over a quarter of the children each
    // (q of them, q even so every quarter starts 16-byte aligned).  Keys
    // are distinct (the pool index field), so the ranks are too.  Those
    // below the expansion threshold (a suffix: value leads the key) stay
    // unexpanded.
    const int c = tid >> 2, part = tid & 3;
    const uint64_t me = c < n_new ? s_aux[c] : ~0ull;
    const int q = ((n_new + 3) / 4 + 1) & ~1;
    int cnt = count_greater(s_aux, part * q, min(n_new, part * q + q), me);
    cnt += xor_lane<1>(cnt);
    cnt += xor_lane<2>(cnt);
    if (part == 0 && c < n_new && cnt < k) {
      const bool kept = !(pool_value_of(me) < a.thr);
      f_at = cnt;
      f_idx = kept ? pool_index_of(me) : -1;
      f_val = pool_value_of(me);
      f_tok = kept ? pool_token_of(me) : -1;
      if (kept && a.thr > 0.f) atomicAdd(&s_nf, 1);
    }
  } else if (tid < k) {
    f_at = tid;  // the last step: no frontier
  }
  // With the stop rule off every one of the k (<= n_new) frontier nodes is
  // kept: the count is known without a reduction.
  int nf = 0;
  if (FIXED || a.step >= a.D || a.thr > 0.f) {
    lds_barrier();  // s_nf complete
    nf = s_nf;
  } else {
    nf = k;
  }
  // phase: frontier written
  // every global store of the merge
  if (mine) {
    a.ws.pool_token[pb + c_pi] = c_tok;
    a.ws.pool_parent[pb + c_pi] = par;
    a.ws.pool_depth[pb + c_pi] = a.step;
    a.ws.pool_conf[pb + c_pi] = c_conf;
    a.ws.pool_value[pb + c_pi] = c_val;
  }
  if (f_at >= 0) {
    a.ws.frontier[fb + f_at] = f_idx;
    if (FIXED || a.step < a.D) a.ws.frontier_val[fb + f_at] = f_val;
    a.next_tokens[(int64_t)b * k + f_at] = f_tok;
  }
  if (tid == 0) {
    a.ws.pool_count[b] = P0 + n_new;
    if (a.step == 1) a.ws.root_token[b] = a.root_tokens[b];
    a.ws.frontier_count[cur * a.B + b] = nf;
    a.next_count[b] = nf;
  }
}

// Scan launch: block (x, j, b) streams chunks [x * cpb, x * cpb + cpb) of
// row j of sequence b and exits.  The first chunk's loads are issued
// before the frontier count arrives (every row j < topk is readable memory
// by contract; rows j >= F are dropped), so the count's latency hides
// behind the logits'.  WAVE: per-wave partials (when a row's S * 4 lists
// fit one merge wave), else per-block partials.
template <bool BF16, bool VEC, int E, bool WAVE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(VEC ? (E > 32 ? 4 : 3) : 1))) void draft_scan_kernel(DraftArgs a) {
  constexpr int kChunkE = kScanThreads * E;
  const int j = blockIdx.y, b = blockIdx.z;  // (step 1 launches row 0 only)
  const char* row = (const char*)a.logits + (b * a.bstride + j * a.rstride) * (BF16 ? 2 : 4);
  const int c0 = blockIdx.x * a.cpb;
  float x[E];
  u32x4_t raw[VEC ? chunk_vectors<BF16, E>() : 1];
  if constexpr (VEC) issue_chunk<BF16, E>(row, c0 * kChunkE, a.V, threadIdx.x, raw);
  else load_chunk<BF16, false, E>(row, c0 * kChunkE, a.V, threadIdx.x, x);
  const int F = a.step == 1 ? 1 : a.ws.frontier_count[((a.step - 1) & 1) * a.B + b];
  if (j >= F) return;
  scan_chunks<BF16, VEC, E, WAVE>(a, row, j, b, c0, min(a.cpb, a.S - c0), x, raw);
}

// Merge launch: one block of k waves per sequence.
template <bool BF16, int KST>
__global__ __launch_bounds__(1024) void draft_merge_kernel(DraftArgs a) {
  merge_rows<BF16, KST, false>(a, nullptr, blockIdx.x);
}
template <bool BF16, int KST>
__global__ __launch_bounds__(1024) void draft_merge_fixed_kernel(DraftArgs a, FixedFrontier fx) {
  merge_rows<BF16, KST, true>(a, &fx, blockIdx.x);
}

// Merge of the last step, then the rerank and flatten of the finished tree
// by the same block (one launch fewer per cycle than et_rerank_mask after
// the step).  The pool nodes of the earlier steps are loaded first, with
// the merge's own loads (clamped to the readable capacity, dropped past
// the pool size once it is known); the step's children come from LDS.
template <bool BF16, int KST, int RP>
__global__ __launch_bounds__(1024) void draft_merge_last_kernel(DraftArgs a, RerankOut o) {
  // The arguments of the merge's first loads, read with the pool's in one
  // round of scalar loads (the compiler would otherwise read them in two
  // more rounds, between the pool loads and the merge's).
  asm volatile("" ::"s"(a.ws.frontier), "s"(a.ws.frontier_val), "s"(a.ws.frontier_count),
               "s"(a.ws.part_m), "s"(a.ws.part_s), "s"(a.ws.part_keys), "s"(a.ws.pool_count),
               "s"(a.ws.root_token), "s"(a.root_tokens), "s"(o.prefix_len), "s"(a.k), "s"(a.B),
               "s"(a.parts), "s"(a.step), "s"(a.cap));
  const int b = blockIdx.x, tid = threadIdx.x, nt = 64 * a.k;  // (the launch has 64 k threads)
  __shared__ RerankLds L;
  const int64_t pb = (int64_t)b * a.cap;
  const int rounds = (a.cap + nt - 1) / nt;  // <= RP (chosen by the host)
  int par[RP], dep[RP], tok[RP];
  float cnf[RP], val[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    val[i] = cnf[i] = 0.f;
    par[i] = dep[i] = tok[i] = -1;
    if (i < rounds) {  // uniform
      const int64_t g = pb + min(tid + nt * i, a.cap - 1);
      val[i] = a.ws.pool_value[g];
      dep[i] = a.ws.pool_depth[g];
      tok[i] = a.ws.pool_token[g];
      par[i] = a.ws.pool_parent[g];
      cnf[i] = a.ws.pool_conf[g];
    }
  }
  const int pre = o.prefix_len[b];
  // (step 1 is also the last when D = 1: the root token is then the
  // input's, the workspace copy being written by this same launch)
  const int root = a.step == 1 ? a.root_tokens[b] : a.ws.root_token[b];
  LastChildren lc;
  merge_rows<BF16, KST, false, true>(a, nullptr, b, &lc);
  // the pool values become opaque only here, so that nothing computed
  // from them is scheduled before the merge (each such use a wait for the
  // memory round trip ahead of the merge's own loads)
#pragma unroll
  for (int i = 0; i < RP; ++i)
    asm volatile("" : "+v"(val[i]), "+v"(dep[i]), "+v"(tok[i]), "+v"(par[i]), "+v"(cnf[i]));
  uint64_t key[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    const int idx = tid + nt * i;
    key[i] = 0;
    if (idx < lc.P0) {
      key[i] = pool_key(val[i], dep[i], tok[i], idx);
    } else if (idx < lc.P0 + lc.n_new) {
      const int c = idx - lc.P0;
      key[i] = lc.key[c];
      par[i] = lc.par[c];
      cnf[i] = lc.conf[c];
    }
  }
  const int P = lc.P0 + lc.n_new;
  rerank_block<true, RP>(o, L, b, nt, key, par, cnf, P < o.N ? P : o.N, root, pre);
}

// Keys staged per list: four when a row has 64 lists (its top k then
// almost always lie within the first four of each), eight with up to 32.
// A launch lasts as long as its slowest block, so a few rows on the exact
// path set the step's time: at 64 sequences of 128256 bf16 ids (32 lists
// per row, half the rows from flat softmaxes) about 1% of the rows needed
// more than four keys of some list, and with eight none did.
constexpr int merge_stage(int parts) { return parts > 32 ? 4 : 8; }

hipError_t launch_draft_merge(const Plan& p, const DraftWs& w, int step,
                              const int32_t* root_tokens, int parts,
                              int32_t* next_tokens, int32_t* next_count, hipStream_t s) {
  DraftArgs a;
  a.ws = w;
  a.logits = nullptr;
  a.bstride = a.rstride = 0;
  a.root_tokens = root_tokens;
  a.next_tokens = next_tokens;
  a.next_count = next_count;
  a.B = p.B;
  a.V = p.V;
  a.k = p.k;
  a.D = p.D;
  a.S = parts;
  a.cpb = 1;
  a.parts = parts;
  a.step = step;
  a.cap = p.cap;
  a.thr = p.cfg.expand_threshold;
  if (merge_stage(parts) == 4) draft_merge_kernel<false, 4><<<p.B, 64 * p.k, 0, s>>>(a);
  else draft_merge_kernel<false, 8><<<p.B, 64 * p.k, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_draft_step(const Plan& p, const DraftWs& w, int step,
                             const int32_t* root_tokens, const void* logits,
                             int64_t bstride, int64_t rstride, bool vec,
                             const FixedFrontier* fixed, int32_t* next_tokens,
                             int32_t* next_count, hipStream_t s, const RerankOut* last) {
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
  a.cpb = p.draft_cpb;
  a.step = step;
  a.cap = p.cap;
  a.thr = p.cfg.expand_threshold;
  const bool bf = p.ldt == ET_BF16;
  // step 1 scans the root row only: one row of blocks per sequence
  const dim3 grid((p.s_draft + p.draft_cpb - 1) / p.draft_cpb, step == 1 ? 1 : p.k, p.B);
  const bool wv = p.s_draft * kWaves <= 64;
  a.parts = wv ? p.s_draft * kWaves : p.s_draft;
#define ET_SCAN(W, X)                                                                                   \
  do {                                                                                                  \
    if (bf && vec) draft_scan_kernel<true, true, X * kElemsBf16, W><<<grid, kScanThreads, 0, s>>>(a);  \
    else if (bf) draft_scan_kernel<true, false, X * kElemsBf16, W><<<grid, kScanThreads, 0, s>>>(a);   \
    else if (vec) draft_scan_kernel<false, true, X * kElemsF32, W><<<grid, kScanThreads, 0, s>>>(a);   \
    else draft_scan_kernel<false, false, X * kElemsF32, W><<<grid, kScanThreads, 0, s>>>(a);          \
  } while (0)
  // wide chunks (twice the elements per thread) for grids of many rows
  if (p.draft_wide) {
    if (wv) ET_SCAN(true, 2);
    else ET_SCAN(false, 2);
  } else {
    if (wv) ET_SCAN(true, 1);
    else ET_SCAN(false, 1);
  }
#undef ET_SCAN
#define ET_MERGE(BF, K)                                                                  \
  do {                                                                                   \
    if (fixed) draft_merge_fixed_kernel<BF, K><<<p.B, 64 * p.k, 0, s>>>(a, *fixed);      \
    else if (last && rp == 1) draft_merge_last_kernel<BF, K, 1><<<p.B, 64 * p.k, 0, s>>>(a, *last); \
    else if (last && rp == 2) draft_merge_last_kernel<BF, K, 2><<<p.B, 64 * p.k, 0, s>>>(a, *last); \
    else if (last) draft_merge_last_kernel<BF, K, 4><<<p.B, 64 * p.k, 0, s>>>(a, *last); \
    else draft_merge_kernel<BF, K><<<p.B, 64 * p.k, 0, s>>>(a);                          \
  } while (0)
  const int kst = merge_stage(a.parts);
  // pool nodes per thread of the last merge (64 k threads): the fewest
  // of 1, 2 and 4 that cover the capacity, which keeps its code short
  const int rounds = (p.cap + 64 * p.k - 1) / (64 * p.k);
  const int rp = rounds <= 1 ? 1 : rounds <= 2 ? 2 : 4;
  if (bf && kst == 4) ET_MERGE(true, 4);
  else if (bf) ET_MERGE(true, 8);
  else if (kst == 4) ET_MERGE(false, 4);
  else ET_MERGE(false, 8);
#undef ET_MERGE
  return hipGetLastError();
}

}  // namespace et
