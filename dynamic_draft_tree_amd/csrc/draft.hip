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
// 256 threads.  Each block streams one 4096-element chunk of one logits
// row with 16-byte loads and produces (max, sum of exp, top-k keys).  The
// last block to finish a row merges that row's S partials; the last row to
// finish a sequence turns the rows into children (conf, value), appends
// them to the pool and selects the next frontier.  No host sync, no
// second launch.
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

constexpr int kCandCap = 512;            // LDS candidate slots per block
constexpr int kWaves = kScanThreads / 64;  // waves per scan block
// wave-list keys of one row: (max chunks per row) * waves * k
constexpr int row_keys_cap(int E) {
  return ((kMaxVocab + kScanThreads * E - 1) / (kScanThreads * E)) * kWaves * kMaxTopk;
}

template <bool BF16, bool VEC, int E>
__global__ __launch_bounds__(256) void draft_step_kernel(DraftArgs a) {
  constexpr int NT = kScanThreads;
  constexpr int kChunkE = NT * E;
  constexpr float kLog2e = 1.4426950408889634f;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k;
  __shared__ uint64_t s_keys[kCandCap];  // also 4 x 128 wave scratch
  constexpr int kRowKeys = row_keys_cap(E);
  __shared__ uint64_t s_aux[kRowKeys];
  __shared__ uint64_t s_top[kMaxTopk];
  __shared__ uint64_t s_red[kWaves];
  __shared__ int s_count;
  __shared__ int s_flag;

  const int prev = (a.step - 1) & 1, cur = a.step & 1;
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

  // ---- stream one chunk: per wave max, sum of exp and top-k -------------
  const int64_t esz = BF16 ? 2 : 4;
  const char* row = (const char*)a.logits + (b * a.bstride + j * a.rstride) * esz;
  const int base = c * kChunkE;
  float x[E];
  load_chunk<BF16, VEC, E>(row, base, a.V, tid, x);
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
  // element of the wave's top-k is >= Lw.  Those elements are compacted
  // into LDS with ballots (branch-free: non-candidates write a spare slot)
  // and ranked by counting; each lands at its rank.
  const float Lw = readlane_f32(wave_sort_desc_f32(lmax), k - 1);
  // phase: wave threshold
  uint64_t* scr = &s_keys[wave * 128];
  int total = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int id = base + elem_off<BF16>(e, tid);
    const bool pred = id < a.V && x[e] >= Lw;
    int n_e;
    const int r = ballot_rank(pred, &n_e);
    if (n_e != 0 && pred && total + r < 64) scr[total + r] = logit_key(x[e], (uint32_t)id);
    total += n_e;
  }
  wave_lds_sync();
  // phase: wave candidates
  const int64_t rowid = (int64_t)b * k + j;
  const int64_t pidx = (rowid * a.S + c) * kWaves + wave;
  uint64_t* dst = &a.ws.part_keys[pidx * kMaxTopk];
  if (total <= 64) {
    // candidate q sits in lane q; compare against each by readlane
    const uint64_t me = lane < total ? scr[lane] : 0;
    int r0 = 0, r1 = 0;
    int q = 0;
    for (; q + 2 <= total; q += 2) {
      r0 += readlane_u64(me, q) > me;
      r1 += readlane_u64(me, q + 1) > me;
    }
    if (q < total) r0 += readlane_u64(me, q) > me;
    const int rank = r0 + r1;
    if (lane < total && rank < k) st_agent(&dst[rank], me);
    if (lane >= total && lane < k) st_agent(&dst[lane], (uint64_t)0);
  } else {
    // Many equal logits: k rounds of wave-wide maximum over the registers.
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
      if (lane == 0) st_agent(&dst[r], w);
      prevk = w;
    }
  }
  // phase: wave top-k
  if (lane == 0) {
    st_agent(&a.ws.part_m[pidx], mw);
    st_agent(&a.ws.part_s[pidx], sw);
  }

  // phase: partial published
  // ---- last block of this row: merge the S chunk partials --------------
  if (!block_arrive_last(&a.ws.row_ticket[rowid], (uint32_t)a.S, &s_flag)) return;
  {
    const int nl = a.S * kWaves;  // sorted wave lists of this row (<= 256)
    const int64_t p0 = rowid * a.S * kWaves;
    const int nk = nl * k;        // <= kRowKeys
    for (int t = tid; t < nk; t += NT) {
      const int li = t / k, r = t - li * k;
      s_aux[t] = ld_agent(&a.ws.part_keys[(p0 + li) * kMaxTopk + r]);
    }
    const float pm = tid < nl ? ld_agent(&a.ws.part_m[p0 + tid]) : -INFINITY;
    const float ps = tid < nl ? ld_agent(&a.ws.part_s[p0 + tid]) : 0.f;
    // phase: row partials read
    // (max, sum of exp) over the nl wave partials, in fp32
    const float m = block_max_f32<NT>(pm, (float*)s_red);
    const float sc = pm > -INFINITY ? ps * expf(pm - m) : 0.f;
    const float srow = block_sum_f32<NT>(sc, (float*)s_red);
    if (tid == 0) {
      st_agent(&a.ws.row_m[rowid], m);
      st_agent(&a.ws.row_s[rowid], srow);
    }
    // Each wave list is sorted, so with at least k lists the k-th largest
    // head bounds the row's k-th largest key from below; rank only the
    // keys above it (with fewer lists every key is a candidate).
    __syncthreads();
    if (tid < nl) s_keys[tid] = s_aux[tid * k];
    // phase: row sum published
    uint64_t Lh = 1;
    if (nl >= k) {
      block_topk<NT>(s_keys, nl, k, s_top, s_red);
      Lh = s_top[k - 1];
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    // phase: row threshold
    for (int t = tid; t < nk; t += NT) {
      const uint64_t v = s_aux[t];
      if (v >= Lh && v != 0) {
        const int slot = atomicAdd(&s_count, 1);
        if (slot < kCandCap) s_keys[slot] = v;
      }
    }
    __syncthreads();
    if (s_count <= kCandCap) block_topk<NT>(s_keys, s_count, k, s_top, s_red);
    else block_topk<NT>(s_aux, nk, k, s_top, s_red);
    if (tid < k) st_agent(&a.ws.row_keys[rowid * kMaxTopk + tid], s_top[tid]);
  }

  // phase: row merged
  // ---- last row of this sequence: children, pool append, next frontier -
  if (!block_arrive_last(&a.ws.seq_ticket[b], (uint32_t)F, &s_flag)) return;
  // phase: sequence ticket won
  const int64_t pb = (int64_t)b * a.cap;
  const int P0 = a.step == 1 ? 0 : a.ws.pool_count[b];
  const int n_new = F * k;  // <= 256 = NT
  if (tid < n_new) {
    const int jj = tid / k, r = tid - jj * k;
    const int64_t rid = (int64_t)b * k + jj;
    const uint64_t key = ld_agent(&a.ws.row_keys[rid * kMaxTopk + r]);
    const float xl = logit_of(key);
    const int tok = (int)id_of(key);
    const float m = ld_agent(&a.ws.row_m[rid]);
    const float conf = expf(xl - m) / ld_agent(&a.ws.row_s[rid]);
    const int par = a.step == 1 ? -1 : a.ws.frontier[(prev * a.B + b) * k + jj];
    const float vpar = par < 0 ? 1.0f : a.ws.pool_value[pb + par];
    const float val = __fmul_rn(vpar, conf);
    const int pi = P0 + tid;
    a.ws.pool_token[pb + pi] = tok;
    a.ws.pool_parent[pb + pi] = par;
    a.ws.pool_depth[pb + pi] = a.step;
    a.ws.pool_conf[pb + pi] = conf;
    a.ws.pool_value[pb + pi] = val;
    s_aux[tid] = pool_key(val, a.step, tok, pi);
  }
  if (tid == 0) {
    a.ws.pool_count[b] = P0 + n_new;
    if (a.step == 1) a.ws.root_token[b] = a.root_tokens[b];
  }
  // phase: children appended
  int nf = 0;
  if (a.step < a.D) {
    // Within a row, children come in order of decreasing confidence, so
    // the first child carries the row's largest value; with at least k
    // rows the k-th largest such head value bounds the layer's k-th
    // largest value from below (with fewer rows every child is a candidate).
    __syncthreads();
    if (tid < F) s_keys[tid] = s_aux[tid * k];
    float vL = 0.f;
    if (F >= k) {
      block_topk<NT>(s_keys, F, k, s_top, s_red);
      vL = pool_value_of(s_top[k - 1]);
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
    // phase: frontier threshold
    if (tid < n_new && !(pool_value_of(s_aux[tid]) < vL))
      s_keys[atomicAdd(&s_count, 1)] = s_aux[tid];
    __syncthreads();
    block_topk<NT>(s_keys, s_count, k, s_top, s_red);
    const uint64_t ftop = tid < k ? s_top[tid] : 0;
    const bool keep = tid < k && ftop != 0 && !(pool_value_of(ftop) < a.thr);
    if (wave == 0) nf = __popcll(__ballot(keep));
    if (tid < k) {
      a.ws.frontier[(cur * a.B + b) * k + tid] = keep ? pool_index_of(ftop) : -1;
      // token field of the pool key: bits 12..29 hold 2^18 - 1 - token
      a.next_tokens[(int64_t)b * k + tid] =
          keep ? (int)((1u << 18) - 1u - (uint32_t)((ftop >> 12) & 0x3FFFFu)) : -1;
    }
  } else if (tid < k) {
    a.ws.frontier[(cur * a.B + b) * k + tid] = -1;
    a.next_tokens[(int64_t)b * k + tid] = -1;
  }
  if (tid == 0) {
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
