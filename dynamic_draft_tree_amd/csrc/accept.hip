// accept.hip -- greedy acceptance of the verified tree (temperature 0).
//
// EAGLE-2 summary page, s2.1: draft tokens are accepted in order along a
// path and the first rejection ends it; EAGLE-3 review, s五: the reported
// speedups use greedy decoding.  At temperature 0 a draft token is
// accepted iff it equals the target model's argmax at its parent.
//
// Two launches.  Scan: grid (chunk groups, T slot rows, B), 256 threads;
// each block streams cpb consecutive chunks of one target row and every
// wave publishes the (max logit, lowest id) key of its quarter of each
// chunk.  Walk: one block per sequence reduces each kept row's keys to
// the row's argmax (in LDS) and one wave walks the tree from the root.
#include "device.h"
#include "internal.h"

namespace et {

struct AcceptArgs {
  AcceptWs ws;
  const void* target;
  int64_t bstride, rstride;
  const int32_t* tokens;
  const int32_t* parent_slot;
  const int32_t* n_kept;
  int32_t* accept_len;
  int32_t* path_slots;
  int32_t* out_tokens;
  int B, V, T, D, S, cpb;
};

constexpr int kAccWaves = kScanThreads / 64;  // keys per chunk

// Scan: the chunk's loads are issued before n_kept arrives (all T rows
// are readable memory by contract; rows past n_kept are dropped), so the
// count's latency hides behind the logits'.
template <bool BF16, bool VEC, int E>
__global__ __launch_bounds__(256) void accept_scan_kernel(AcceptArgs a) {
  constexpr int kChunkE = kScanThreads * E;
  constexpr int per = BF16 ? 8 : 4;
  const int srow = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const char* row = (const char*)a.target + (b * a.bstride + srow * a.rstride) * (BF16 ? 2 : 4);
  const int c0 = blockIdx.x * a.cpb;
  const int nch = min(a.cpb, a.S - c0);
  float x[E];
  u32x4_t raw[VEC ? chunk_vectors<BF16, E>() : 1];
  // n_kept's address with the arguments the loads need, in one round
  uint64_t u_nk = (uint64_t)a.n_kept;
  asm volatile("" : "+s"(u_nk));
  int nkv = ((const gmem_i32*)u_nk)[b];
  if constexpr (VEC) issue_chunk<BF16, E>(row, c0 * kChunkE, a.V, tid, raw);
  else load_chunk<BF16, false, E>(row, c0 * kChunkE, a.V, tid, x);
  // The pins keep the loads ahead of the test (the compiler otherwise
  // moves the test, and its wait for n_kept, in front of them).
  pin_loaded<VEC, E>(raw, x);
  asm volatile("" : "+v"(nkv));
  if (srow > __builtin_amdgcn_readfirstlane(nkv)) return;
  const int64_t rowid = (int64_t)b * a.T + srow;
  for (int ci = 0; ci < nch; ++ci) {
    const int c = c0 + ci;
    const int base = c * kChunkE;
    if constexpr (VEC) {
      decode_chunk<BF16, E>(row, base, a.V, tid, raw, x);
      if (ci + 1 < nch) issue_chunk<BF16, E>(row, base + kChunkE, a.V, tid, raw);
    }
    // phase: chunk loaded
    // (max logit, lowest id) of the wave's elements: the lane maximum as a
    // tree of three-input maxima, the wave maximum, then the lowest id
    // holding it (a lane's ids increase with e).
    float mx[E];
#pragma unroll
    for (int e = 0; e < E; ++e) mx[e] = x[e];
#pragma unroll
    for (int n = E; n > 1; n = (n + 2) / 3)
#pragma unroll
      for (int i = 0; i < (n + 2) / 3; ++i) {
        float m = mx[3 * i];
        if (3 * i + 1 < n) m = fmaxf(m, mx[3 * i + 1]);
        if (3 * i + 2 < n) m = fmaxf(m, mx[3 * i + 2]);
        mx[i] = m;
      }
    const float wm = wave_max_f32(mx[0]);
    const int lid = base + tid * per;  // element e's id is lid + elem_off(e, 0)
    uint32_t best = 0xFFFFFFFFu;
    // ids past V read -inf: with a finite maximum no bound check is needed
    if (wm > -INFINITY) {
#pragma unroll
      for (int e = E - 1; e >= 0; --e)
        if (x[e] == wm) best = (uint32_t)(lid + elem_off<BF16>(e, 0));
    } else {
#pragma unroll
      for (int e = E - 1; e >= 0; --e)
        if (x[e] == wm && elem_off<BF16>(e, 0) < a.V - lid) best = (uint32_t)(lid + elem_off<BF16>(e, 0));
    }
    const uint32_t wid = wave_min_u32(best);
    if (lane == 0)
      a.ws.part[(rowid * a.S + c) * kAccWaves + wave] = wid == 0xFFFFFFFFu ? 0 : logit_key(wm, wid);
    if constexpr (!VEC)
      if (ci + 1 < nch) load_chunk<BF16, false, E>(row, base + kChunkE, a.V, tid, x);
  }
}

// Walk: rows are reduced by segments of SP lanes (SP = the power of two
// >= the row's key count, at most 64; a lane takes every SP-th key), 16
// waves at a time, into LDS; then wave 0 walks.  NR (a power of two) is
// at least the number of such rounds that cover the T rows.
constexpr int kWalkWaves = 16;
template <int NR>
__global__ __launch_bounds__(kWalkWaves * 64) void accept_walk_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_am[kMaxBudget + 1];
  const int P = a.S * kAccWaves;  // keys per row
  int SP = 1;
  while (SP < P && SP < 64) SP <<= 1;
  const int RW = 64 / SP;  // rows per wave
  const int seg = lane / SP, q = lane - seg * SP;
  // Nothing waits for n_kept before it is needed: every slot row below T
  // is reduced (its partials and the tree's token and parent arrays are
  // readable for all T slots; rows past n_kept are never used), and wave
  // 0 loads the tree before the barrier.
  const int32_t* tk = a.tokens + (int64_t)b * a.T;
  const int32_t* ps = a.parent_slot + (int64_t)b * a.T;
  int r_tok[4], r_par[4];
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(lane + 64 * i, a.T - 1);
      r_tok[i] = tk[s];
      r_par[i] = ps[s];
    }
  }
  const int n_kept = a.n_kept[b];
  // Every partial key of every round is loaded before the first is used,
  // with no branch between the loads (rows are clamped to T - 1, keys to
  // P - 1, and the surplus zeroed after): a lane holds keys q and q + SP
  // of its row (P <= 128 at the largest vocabulary).
  constexpr int kKeys = 2;
  static_assert(kMaxVocab / accept_chunk_elems(ET_F32) * kAccWaves <= kKeys * 64,
                "a row's keys exceed two per lane");
  const int per_round = kWalkWaves * RW;
  const uint64_t* pb = a.ws.part + (int64_t)b * a.T * P;
  const int i0 = min(q, P - 1), i1 = min(q + SP, P - 1);
  uint64_t v[NR][kKeys];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int o = min(r * per_round + wave * RW + seg, a.T - 1) * P;
    v[r][0] = pb[o + i0];
    v[r][1] = pb[o + i1];
  }
  // keeps each load where it is (not sunk into the code that uses it)
#pragma unroll
  for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(v[r][0]), "+v"(v[r][1]));
  int n = n_kept;
  asm volatile("" : "+s"(n));  // n_kept read beside the keys, not after the barrier
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int s = r * per_round + wave * RW + seg;
    const uint64_t v0 = s < a.T && q < P ? v[r][0] : 0;
    const uint64_t v1 = s < a.T && q + SP < P ? v[r][1] : 0;
    uint64_t m = v0 > v1 ? v0 : v1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
      if (d < SP) {
        const uint64_t o = xor_lane_rt(m, d);
        m = o > m ? o : m;
      }
    if (q == 0 && s < a.T) s_am[s] = (int)id_of(m);
  }
  __syncthreads();
  // phase: rows merged
  if (wave != 0) return;

  // Greedy walk from the root (one wave).  Lane l holds slots l, l+64, ...
  // (T <= 256); siblings carry distinct tokens, so at most one child of the
  // current slot matches.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = lane + 64 * i <= n;
    r_tok[i] = ok ? r_tok[i] : -1;
    r_par[i] = ok ? r_par[i] : -2;
  }
  int32_t* path = a.path_slots + (int64_t)b * (a.D + 1);
  int32_t* outt = a.out_tokens + (int64_t)b * (a.D + 1);
  int cur = 0, len = 0;
  if (lane == 0) path[0] = 0;
  for (;;) {
    const int want = s_am[cur];
    int found = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t bal = __ballot(r_par[i] == cur && r_tok[i] == want);
      if (found < 0 && bal) found = 64 * i + __ffsll((unsigned long long)bal) - 1;
    }
    if (found < 0 || len >= a.D) break;
    if (lane == 0) {
      path[len + 1] = found;
      outt[len] = want;
    }
    ++len;
    cur = found;
  }
  // phase: walk done
  if (lane == 0) {
    outt[len] = s_am[cur];
    a.accept_len[b] = len;
  }
  for (int i = lane; i <= a.D; i += 64) {
    if (i > len) {
      path[i] = -1;
      outt[i] = -1;
    }
  }
}

hipError_t launch_accept(const Plan& p, const AcceptWs& w, const void* target,
                         int64_t bstride, int64_t rstride, bool vec,
                         const int32_t* tokens, const int32_t* parent_slot,
                         const int32_t* n_kept, int32_t* accept_len,
                         int32_t* path_slots, int32_t* out_tokens,
                         hipStream_t s) {
  AcceptArgs a;
  a.ws = w;
  a.target = target;
  a.bstride = bstride;
  a.rstride = rstride;
  a.tokens = tokens;
  a.parent_slot = parent_slot;
  a.n_kept = n_kept;
  a.accept_len = accept_len;
  a.path_slots = path_slots;
  a.out_tokens = out_tokens;
  a.B = p.B;
  a.V = p.V;
  a.T = p.T;
  a.D = p.D;
  a.S = p.s_accept;
  a.cpb = p.accept_cpb;
  const bool bf = p.ldt == ET_BF16;
  dim3 grid((p.s_accept + p.accept_cpb - 1) / p.accept_cpb, p.T, p.B);
  if (bf && vec) accept_scan_kernel<true, true, kAccElemsBf16><<<grid, kScanThreads, 0, s>>>(a);
  else if (bf) accept_scan_kernel<true, false, kAccElemsBf16><<<grid, kScanThreads, 0, s>>>(a);
  else if (vec) accept_scan_kernel<false, true, kAccElemsF32><<<grid, kScanThreads, 0, s>>>(a);
  else accept_scan_kernel<false, false, kAccElemsF32><<<grid, kScanThreads, 0, s>>>(a);
  // rounds of the row reduction, as the walk kernel counts them
  const int P = p.s_accept * kAccWaves;
  int SP = 1;
  while (SP < P && SP < 64) SP <<= 1;
  const int rounds = (p.T + kWalkWaves * (64 / SP) - 1) / (kWalkWaves * (64 / SP));
  if (rounds <= 1) accept_walk_kernel<1><<<p.B, kWalkWaves * 64, 0, s>>>(a);
  else if (rounds <= 2) accept_walk_kernel<2><<<p.B, kWalkWaves * 64, 0, s>>>(a);
  else if (rounds <= 4) accept_walk_kernel<4><<<p.B, kWalkWaves * 64, 0, s>>>(a);
  else if (rounds <= 8) accept_walk_kernel<8><<<p.B, kWalkWaves * 64, 0, s>>>(a);
  else accept_walk_kernel<(kMaxBudget + 1) / kWalkWaves><<<p.B, kWalkWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace et
