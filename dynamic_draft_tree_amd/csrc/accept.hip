// accept.hip -- greedy acceptance of the verified tree (temperature 0).
//
// EAGLE-2 summary page, s2.1: draft tokens are accepted in order along a
// path and the first rejection ends it; EAGLE-3 review, s五: the reported
// speedups use greedy decoding.  At temperature 0 a draft token is
// accepted iff it equals the target model's argmax at its parent.
//
// One launch.  Grid (S chunks, T slot rows, B), 256 threads.  Each block
// finds the (max logit, lowest id) of one chunk of one target row; the
// last block of a row merges the chunks into that row's argmax; the last
// row of a sequence walks the tree from the root.
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
  int B, V, T, D, S;
};

template <bool BF16, bool VEC, int E>
__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a) {
  constexpr int kChunkE = kScanThreads * E;
  const int c = blockIdx.x, srow = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint64_t s_best[4];
  __shared__ int s_flag;

  const int n = a.n_kept[b];
  if (srow > n) return;

  const int64_t esz = BF16 ? 2 : 4;
  const char* row = (const char*)a.target + (b * a.bstride + srow * a.rstride) * esz;
  const int base = c * kChunkE;
  float x[E];
  load_chunk<BF16, VEC, E>(row, base, a.V, tid, x);
  // phase: chunk loaded
  // (max logit, lowest id) of the chunk: the lane maximum, the wave
  // maximum, then the lowest id holding it (a lane's ids increase with e).
  float mx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) mx[e] = x[e];
#pragma unroll
  for (int w = E / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < w; ++e) mx[e] = fmaxf(mx[e], mx[e + w]);
  const float wm = wave_max_f32(mx[0]);
  uint32_t lid = 0xFFFFFFFFu;
#pragma unroll
  for (int e = E - 1; e >= 0; --e) {
    const int id = base + elem_off<BF16>(e, tid);
    if (x[e] == wm && id < a.V) lid = (uint32_t)id;
  }
  const uint32_t wid = wave_min_u32(lid);
  if (lane == 0) s_best[wave] = wid == 0xFFFFFFFFu ? 0 : logit_key(wm, wid);
  __syncthreads();
  // phase: chunk argmax
  const int64_t rowid = (int64_t)b * a.T + srow;
  if (tid == 0) {
    uint64_t m = s_best[0];
    for (int w = 1; w < 4; ++w) m = s_best[w] > m ? s_best[w] : m;
    st_agent(&a.ws.part[rowid * a.S + c], m);
  }
  // phase: partial published
  if (!block_arrive_last(&a.ws.row_ticket[rowid], (uint32_t)a.S, &s_flag)) return;
  if (wave == 0) {
    uint64_t m = lane < a.S ? ld_agent(&a.ws.part[rowid * a.S + lane]) : 0;
    m = wave_max_u64(m);
    if (lane == 0) st_agent(&a.ws.amax[rowid], (int32_t)id_of(m));
  }
  // phase: row merged
  if (!block_arrive_last(&a.ws.seq_ticket[b], (uint32_t)(n + 1), &s_flag)) return;
  // phase: sequence ticket won
  if (wave != 0) return;

  // Greedy walk from the root (one wave).  Lane l holds slots l, l+64, ...
  // (T <= 256); siblings carry distinct tokens, so at most one child of the
  // current slot matches.
  const int32_t* tk = a.tokens + (int64_t)b * a.T;
  const int32_t* ps = a.parent_slot + (int64_t)b * a.T;
  const int32_t* am = a.ws.amax + (int64_t)b * a.T;
  int r_tok[4], r_par[4], r_am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = lane + 64 * i;
    const bool ok = s <= n;
    r_tok[i] = ok ? tk[s] : -1;
    r_par[i] = ok ? ps[s] : -2;
    r_am[i] = ok ? ld_agent(&am[s]) : -1;
  }
  // phase: walk inputs read
  int32_t* path = a.path_slots + (int64_t)b * (a.D + 1);
  int32_t* outt = a.out_tokens + (int64_t)b * (a.D + 1);
  int cur = 0, len = 0;
  if (lane == 0) path[0] = 0;
  auto amax_of = [&](int s) {
    const int w = s >> 6, l = s & 63;
    const int v = w == 0 ? r_am[0] : w == 1 ? r_am[1] : w == 2 ? r_am[2] : r_am[3];
    return __builtin_amdgcn_readlane(v, l);
  };
  for (;;) {
    const int want = amax_of(cur);
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
  // readlane must run with every lane active (amax_of selects per lane).
  const int bonus = amax_of(cur);
  if (lane == 0) {
    outt[len] = bonus;
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
  // Chunks of 16K bf16 (8K fp32) elements: eight 16-byte loads in flight
  // per thread and a merge fan-in of 8 per 128K-token row
  constexpr int EB = 64, EF = 32;
  const bool bf = p.ldt == ET_BF16;
  const int ce = kScanThreads * (bf ? EB : EF);
  a.S = (p.V + ce - 1) / ce;
  dim3 grid(a.S, p.T, p.B);
  if (bf && vec) accept_kernel<true, true, EB><<<grid, kScanThreads, 0, s>>>(a);
  else if (bf) accept_kernel<true, false, EB><<<grid, kScanThreads, 0, s>>>(a);
  else if (vec) accept_kernel<false, true, EF><<<grid, kScanThreads, 0, s>>>(a);
  else accept_kernel<false, false, EF><<<grid, kScanThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace et
