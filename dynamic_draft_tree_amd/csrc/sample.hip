// sample.hip -- stochastic acceptance of the verified tree at temperature > 0.
//
// EAGLE-2 summary page: s2.1, draft tokens are accepted one after another
// by the ratio of target to draft probability; s2.2, a tree lets the
// siblings of a rejected token be tried; s1, the output keeps the target
// model's distribution.  A node's children are its top-k (chosen, not
// sampled), so each is a point-mass proposal: child token t passes with
// probability p(t) over the target mass not yet rejected at the node, and
// when every child fails the bonus token is drawn from the residual (the
// target softmax without the rejected tokens) by inverse CDF in id order.
// p is softmax(x / temperature); weights are exp2((x - max) * c) with
// c = log2(e) / temperature.  Random numbers come in as inputs: u[b][s] for
// the test of slot s, u[b][0] for the bonus draw.
//
// Two launches.  Scan: grid (chunk groups, T slot rows, B), 256 threads.
// Wave w of chunk c owns the contiguous id range ("segment") j = 4c + w of
// 64 * E ids (lane l holds the 16-byte vectors i * 64 + l of it) and
// publishes (segment max m_j, mass of the segment relative to m_j).  Walk:
// one block of 8 waves per sequence stages the segments of all T rows in
// LDS and gathers each slot's token logit at its parent row; wave 0 runs
// the ratio tests level by level (the visited row's max and total mass
// from its segments), then picks the segment of the final row where the
// running residual mass passes u[0] * R; all 8 waves then find the id
// inside it, one 16-byte vector per thread.
//
// Precision.  The inverse CDF maps one uniform onto up to 2^18 ids, so a
// relative error e in the running mass moves the draw by about e * V ids.
// Every sum is fp64; a weight exp2((x - m_j) * c) is fp32, its exponent
// taken with c split into two floats so that its rounding is per element
// rather than one shared bias, and it is the same fp32 value in the scan
// and in the bonus search.  The final row's segment scales
// exp2((m_j - max) * c) are fp64; the ratio tests, which need no such
// resolution, use fp32 scales and masses (one rounding each).
#include <cfloat>
#include <cmath>

#include "device.h"
#include "internal.h"

namespace et {

struct SampleArgs {
  double2* part;           // [B][T][S * 4] (segment max, mass) per segment
  const void* target;
  int64_t bstride, rstride;
  const int32_t* tokens;
  const int32_t* parent_slot;
  const int32_t* n_kept;
  const float* uniforms;   // [B][T]
  double c;                // log2(e) / temperature
  float c_hi, c_lo;        // c as a float pair
  int32_t* accept_len;
  int32_t* path_slots;
  int32_t* out_tokens;
  int B, V, T, D, S, cpb;
};

constexpr int kSegsPerChunk = kScanThreads / 64;

// fp32 weight of logit x against a segment max m: exp2(d * (c_hi + c_lo)),
// d = x - m <= 0.  c_lo is a positive normal float, so d = -inf gives
// -inf + -inf in the exponent and weight 0 with no test.  The hardware
// exp2 (v_exp_f32) flushes results below 2^-126 to zero, which drops less
// than 2^-114 of a 4096-id segment's mass (its maximum has weight 1);
// exp2f's denormal-range scaling would cost five more instructions per
// element.
__device__ __forceinline__ float seg_weight(float x, float m, float c_hi, float c_lo) {
  const float d = x - m;
  return __builtin_amdgcn_exp2f(fmaf(d, c_hi, d * c_lo));
}

// Scan layout: vector i of a lane is at base + (i * 64 + lane) * per (a
// wave's load instruction covers 64 consecutive vectors).  Vector path in
// two halves: issue the loads (a vector past the row end loads the row's
// first vector, in bounds), then widen them (ids past the end rebuilt
// element-wise, -inf beyond the row).
template <bool BF16, int E>
__device__ __forceinline__ void issue_range(const void* row, int base, int V, int lane,
                                            u32x4_t (&raw)[chunk_vectors<BF16, E>()]) {
  constexpr int per = BF16 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < chunk_vectors<BF16, E>(); ++i) {
    const int off = base + (i * 64 + lane) * per;
    const int src = off + per <= V ? off : 0;
    raw[i] = *(const u32x4_t*)((const char*)row + (size_t)src * (BF16 ? 2 : 4));
  }
}
template <bool BF16, int E>
__device__ __forceinline__ void decode_range(const void* row, int base, int V, int lane,
                                             const u32x4_t (&raw)[chunk_vectors<BF16, E>()],
                                             float (&x)[E]) {
  constexpr int per = BF16 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < chunk_vectors<BF16, E>(); ++i) {
    const int off = base + (i * 64 + lane) * per;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (BF16) {
        x[i * 8 + 2 * q] = __uint_as_float(raw[i][q] << 16);
        x[i * 8 + 2 * q + 1] = __uint_as_float(raw[i][q] & 0xFFFF0000u);
      } else {
        x[i * 4 + q] = __uint_as_float(raw[i][q]);
      }
    }
    if (off + per > V) {
#pragma unroll
      for (int u = 0; u < per; ++u)
        x[i * per + u] = off + u < V
            ? (BF16 ? bf16_bits_to_f32(((const uint16_t*)row)[off + u])
                    : ((const float*)row)[off + u])
            : -INFINITY;
    }
  }
}
// Element path (rows not 16-byte aligned), same layout.
template <bool BF16, int E>
__device__ __forceinline__ void load_range_elems(const void* row, int base, int V, int lane,
                                                 float (&x)[E]) {
  constexpr int per = BF16 ? 8 : 4;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int off = base + ((e / per) * 64 + lane) * per + e % per;
    x[e] = off < V ? (BF16 ? bf16_bits_to_f32(((const uint16_t*)row)[off])
                           : ((const float*)row)[off])
                   : -INFINITY;
  }
}

// Element i of one 16-byte vector.
template <bool BF16>
__device__ __forceinline__ float raw_elem1(const u32x4_t& r, int i) {
  if constexpr (BF16) return __uint_as_float(i % 2 ? (r[i / 2] & 0xFFFF0000u) : (r[i / 2] << 16));
  else return __uint_as_float(r[i]);
}

template <bool BF16, bool VEC, int E>
__global__ __launch_bounds__(256) void sample_scan_kernel(SampleArgs a) {
  constexpr int kSeg = 64 * E;
  const int srow = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* row = (const char*)a.target + (b * a.bstride + srow * a.rstride) * (BF16 ? 2 : 4);
  const int c0 = blockIdx.x * a.cpb;
  const int nch = min(a.cpb, a.S - c0);
  float x[E];
  u32x4_t raw[VEC ? chunk_vectors<BF16, E>() : 1];
  // the first range is in flight before n_kept arrives (all T rows are
  // readable memory by contract; rows past n_kept are dropped)
  const int j0 = c0 * kSegsPerChunk + wave;
  // n_kept's address with the arguments the loads need, in one round
  uint64_t u_nk = (uint64_t)a.n_kept;
  asm volatile("" : "+s"(u_nk));
  int nkv = ((const gmem_i32*)u_nk)[b];
  if constexpr (VEC) issue_range<BF16, E>(row, j0 * kSeg, a.V, lane, raw);
  else load_range_elems<BF16, E>(row, j0 * kSeg, a.V, lane, x);
  // (the pins keep the loads ahead of the test and its wait for n_kept)
  pin_loaded<VEC, E>(raw, x);
  asm volatile("" : "+v"(nkv));
  if (srow > __builtin_amdgcn_readfirstlane(nkv)) return;
  double2* out = a.part + ((int64_t)b * a.T + srow) * (a.S * kSegsPerChunk);
  for (int ci = 0; ci < nch; ++ci) {
    const int j = j0 + ci * kSegsPerChunk;
    if constexpr (VEC) {
      decode_range<BF16, E>(row, j * kSeg, a.V, lane, raw, x);
      if (ci + 1 < nch) issue_range<BF16, E>(row, (j + kSegsPerChunk) * kSeg, a.V, lane, raw);
    }
    // phase: chunk loaded
    float t[E];
#pragma unroll
    for (int e = 0; e < E; ++e) t[e] = x[e];
#pragma unroll
    for (int n = E; n > 1; n = (n + 2) / 3)
#pragma unroll
      for (int i = 0; i < (n + 2) / 3; ++i) {
        float m = t[3 * i];
        if (3 * i + 1 < n) m = fmaxf(m, t[3 * i + 1]);
        if (3 * i + 2 < n) m = fmaxf(m, t[3 * i + 2]);
        t[i] = m;
      }
    const float wm = wave_max_f32(t[0]);
    // mass: fp32 sums of 8 weights, fp64 above
    double ls = 0.0;
    if (wm != -INFINITY) {
#pragma unroll
      for (int g = 0; g < E; g += 8) {
        float w8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w8[e] = seg_weight(x[g + e], wm, a.c_hi, a.c_lo);
#pragma unroll
        for (int h = 4; h >= 1; h >>= 1)
#pragma unroll
          for (int e = 0; e < h; ++e) w8[e] += w8[e + h];
        ls += (double)w8[0];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ls += xor_lane_rt(ls, m);
    if (lane == 0) out[j] = make_double2((double)wm, ls);
    if constexpr (!VEC)
      if (ci + 1 < nch) load_range_elems<BF16, E>(row, (j + kSegsPerChunk) * kSeg, a.V, lane, x);
  }
}

// DPP move of a double (both halves with one control); lanes without a
// source, or in rows outside ROW_MASK, get 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Inclusive prefix sum over the wave in lane order: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then lane 15 added to rows 1 and 3 and
// lane 31 to rows 2 and 3.  All lanes must be active.
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

// Scale of a segment's mass to the row max m, exp2((m_j - m) * c): fp64
// where it places the bonus draw, fp32 (one rounding, random per segment)
// for the row totals and ratio tests.
__device__ __forceinline__ double seg_scale(double mj, float m, double c) {
  return mj == -INFINITY ? 0.0 : exp2((mj - (double)m) * c);
}
__device__ __forceinline__ double seg_scale32(float mj, float m, float c_hi, float c_lo) {
  return (double)seg_weight(mj, m, c_hi, c_lo);
}

constexpr int kSampleWalkWaves = 8;
constexpr int kWalkThreads = kSampleWalkWaves * 64;
// (segment max, mass) of all T rows are staged in LDS when they fit
constexpr int kSegStash = 2048;
constexpr int kMaxSegs = kMaxVocab / (kScanThreads * kAccElemsF32) * kSegsPerChunk;

template <bool BF16, bool VEC, int E, bool STASH>
__global__ __launch_bounds__(kWalkThreads) void sample_walk_kernel(SampleArgs a) {
  constexpr int kSeg = 64 * E;
  constexpr int per = BF16 ? 8 : 4;
  static_assert(kSeg == kWalkThreads * per, "a segment is one 16-byte vector per thread");
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_x[kMaxBudget + 1];   // slot's token logit at its parent row
  __shared__ float s_u[kMaxBudget + 1];
  __shared__ int s_tok[kMaxBudget + 1], s_par[kMaxBudget + 1];
  __shared__ float s_seg_m[STASH ? kSegStash : 1];   // [row][segment] max
  __shared__ double s_seg_s[STASH ? kSegStash : 1];  // mass relative to it
  __shared__ double s_fin_w[kMaxSegs];    // final row: residual mass per segment
  __shared__ double s_fin_sc[kMaxSegs];   // and its fp64 scale
  __shared__ int s_ex[kMaxTopk];          // rejected children (slots) of the final slot,
  __shared__ int s_exj[kMaxTopk];         // their segments
  __shared__ double s_exw[kMaxTopk];      // and weights
  __shared__ double s_wsum[kSampleWalkWaves];
  __shared__ int s_first[kSampleWalkWaves], s_last[kSampleWalkWaves];
  __shared__ int s_len, s_nex, s_jsel, s_cur;
  __shared__ double s_tsel;
  const int T = a.T, P = a.S * kSegsPerChunk;
  const size_t esz = BF16 ? 2 : 4;
  const int32_t* tk = a.tokens + (int64_t)b * T;
  const int32_t* ps = a.parent_slot + (int64_t)b * T;
  int32_t* path = a.path_slots + (int64_t)b * (a.D + 1);
  int32_t* outt = a.out_tokens + (int64_t)b * (a.D + 1);
  const double2* pb = a.part + (int64_t)b * T * P;

  // Per slot, for all T slots (no wait on n_kept): token, parent, uniform
  // and the token's logit at the parent row.
  const int nk = a.n_kept[b];
  for (int s = tid; s < T; s += kWalkThreads) {
    const int tok = tk[s], par = ps[s];
    s_tok[s] = tok;
    s_par[s] = par;
    s_u[s] = a.uniforms[(int64_t)b * T + s];
    if (s >= 1) {
      const int pc = min(max(par, 0), T - 1);
      const int tc = min(max(tok, 0), a.V - 1);
      const char* prow = (const char*)a.target + (b * a.bstride + pc * a.rstride) * esz;
      s_x[s] = BF16 ? bf16_bits_to_f32(((const uint16_t*)prow)[tc]) : ((const float*)prow)[tc];
    }
  }
  // The partials of all T rows go to LDS in one round of loads (rows past
  // n_kept hold stale values and are dropped).
  if constexpr (STASH) {
    constexpr int kU = kSegStash / kWalkThreads;
    double2 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = u * kWalkThreads + tid;
      if (i < T * P) v[u] = pb[i];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = u * kWalkThreads + tid;
      if (i < T * P) {
        s_seg_m[i] = (float)v[u].x;
        s_seg_s[i] = v[u].y;
      }
    }
  }
  auto seg_m = [&](int i) { return STASH ? s_seg_m[i] : (float)pb[i].x; };
  auto seg_s = [&](int i) { return STASH ? s_seg_s[i] : pb[i].y; };
  const int n = min(max(nk, 0), T - 1);
  // phase: partials staged
  __syncthreads();

  if (wave == 0) {
    // Ratio tests, one level per iteration.  Lane l holds slots l, l+64, ...
    // (T <= 256).  A child's test assumes every earlier sibling (lower
    // slot) failed, so the first passing sibling is the one accepted.
    int r_tok[4], r_par[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = lane + 64 * i;
      const bool ok = s >= 1 && s <= n;
      r_tok[i] = ok ? s_tok[s] : -1;
      r_par[i] = ok ? s_par[s] : -2;
    }
    // Max and total mass of a row from its segments (visited rows only).
    auto row_stats = [&](int r, float& m, double& z) {
      m = -INFINITY;
      for (int j = lane; j < P; j += 64) m = fmaxf(m, seg_m(r * P + j));
      m = wave_max_f32(m);
      z = 0.0;
      for (int j = lane; j < P; j += 64)
        z += seg_s(r * P + j) * seg_scale32(seg_m(r * P + j), m, a.c_hi, a.c_lo);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) z += xor_lane_rt(z, d);
    };
    if (lane == 0) path[0] = 0;
    int cur = 0, len = 0;
    float mc;
    for (;;) {
      double rb;
      row_stats(cur, mc, rb);
      int acc = -1, acc_tok = -1;
      if (len < a.D) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (64 * i > n) break;
          const int s = lane + 64 * i;
          const bool ch = r_par[i] == cur;
          const double p = ch ? (double)seg_weight(s_x[s], mc, a.c_hi, a.c_lo) : 0.0;
          const double incl = wave_incl_scan_f64(p);
          const bool pass = ch && (double)s_u[s] * (rb - (incl - p)) < p;
          const uint64_t bal = __ballot(pass);
          if (bal) {
            const int l = __ffsll((unsigned long long)bal) - 1;
            acc = 64 * i + l;
            acc_tok = __shfl(r_tok[i], l, 64);
            break;
          }
          rb -= __shfl(incl, 63, 64);
        }
      }
      if (acc < 0) break;
      if (lane == 0) {
        path[len + 1] = acc;
        outt[len] = acc_tok;
      }
      ++len;
      cur = acc;
    }
    // phase: walk done
    for (int i = lane; i <= a.D; i += 64) {
      if (i > len) {
        path[i] = -1;
        outt[i] = -1;
      }
    }
    // The residual excludes the final slot's children (all rejected)
    // unless the depth limit stopped the walk before any test: each child
    // lane lists its slot, segment and weight (as the scan formed it).
    int nex = 0;
    if (len < a.D) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = lane + 64 * i;
        const bool ch = r_par[i] == cur;
        int cnt;
        const int r = ballot_rank(ch, &cnt);
        if (ch && nex + r < kMaxTopk) {
          const int tok = r_tok[i];
          int je = -1;
          double we = 0.0;
          if (tok >= 0 && tok < a.V) {
            je = tok / kSeg;
            const float mje = seg_m(cur * P + je);
            we = (double)seg_weight(s_x[s], mje, a.c_hi, a.c_lo) * seg_scale((double)mje, mc, a.c);
          }
          s_ex[nex + r] = s;
          s_exj[nex + r] = je;
          s_exw[nex + r] = we;
        }
        nex = min(nex + cnt, kMaxTopk);
      }
    }
    wave_lds_fence();
    // Residual mass per segment of the final row with fp64 scales, and
    // their total R; t = u[0] * R.
    double total = 0.0;
    for (int j0 = 0; j0 < P; j0 += 64) {
      const int j = j0 + lane;
      double M = 0.0;
      if (j < P) {
        const float mj = seg_m(cur * P + j);
        const double sc = seg_scale((double)mj, mc, a.c);
        M = seg_s(cur * P + j) * sc;
#pragma unroll
        for (int e = 0; e < kMaxTopk; ++e)
          if (e < nex && s_exj[e] == j) M -= s_exw[e];
        M = fmax(M, 0.0);
        s_fin_w[j] = M;
        s_fin_sc[j] = sc;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) M += xor_lane_rt(M, d);
      total += M;
    }
    wave_lds_fence();
    const double t = (double)s_u[0] * total;
    // segment where the running residual passes t
    double cbase = 0.0, tsel = 0.0;
    int jsel = -1, jlast = -1;
    for (int j0 = 0; j0 < P; j0 += 64) {
      const int j = j0 + lane;
      const double M = j < P ? s_fin_w[j] : 0.0;
      const double incl = wave_incl_scan_f64(M);
      const uint64_t bal = __ballot(M > 0.0 && cbase + incl > t);
      if (bal) {
        const int l = __ffsll((unsigned long long)bal) - 1;
        jsel = j0 + l;
        tsel = t - (cbase + __shfl(incl - M, l, 64));
        break;
      }
      const uint64_t pos = __ballot(M > 0.0);
      if (pos) jlast = j0 + 63 - __clzll((long long)pos);
      cbase += __shfl(incl, 63, 64);
    }
    if (jsel < 0 && jlast >= 0) {
      jsel = jlast;
      tsel = INFINITY;  // the segment's last id of positive mass
    }
    if (lane == 0) {
      s_cur = cur;
      s_len = len;
      s_nex = nex;
      s_jsel = jsel;
      s_tsel = jsel >= 0 ? tsel / s_fin_sc[jsel] : 0.0;  // in unscaled weights
      a.accept_len[b] = len;
    }
  }
  __syncthreads();
  // phase: segment chosen

  // The id inside the segment: thread t holds ids lo .. lo + per - 1, one
  // 16-byte vector; a block-wide prefix of the per-thread masses finds the
  // thread, which then walks its ids.
  const int jsel = s_jsel, len = s_len, nex = s_nex, cur = s_cur;
  if (jsel >= 0) {
    const char* row = (const char*)a.target + (b * a.bstride + cur * a.rstride) * esz;
    const int lo = jsel * kSeg + tid * per;
    const float mj = seg_m(cur * P + jsel);
    const double tsel = s_tsel;
    float x[per];
    if (VEC && lo + per <= a.V) {
      const u32x4_t r = *(const u32x4_t*)(row + (size_t)lo * esz);
#pragma unroll
      for (int i = 0; i < per; ++i) x[i] = raw_elem1<BF16>(r, i);
    } else {
#pragma unroll
      for (int i = 0; i < per; ++i)
        x[i] = lo + i < a.V ? (BF16 ? bf16_bits_to_f32(((const uint16_t*)row)[lo + i])
                                    : ((const float*)row)[lo + i])
                            : -INFINITY;
    }
    // phase: segment loaded
    uint32_t exm = 0;
    for (int e = 0; e < nex; ++e) {
      const int d = s_tok[s_ex[e]] - lo;
      if (d >= 0 && d < per) exm |= 1u << d;
    }
    float w[per];
    int lpos = -1;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      w[i] = (exm >> i) & 1 ? 0.0f : seg_weight(x[i], mj, a.c_hi, a.c_lo);
      if (w[i] > 0.0f) lpos = i;
    }
    double ts = 0.0;
#pragma unroll
    for (int i = 0; i < per; ++i) ts += (double)w[i];
    const double incl = wave_incl_scan_f64(ts);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    double base = incl - ts;
    for (int v = 0; v < wave; ++v) base += s_wsum[v];
    const uint64_t bal = __ballot(ts > 0.0 && base + ts > tsel);
    const uint64_t pos = __ballot(lpos >= 0);
    if (lane == 0) {
      s_first[wave] = bal ? wave * 64 + __ffsll((unsigned long long)bal) - 1 : INT_MAX;
      s_last[wave] = pos ? wave * 64 + 63 - __clzll((long long)pos) : -1;
    }
    __syncthreads();
    int first = INT_MAX, last = -1;
    for (int v = 0; v < kSampleWalkWaves; ++v) {
      first = min(first, s_first[v]);
      last = max(last, s_last[v]);
    }
    if (tid == first) {
      int pick = lo + lpos;  // rounding fallback: the thread's last id of positive mass
      double cum = base;
#pragma unroll
      for (int i = 0; i < per; ++i) {
        if (w[i] > 0.0f) {
          cum += (double)w[i];
          if (cum > tsel) {
            pick = lo + i;
            break;
          }
        }
      }
      outt[len] = pick;
    } else if (first == INT_MAX && tid == last) {
      outt[len] = lo + lpos;
    }
    if (first != INT_MAX || last >= 0) return;
  }
  if (tid == 0) {
    // no residual mass anywhere: the lowest id not rejected
    int pick = 0;
    for (bool again = true; again && pick < a.V - 1;) {
      again = false;
      for (int e = 0; e < nex; ++e)
        if (s_tok[s_ex[e]] == pick) again = true;
      if (again) ++pick;
    }
    outt[len] = pick;
  }
}

hipError_t launch_accept_sample(const Plan& p, const AcceptWs& w, const void* target,
                                int64_t bstride, int64_t rstride, bool vec,
                                const int32_t* tokens, const int32_t* parent_slot,
                                const int32_t* n_kept, double c, const float* uniforms,
                                int32_t* accept_len, int32_t* path_slots,
                                int32_t* out_tokens, hipStream_t s) {
  SampleArgs a;
  a.part = (double2*)w.part;
  a.target = target;
  a.bstride = bstride;
  a.rstride = rstride;
  a.tokens = tokens;
  a.parent_slot = parent_slot;
  a.n_kept = n_kept;
  a.uniforms = uniforms;
  a.c = c;
  // c = c_hi + c_lo with c_hi rounded toward zero, so c_lo >= 0; it is
  // kept a positive normal float (see seg_weight)
  float hi = (float)c;
  if ((double)hi > c) hi = nextafterf(hi, 0.0f);
  a.c_hi = hi;
  a.c_lo = fmaxf((float)(c - (double)hi), FLT_MIN);
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
  const bool stash = p.T * p.s_accept * kSegsPerChunk <= kSegStash;
  dim3 grid((p.s_accept + p.accept_cpb - 1) / p.accept_cpb, p.T, p.B);
#define ET_SAMPLE(BF, VC, E)                                                        \
  do {                                                                              \
    sample_scan_kernel<BF, VC, E><<<grid, kScanThreads, 0, s>>>(a);                 \
    if (stash) sample_walk_kernel<BF, VC, E, true><<<p.B, kWalkThreads, 0, s>>>(a); \
    else sample_walk_kernel<BF, VC, E, false><<<p.B, kWalkThreads, 0, s>>>(a);      \
  } while (0)
  if (bf && vec) ET_SAMPLE(true, true, kAccElemsBf16);
  else if (bf) ET_SAMPLE(true, false, kAccElemsBf16);
  else if (vec) ET_SAMPLE(false, true, kAccElemsF32);
  else ET_SAMPLE(false, false, kAccElemsF32);
#undef ET_SAMPLE
  return hipGetLastError();
}

}  // namespace et
