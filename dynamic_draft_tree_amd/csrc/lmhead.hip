// lmhead.hip -- a draft step taken from the draft model's final hidden
// states: the LM head (logits = h . W^T) on the matrix cores, fused with the
// per-row softmax statistics and top-k, so the logits never reach HBM.
//
// EAGLE-2 summary page, s4.1: a node's confidence is the draft model's
// softmax probability of its token; EAGLE notes, section on the method: the
// draft model reuses the target model's LM head.  What the step computes
// from the logits is et_draft_step's (children = each row's top-k by logit
// then id, conf, value, next frontier); only where the logits come from
// changes.
//
// Three launches.  GEMM: grid (vocab blocks of 512, B), 8 waves; wave w
// owns 64 vocab rows of W (four 16-row tiles of v_mfma_f32_16x16x32_bf16:
// A = 16 rows of W, B = the 16 hidden rows, so a lane ends with one hidden
// row, lane % 16, and 4 consecutive vocab ids per tile).  The k loop keeps
// two groups of four k-steps of loads in flight.  The 16 x 512 fp32 logits
// go through LDS and each kept row publishes its block's (max, sum of exp,
// top-k logit keys).  Reduce: groups of 8 such lists become one.  Merge:
// the draft step's own merge over those lists.  HBM traffic is W once per
// step plus the lists.
#include "device.h"
#include "internal.h"

namespace et {

typedef __bf16 lm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float lm_f32x4_t __attribute__((ext_vector_type(4)));

struct LmArgs {
  const uint16_t* hidden;   // bf16 [B][rows][H], element strides hb, hr
  int64_t hb, hr;
  const uint16_t* W;        // bf16 [V][H]
  DraftWs ws;
  LmWs lm;
  int B, V, k, H, L1, L2, step;
};

// Measured at 128256 x 4096 (per step): 8 waves 207.7 us, 4 waves (256-id
// blocks, twice the lists) 235.2 us; two k-steps per load group 206.8 us;
// non-temporal W loads 225.5 us.
constexpr int kLmWaves = ET_LM_WAVES;   // kLmCols = 64 per wave
constexpr int kLmGroup = 8;             // level-1 lists per level-2 list
constexpr int kLmKG = 4;                // k-steps (of 32) per load group
constexpr float kLmLog2e = 1.4426950408889634f;

__global__ __launch_bounds__(kLmWaves * 64) void lmhead_gemm_kernel(LmArgs a) {
  const int blk = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int arow = lane & 15, kq = (lane >> 4) * 8;
  const int n_wave = blk * kLmCols + wave * 64;
  // B operand: hidden row lane % 16 (rows past k read row k - 1; their
  // outputs are never used); A operand: vocab row n of each tile (ids past
  // V read row V - 1, dropped below).
  const uint16_t* hp = a.hidden + b * a.hb + (int64_t)min(arow, a.k - 1) * a.hr + kq;
  const uint16_t* wp[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    wp[t] = a.W + (int64_t)min(n_wave + 16 * t + arow, a.V - 1) * a.H + kq;
  lm_f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = lm_f32x4_t{0.f, 0.f, 0.f, 0.f};
  lm_bf16x8_t fa[2][kLmKG][4], fb[2][kLmKG];
  auto load = [&](int buf, int k0) {
#pragma unroll
    for (int s = 0; s < kLmKG; ++s) {
      const int kk = k0 + 32 * s;
      fb[buf][s] = *(const lm_bf16x8_t*)(hp + kk);
#pragma unroll
      for (int t = 0; t < 4; ++t) fa[buf][s][t] = *(const lm_bf16x8_t*)(wp[t] + kk);
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kLmKG; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[buf][s][t], fb[buf][s], acc[t], 0, 0, 0);
  };
  const int ng = a.H / (32 * kLmKG);
  load(0, 0);
  for (int g = 0; g < ng; g += 2) {
    if (g + 1 < ng) load(1, (g + 1) * 32 * kLmKG);
    mma(0);
    if (g + 2 < ng) load(0, (g + 2) * 32 * kLmKG);
    if (g + 1 < ng) mma(1);
  }
  // phase: logits computed
  // lane holds hidden row arow, vocab ids n_wave + 16t + 4(lane/16) + e
  __shared__ float s_log[16][kLmCols + 4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_log[arow][wave * 64 + 16 * t + (lane >> 4) * 4 + e] = acc[t][e];
  __syncthreads();
  const int F = a.step == 1 ? 1 : a.ws.frontier_count[((a.step - 1) & 1) * a.B + b];
  const int nrow = min(F, a.k);
  for (int r = wave; r < nrow; r += kLmWaves) {
    float x[kLmCols / 64];
    uint64_t key[kLmCols / 64];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kLmCols / 64; ++i) {
      const int n = blk * kLmCols + lane + 64 * i;
      x[i] = n < a.V ? s_log[r][lane + 64 * i] : -INFINITY;
      key[i] = n < a.V ? logit_key(x[i], (uint32_t)n) : 0;
      m = fmaxf(m, x[i]);
    }
    m = wave_max_f32(m);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kLmCols / 64; ++i)
      s += x[i] > -INFINITY ? __builtin_amdgcn_exp2f((x[i] - m) * kLmLog2e) : 0.f;
    s = wave_sum_f32(s);
    const int64_t li = (int64_t)(b * a.k + r) * a.L1 + blk;
    uint64_t prev = ~0ull;
    for (int q = 0; q < a.k; ++q) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kLmCols / 64; ++i)
        if (key[i] < prev && key[i] > best) best = key[i];
      const uint64_t w = wave_max_u64(best);
      if (lane == 0) a.lm.keys[li * kMaxTopk + q] = w;
      prev = w;
    }
    if (lane == 0) {
      a.lm.m[li] = m;
      a.lm.s[li] = s;
    }
  }
}

// Level-2 lists: wave w of block (x, r, b) merges level-1 lists
// [g * 8, g * 8 + 8) of row r, g = 4x + w, into the draft merge's partial
// layout (keys rank-major [B][k][kMaxTopk][L2]).
__global__ __launch_bounds__(256) void lmhead_reduce_kernel(LmArgs a) {
  const int r = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x * 4 + wave;
  const int F = a.step == 1 ? 1 : a.ws.frontier_count[((a.step - 1) & 1) * a.B + b];
  if (g >= a.L2 || r >= min(F, a.k)) return;
  const int64_t rr = (int64_t)b * a.k + r;
  const int l0 = g * kLmGroup, nl = min(kLmGroup, a.L1 - l0);
  const float ml = lane < nl ? a.lm.m[rr * a.L1 + l0 + lane] : -INFINITY;
  const float sl = lane < nl ? a.lm.s[rr * a.L1 + l0 + lane] : 0.f;
  const float m = wave_max_f32(ml);
  const float s = wave_sum_f32(ml > -INFINITY ? sl * __builtin_amdgcn_exp2f((ml - m) * kLmLog2e) : 0.f);
  uint64_t key[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = lane + 64 * i;  // rank idx % k of list idx / k
    const int l = idx / a.k;
    key[i] = l < nl ? a.lm.keys[(rr * a.L1 + l0 + l) * kMaxTopk + idx % a.k] : 0;
  }
  uint64_t prev = ~0ull;
  for (int q = 0; q < a.k; ++q) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (key[i] < prev && key[i] > best) best = key[i];
    const uint64_t w = wave_max_u64(best);
    if (lane == 0) a.ws.part_keys[(rr * kMaxTopk + q) * a.L2 + g] = w;
    prev = w;
  }
  if (lane == 0) {
    a.ws.part_m[rr * a.L2 + g] = m;
    a.ws.part_s[rr * a.L2 + g] = s;
  }
}

hipError_t launch_draft_step_hidden(const Plan& p, const DraftWs& w, const LmWs& lm, int step,
                                    const int32_t* root_tokens, const void* hidden,
                                    int64_t hb, int64_t hr, const void* lm_head, int H,
                                    int32_t* next_tokens, int32_t* next_count,
                                    hipStream_t s) {
  LmArgs a;
  a.hidden = (const uint16_t*)hidden;
  a.hb = hb;
  a.hr = hr;
  a.W = (const uint16_t*)lm_head;
  a.ws = w;
  a.lm = lm;
  a.B = p.B;
  a.V = p.V;
  a.k = p.k;
  a.H = H;
  a.L1 = lm_lists1(p.V);
  a.L2 = lm_lists2(p.V);
  a.step = step;
  lmhead_gemm_kernel<<<dim3(a.L1, p.B), kLmWaves * 64, 0, s>>>(a);
  lmhead_reduce_kernel<<<dim3((a.L2 + 3) / 4, p.k, p.B), 256, 0, s>>>(a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draft_merge(p, w, step, root_tokens, a.L2, next_tokens, next_count, s);
}

}  // namespace et
