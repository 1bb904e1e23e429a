// attention.hip -- tree-masked attention: the single verify pass.
//
// EAGLE-2 summary page s4.2: the kept tokens are flattened into one
// sequence with an attention mask that keeps branches apart; explainer
// "EAGLE-2: Dynamic Draft Trees": the chosen tree is verified in a single
// tree-attention pass; EAGLE notes (方法): Medusa-style tree attention.
// Query slot s of sequence b attends to every prefix key and to the tree
// keys of its ancestors and itself (bit t of mask[b][s]).
//
// bf16 path (matrix cores, gfx950 v_mfma_f32_16x16x32_bf16):
//   grid (S splits, q blocks of 64 rows, B * Hkv); 4 waves, 16 rows each.
//   The rows of one kv head are the G query heads of every slot, row
//   r = slot * G + g, so the K/V tile staged in LDS serves G*T queries.
//   Scores are computed transposed, S^T = K . Q^T, which leaves each lane
//   holding one query row (lane % 16) and 4 consecutive keys per 16-key
//   sub-tile; that register layout is directly the B operand of
//   O^T = V^T . P^T when the MFMA's k index is permuted to
//   {4g..4g+3, 16+4g..16+4g+3} (the A operand V^T reads the same keys
//   from a transposed V tile in LDS).  Online softmax in fp32 registers
//   with exp2 and a pre-multiplied log2(e) scale; the ancestor bitmask is
//   tested per key in registers.  With S > 1 each split writes (O, m, l)
//   partials and a merge kernel combines them.
// fp32 path: plain per-row kernel (vector ALU), for fp32 inputs.
#include "device.h"
#include "internal.h"

namespace et {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kt;
  const void* vt;
  const int32_t* prefix_len;
  const uint64_t* mask;
  const int32_t* n_kept;
  void* out;
  float* po;
  float* pm;
  float* pl;
  int B, T, Hq, Hkv, G, Pcap, W, nqb, S;
  float scale, scale_log2;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint64_t pick_word(const uint64_t (&m)[4], int w) {
  return w == 0 ? m[0] : w == 1 ? m[1] : w == 2 ? m[2] : m[3];
}

template <int HD>
__global__ __launch_bounds__(256) void tree_attn_bf16_kernel(AttnArgs a) {
  constexpr int KSTEPS = HD / 32;
  constexpr int DT = HD / 16;
  constexpr int KPAD = HD + 8;
  constexpr int VPAD = kAttnTile + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kAttnTile * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[HD * VPAD];

  const int split = blockIdx.x, qb = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, kvh = bh - b * a.Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int n = a.n_kept[b];
  const int R = (n + 1) * a.G;
  const int RT = a.T * a.G;
  const int row0 = qb * kAttnRows;
  uint16_t* out = (uint16_t*)a.out;

  if (row0 >= R) {
    if (a.S == 1) {
      for (int e = tid; e < kAttnRows * HD; e += 256) {
        int r = row0 + e / HD;
        if (r >= RT) break;
        int slot = r / a.G, gg = r - slot * a.G;
        out[(((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD + e % HD] = 0;
      }
    }
    return;
  }

  const int P = a.prefix_len[b];
  const int ntiles = (P + kAttnTile - 1) / kAttnTile;
  const int t_begin = (int)((int64_t)split * ntiles / a.S);
  const int t_end = (int)((int64_t)(split + 1) * ntiles / a.S);
  const int ntree = (a.T + kAttnTile - 1) / kAttnTile;
  const int nprefix = t_end - t_begin;
  const int total = nprefix + (split == a.S - 1 ? ntree : 0);

  const int r = row0 + wave * 16 + r16;
  const bool rvalid = r < R;
  const int slot = r / a.G, gg = r - slot * a.G;
  bf16x8_t qf[KSTEPS];
  uint64_t mrow[4] = {0, 0, 0, 0};
  {
    const uint16_t* qr = (const uint16_t*)a.q +
                         (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (rvalid) {
        qf[kk] = *(const bf16x8_t*)(qr + kk * 32 + g * 8);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[kk][i] = (__bf16)0.0f;
      }
    }
    if (rvalid) {
      const uint64_t* mr = a.mask + ((int64_t)b * a.T + slot) * a.W;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (w < a.W) mrow[w] = mr[w];
    }
  }

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t kvb = (int64_t)b * a.Hkv + kvh;
  const uint16_t* kcb = (const uint16_t*)a.kc + kvb * a.Pcap * HD;
  const uint16_t* vcb = (const uint16_t*)a.vc + kvb * a.Pcap * HD;
  const uint16_t* ktb = (const uint16_t*)a.kt + kvb * a.T * HD;
  const uint16_t* vtb = (const uint16_t*)a.vt + kvb * a.T * HD;

  // K/V tiles are staged global -> registers -> LDS; the loads of tile
  // it+1 are issued before tile it is computed so their latency overlaps.
  constexpr int CH = kAttnTile * (HD / 8) / 256;  // 16-byte chunks per thread
  uint4 kreg[CH], vreg[CH];
  auto load_tile = [&](int it) {
    const bool tr = it >= nprefix;
    const int k0 = (tr ? it - nprefix : t_begin + it) * kAttnTile;
    const int km = tr ? a.T : P;
    const uint16_t* Kg = tr ? ktb : kcb;
    const uint16_t* Vg = tr ? vtb : vcb;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i;
      const int kk = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      kreg[i] = make_uint4(0u, 0u, 0u, 0u);
      vreg[i] = make_uint4(0u, 0u, 0u, 0u);
      if (k0 + kk < km) {
        kreg[i] = *(const uint4*)(Kg + (int64_t)(k0 + kk) * HD + d0);
        vreg[i] = *(const uint4*)(Vg + (int64_t)(k0 + kk) * HD + d0);
      }
    }
  };
  if (total > 0) load_tile(0);

  for (int it = 0; it < total; ++it) {
    const bool tree = it >= nprefix;
    const int tile = tree ? it - nprefix : t_begin + it;
    const int key0 = tile * kAttnTile;

    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i;
      const int kk = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      *(uint4*)&sK[kk * KPAD + d0] = kreg[i];
      const uint32_t w4[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sVt[(d0 + 2 * q) * VPAD + kk] = (uint16_t)(w4[q] & 0xFFFFu);
        sVt[(d0 + 2 * q + 1) * VPAD + kk] = (uint16_t)(w4[q] >> 16);
      }
    }
    __syncthreads();
    if (it + 1 < total) load_tile(it + 1);

    // S^T = K . Q^T: lane holds row r16, keys sub*16 + 4g + i.
    f32x4_t sacc[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      sacc[sub] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        bf16x8_t af = *(const bf16x8_t*)&sK[(sub * 16 + r16) * KPAD + kk * 32 + g * 8];
        sacc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[kk], sacc[sub], 0, 0, 0);
      }
    }

    float sc[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + sub * 16 + g * 4 + i;
        bool ok;
        if (tree) ok = (pick_word(mrow, key >> 6) >> (key & 63)) & 1ull;
        else ok = key < P;
        float v = ok ? sacc[sub][i] * a.scale_log2 : -INFINITY;
        sc[sub][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, xor_lane<16>(tmax));
    tmax = fmaxf(tmax, xor_lane<32>(tmax));
    // Branch-free: a row that has seen no visible key yet keeps m = -inf,
    // alpha = 1 and p = 0 (the matrix instructions below need all lanes).
    const float m_new = fmaxf(m_run, tmax);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t pf[2];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = none ? 0.f : exp2f(sc[sub][i] - m_new);
        psum += p;
        pf[sub >> 1][(sub & 1) * 4 + i] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // O^T += V^T . P^T over two 32-key steps.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = &sVt[(dt * 16 + r16) * VPAD + ks * 32 + g * 4];
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 16);
        bf16x8_t af;
        uint32_t* afw = (uint32_t*)&af;
        afw[0] = lo.x;
        afw[1] = lo.y;
        afw[2] = hi.x;
        afw[3] = hi.y;
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[ks], oacc[dt], 0, 0, 0);
      }
  }

  l_run += xor_lane<16>(l_run);
  l_run += xor_lane<32>(l_run);
  if (r >= RT) return;
  if (a.S == 1) {
    uint16_t* orow = out + (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD;
    const float inv = (rvalid && l_run > 0.f) ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16_rne(oacc[dt][0] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16_rne(oacc[dt][2] * inv) |
            ((uint32_t)f32_to_bf16_rne(oacc[dt][3] * inv) << 16);
      *(uint2*)(orow + dt * 16 + g * 4) = w;
    }
  } else {
    const int64_t pr = ((int64_t)(bh * a.nqb + qb) * a.S + split) * kAttnRows +
                       wave * 16 + r16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *(f32x4_t*)(a.po + pr * HD + dt * 16 + g * 4) = oacc[dt];
    if (g == 0) {
      a.pm[pr] = m_run;
      a.pl[pr] = l_run;
    }
  }
}

// Combine the S split partials: o = sum_i O_i 2^(m_i - m) / l.  Grid
// (nqb * 16, B * Hkv); a block covers 4 rows; thread = (row, 4 columns).
// All of a thread's loads are independent, so they are issued together.
template <int HD>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a) {
  constexpr int TPR = HD / 4;            // threads per row
  constexpr int RPB = 256 / TPR;         // rows per block
  const int qb = blockIdx.x / (kAttnRows / RPB);
  const int rr = (blockIdx.x % (kAttnRows / RPB)) * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv, kvh = bh - b * a.Hkv;
  const int r = qb * kAttnRows + rr;
  const int RT = a.T * a.G;
  if (r >= RT) return;
  const int R = (a.n_kept[b] + 1) * a.G;
  const int slot = r / a.G, gg = r - slot * a.G;
  uint16_t* orow = (uint16_t*)a.out +
                   (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD + col;
  if (r >= R) {
    *(uint2*)orow = make_uint2(0u, 0u);
    return;
  }
  const int64_t base = (int64_t)(bh * a.nqb + qb) * a.S;
  constexpr int kMaxS = 64;
  float m = -INFINITY;
  for (int i = 0; i < a.S; ++i) m = fmaxf(m, a.pm[(base + i) * kAttnRows + rr]);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int i = 0; i < kMaxS; ++i) {
    if (i >= a.S) break;
    const int64_t pr = (base + i) * kAttnRows + rr;
    const float mi = a.pm[pr];
    const float f = mi == -INFINITY ? 0.f : exp2f(mi - m);
    const float4 v = *(const float4*)(a.po + pr * HD + col);
    l += a.pl[pr] * f;
    acc.x += v.x * f;
    acc.y += v.y * f;
    acc.z += v.z * f;
    acc.w += v.w * f;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint2 w;
  w.x = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  w.y = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  *(uint2*)orow = w;
}

// fp32 inputs: one block per (slot, q head, sequence), keys in chunks of
// 256 with an online softmax; thread t < d accumulates output element t.
__global__ __launch_bounds__(256) void tree_attn_f32_kernel(AttnArgs a, int HD) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  __shared__ float sq[128];
  __shared__ float sp[256];
  __shared__ float sred[4];
  float* out = (float*)a.out + (((int64_t)b * a.T + s) * a.Hq + h) * HD;
  const int n = a.n_kept[b];
  if (s > n) {
    if (tid < HD) out[tid] = 0.f;
    return;
  }
  const int kvh = h / a.G;
  const float* qr = (const float*)a.q + (((int64_t)b * a.T + s) * a.Hq + h) * HD;
  if (tid < HD) sq[tid] = qr[tid];
  const int64_t kvb = (int64_t)b * a.Hkv + kvh;
  const float* kc = (const float*)a.kc + kvb * a.Pcap * HD;
  const float* vc = (const float*)a.vc + kvb * a.Pcap * HD;
  const float* kt = (const float*)a.kt + kvb * a.T * HD;
  const float* vt = (const float*)a.vt + kvb * a.T * HD;
  const uint64_t* mrow = a.mask + ((int64_t)b * a.T + s) * a.W;
  const int P = a.prefix_len[b];
  const int nkeys = P + a.T;
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  for (int c0 = 0; c0 < nkeys; c0 += 256) {
    const int j = c0 + tid;
    float sc = -INFINITY;
    if (j < nkeys) {
      const float* kr = nullptr;
      if (j < P) {
        kr = kc + (int64_t)j * HD;
      } else {
        const int t = j - P;
        if ((mrow[t >> 6] >> (t & 63)) & 1ull) kr = kt + (int64_t)t * HD;
      }
      if (kr) {
        float dot = 0.f;
        for (int d = 0; d < HD; ++d) dot = fmaf(sq[d], kr[d], dot);
        sc = dot * a.scale;
      }
    }
    float cm = wave_max_f32(sc);
    if ((tid & 63) == 0) sred[tid >> 6] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, cm);
    const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
    const float p = m_new == -INFINITY ? 0.f : expf(sc - m_new);
    sp[tid] = p;
    float ps = wave_sum_f32(p);
    if ((tid & 63) == 0) sred[tid >> 6] = ps;
    __syncthreads();
    ps = sred[0] + sred[1] + sred[2] + sred[3];
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (tid < HD) {
      o *= alpha;
      const int lim = nkeys - c0 < 256 ? nkeys - c0 : 256;
      for (int jj = 0; jj < lim; ++jj) {
        const float pj = sp[jj];
        if (pj == 0.f) continue;
        const int j2 = c0 + jj;
        const float* vr = j2 < P ? vc + (int64_t)j2 * HD : vt + (int64_t)(j2 - P) * HD;
        o = fmaf(pj, vr[tid], o);
      }
    }
    __syncthreads();
  }
  if (tid < HD) out[tid] = o / l_run;
}

hipError_t launch_tree_attention(const Plan& p, const AttnWs& w,
                                 const void* q, const void* kc,
                                 const void* vc, const void* kt,
                                 const void* vt, const int32_t* prefix_len,
                                 const uint64_t* mask, const int32_t* n_kept,
                                 float scale, void* out, hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.kt = kt;
  a.vt = vt;
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.n_kept = n_kept;
  a.out = out;
  a.po = w.o;
  a.pm = w.m;
  a.pl = w.l;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Pcap = p.Pcap;
  a.W = p.W;
  a.nqb = p.attn_nqb;
  a.S = p.attn_splits;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (p.qdt == ET_F32) {
    tree_attn_f32_kernel<<<dim3(p.T, p.Hq, p.B), 256, 0, s>>>(a, p.HD);
    return hipGetLastError();
  }
  dim3 grid(p.attn_splits, p.attn_nqb, p.B * p.Hkv);
  if (p.HD == 128) tree_attn_bf16_kernel<128><<<grid, 256, 0, s>>>(a);
  else tree_attn_bf16_kernel<64><<<grid, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.attn_splits == 1) return e;
  dim3 mgrid(p.attn_nqb * (kAttnRows / (256 / (p.HD / 4))), p.B * p.Hkv);
  if (p.HD == 128) tree_attn_merge_kernel<128><<<mgrid, 256, 0, s>>>(a);
  else tree_attn_merge_kernel<64><<<mgrid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace et
