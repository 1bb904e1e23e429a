// device.h -- wave64 primitives and ordering keys shared by the kernels.
#pragma once

#include <cfloat>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace et {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Order-preserving map of a non-NaN float onto uint32 (-0 and +0 equal).
__device__ __forceinline__ uint32_t ordered_f32(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Logit key: larger logit first, then lower token id.  0 = "no element".
__device__ __forceinline__ uint64_t logit_key(float x, uint32_t id) {
  return ((uint64_t)ordered_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ float logit_of(uint64_t key) {
  return unordered_f32((uint32_t)(key >> 32));
}
__device__ __forceinline__ uint32_t id_of(uint64_t key) {
  return 0xFFFFFFFFu - (uint32_t)key;
}

// Pool key: larger value, then shallower depth, then lower token, then
// earlier creation.  value in [0, 1] needs 30 bits, depth <= 15 needs 4,
// token < 2^18 needs 18, pool index <= 4095 needs 12: 64 in total.
__device__ __forceinline__ uint64_t pool_key(float value, int depth,
                                             int token, int idx) {
  return ((uint64_t)__float_as_uint(value) << 34) |
         ((uint64_t)(15 - depth) << 30) |
         ((uint64_t)((1 << 18) - 1 - token) << 12) | (uint64_t)(4095 - idx);
}
__device__ __forceinline__ int pool_index_of(uint64_t key) {
  return 4095 - (int)(key & 0xFFFu);
}
__device__ __forceinline__ float pool_value_of(uint64_t key) {
  return __uint_as_float((uint32_t)(key >> 34));
}
__device__ __forceinline__ int pool_token_of(uint64_t key) {
  return (1 << 18) - 1 - (int)((key >> 12) & 0x3FFFFu);
}

// ---- cross-lane exchange without LDS traffic -----------------------------
// xor_lane<M>(v) returns the value of lane (lane ^ M).  Within a 16-lane
// row: DPP quad_perm (M = 1, 2), row_ror (M = 8; M = 4 picks row_ror:4 or
// row_ror:12 by lane bit 2, since row_ror:n reads lane (i - n) mod 16).
// Across rows: v_permlane16_swap / v_permlane32_swap, whose two results
// hold the lower / upper partner row or half; lane bit 4 / 5 picks one.
// All lanes of the wave must be active.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int iv = (int)v;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false);
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x12C, 0xF, 0xF, false);
    return (threadIdx.x & 4) ? dn : up;
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, iv, 0x128, 0xF, 0xF, false);
  } else if constexpr (M == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? (uint32_t)r[0] : (uint32_t)r[1];
  } else {
    static_assert(M == 32, "xor distance");
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? (uint32_t)r[0] : (uint32_t)r[1];
  }
}
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  return __uint_as_float(xor_lane<M>(__float_as_uint(v)));
}
template <int M>
__device__ __forceinline__ int xor_lane(int v) {
  return (int)xor_lane<M>((uint32_t)v);
}
template <int M>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v) {
  const uint32_t lo = xor_lane<M>((uint32_t)v);
  const uint32_t hi = xor_lane<M>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int M>
__device__ __forceinline__ double xor_lane(double v) {
  return __longlong_as_double((long long)xor_lane<M>((uint64_t)__double_as_longlong(v)));
}
// Runtime distance (a compile-time constant after unrolling).
template <typename T>
__device__ __forceinline__ T xor_lane_rt(T v, int m) {
  switch (m) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
  }
}

// Butterfly reductions: every lane ends with the same result.
// Reductions with lane l ^ 16 (M = 16) or l ^ 32 (M = 32): a row (half)
// swap of v with itself leaves, in its two result registers, v and the
// partner's value in an order that depends on the lane, so a symmetric
// combination of the two needs no select.  The maximum is taken as the
// median of the two and FLT_MAX, which needs no canonicalising of its
// operands (values are finite or -inf: no NaN, no +inf).  Results equal
// those of combining v with xor_lane<M>(v).
template <int M>
__device__ __forceinline__ void xor_rows_pair(uint32_t v, uint32_t* a, uint32_t* b) {
  static_assert(M == 16 || M == 32, "row distance");
  if constexpr (M == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    *a = (uint32_t)r[0];
    *b = (uint32_t)r[1];
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    *a = (uint32_t)r[0];
    *b = (uint32_t)r[1];
  }
}
template <int M>
__device__ __forceinline__ float max_xor_rows(float v) {
  uint32_t a, b;
  xor_rows_pair<M>(__float_as_uint(v), &a, &b);
  return __builtin_amdgcn_fmed3f(__uint_as_float(a), __uint_as_float(b), FLT_MAX);
}
template <int M>
__device__ __forceinline__ float sum_xor_rows(float v) {
  uint32_t a, b;
  xor_rows_pair<M>(__float_as_uint(v), &a, &b);
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = max_xor_rows<32>(v);
  v = max_xor_rows<16>(v);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = fmaxf(v, xor_lane_rt(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = sum_xor_rows<32>(v);
  v = sum_xor_rows<16>(v);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += xor_lane_rt(v, m);
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  uint32_t a, b;
  xor_rows_pair<32>(v, &a, &b);
  v = min(a, b);
  xor_rows_pair<16>(v, &a, &b);
  v = min(a, b);
  v = min(v, xor_lane<8>(v));
  v = min(v, xor_lane<4>(v));
  v = min(v, xor_lane<2>(v));
  return min(v, xor_lane<1>(v));
}
template <int M>
__device__ __forceinline__ uint64_t max_xor_rows(uint64_t v) {
  uint32_t alo, blo, ahi, bhi;
  xor_rows_pair<M>((uint32_t)v, &alo, &blo);
  xor_rows_pair<M>((uint32_t)(v >> 32), &ahi, &bhi);
  const uint64_t a = ((uint64_t)ahi << 32) | alo, b = ((uint64_t)bhi << 32) | blo;
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_xor_rows<32>(v);
  v = max_xor_rows<16>(v);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    const uint64_t o = xor_lane_rt(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Rank of this lane among the lanes whose `pred` is set, and their count.
__device__ __forceinline__ int ballot_rank(bool pred, int* count) {
  const uint64_t m = __ballot(pred);
  *count = __popcll(m);
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the wave of small non-negative values (below
// 2^BITS), from one ballot per bit plane (each a round trip through the
// scalar unit, so BITS is kept to what the values need); *total receives
// the wave sum.
template <int BITS>
__device__ __forceinline__ int wave_excl_prefix_small(int v, int* total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int bit = 0; bit < BITS; ++bit) {
    int cnt;
    const int r = ballot_rank((v >> bit) & 1, &cnt);
    pre += r << bit;
    tot += cnt << bit;
  }
  *total = tot;
  return pre;
}

// Block barrier for LDS data only: each wave waits for its own LDS
// operations, then all waves meet.  Unlike __syncthreads it does not wait
// for outstanding global memory operations (__syncthreads waits for every
// global store of the block to be acknowledged, about a microsecond).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS writes of this wave visible to its later LDS reads, without waiting
// for outstanding global loads.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// ---- row chunk loader shared by the vocab scans ---------------------------
constexpr int kLoadThreads = 256;
// Element e of a thread's E lies at chunk offset elem_off(e): 16-byte
// vectors of `per` elements, vector v of thread t at (v * 256 + t) * per.
// The scalar path (rows not 16-byte aligned) uses the same mapping so the
// per-thread sums, and hence every output bit, do not depend on alignment.
template <bool BF16>
__device__ __forceinline__ int elem_off(int e, int tid) {
  constexpr int per = BF16 ? 8 : 4;
  return ((e / per) * kLoadThreads + tid) * per + (e % per);
}

// Global-memory (address space 1) element types, for pointers that come
// back from an asm statement as integers: loads through them stay global
// loads rather than flat ones.
typedef __attribute__((address_space(1))) int32_t gmem_i32;
typedef __attribute__((address_space(1))) float gmem_f32;
typedef __attribute__((address_space(1))) uint16_t gmem_u16;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte vectors a thread holds for E elements of a chunk
template <bool BF16, int E>
constexpr int chunk_vectors() { return E / (BF16 ? 8 : 4); }

// Holds the values of a chunk's loads (raw on the vector path, x on the
// element path) in registers at this point, so a test that follows cannot
// be moved by the compiler in front of the loads' issue.
template <bool VEC, int E, int NV>
__device__ __forceinline__ void pin_loaded(u32x4_t (&raw)[NV], float (&x)[E]) {
  if constexpr (VEC) {
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" : "+v"(raw[i]));
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) asm volatile("" : "+v"(x[e]));
  }
}

// Vector path, first half: issue the thread's 16-byte loads of the chunk
// at `base`.  A vector that runs past the row end loads the row's first
// vector instead (in bounds, as the vector path needs V >= per); the
// decode redoes it element-wise.
template <bool BF16, int E>
__device__ __forceinline__ void issue_chunk(const void* row, int base, int V, int tid,
                                            u32x4_t (&raw)[chunk_vectors<BF16, E>()]) {
  constexpr int per = BF16 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < chunk_vectors<BF16, E>(); ++i) {
    const int off = base + (i * kLoadThreads + tid) * per;
    const int src = off + per <= V ? off : 0;
    raw[i] = *(const u32x4_t*)((const char*)row + (size_t)src * (BF16 ? 2 : 4));
  }
}

// Vector path, second half: widen the loaded vectors to fp32 (elements
// past the row end become -inf).
template <bool BF16, int E>
__device__ __forceinline__ void decode_chunk(const void* row, int base, int V, int tid,
                                             const u32x4_t (&raw)[chunk_vectors<BF16, E>()],
                                             float (&x)[E]) {
  constexpr int per = BF16 ? 8 : 4;
  constexpr int NV = chunk_vectors<BF16, E>();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int off = base + (i * kLoadThreads + tid) * per;
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

// Vector path, tail: a vector that runs past the row end is rebuilt in
// place from element loads, elements past the end becoming -inf.
template <bool BF16, int E>
__device__ __forceinline__ void fix_chunk_tail(const void* row, int base, int V, int tid,
                                               u32x4_t (&raw)[chunk_vectors<BF16, E>()]) {
  constexpr int per = BF16 ? 8 : 4;
#pragma unroll
  for (int i = 0; i < chunk_vectors<BF16, E>(); ++i) {
    const int off = base + (i * kLoadThreads + tid) * per;
    if (off + per > V) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          const uint16_t* r16 = (const uint16_t*)row;
          const uint32_t lo = off + 2 * q < V ? r16[off + 2 * q] : 0xFF80u;
          const uint32_t hi = off + 2 * q + 1 < V ? r16[off + 2 * q + 1] : 0xFF80u;
          raw[i][q] = lo | (hi << 16);
        } else {
          raw[i][q] = off + q < V ? ((const uint32_t*)row)[off + q] : 0xFF800000u;
        }
      }
    }
  }
}

template <bool BF16, bool VEC, int E>
__device__ __forceinline__ void load_chunk(const void* row, int base, int V,
                                           int tid, float (&x)[E]) {
  if constexpr (VEC) {
    // all vector loads are issued before any is used
    u32x4_t raw[chunk_vectors<BF16, E>()];
    issue_chunk<BF16, E>(row, base, V, tid, raw);
    decode_chunk<BF16, E>(row, base, V, tid, raw, x);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int off = base + elem_off<BF16>(e, tid);
      x[e] = off < V ? (BF16 ? bf16_bits_to_f32(((const uint16_t*)row)[off])
                             : ((const float*)row)[off])
                     : -INFINITY;
    }
  }
}

}  // namespace et
