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
//   A unit is one kv head of one sequence; its rows are the G query heads
//   of every slot, row r = slot * G + g, so a K/V tile staged in LDS serves
//   G*T queries.  Rows are cut into blocks of 64*WR (4 waves, 16*WR rows
//   each) and the unit's key tiles (prefix tiles, then tree tiles) into S
//   contiguous splits; one block per (unit, row block, split).  Block i
//   runs on XCD i % 8, so the launch maps every block of a unit to one XCD
//   and the unit's row blocks share its K/V tiles through that XCD's L2
//   (split partials do not stay there: the end of the launch writes them
//   back, and the merge reads them from beyond the L2).  When the
//   grid is larger than the chip holds at once, units are taken in order
//   of their sequence's prefix length, longest first (up to 64 sequences
//   each wave ranks the batch itself, above that a one-block kernel does),
//   so that the blocks left for the end are short.
//   Scores are computed transposed, S^T = K . Q^T, which leaves each lane
//   holding one query row (lane % 16) and 4 consecutive keys per 16-key
//   sub-tile; that register layout is directly the B operand of
//   O^T = V^T . P^T when the MFMA's k index is permuted to
//   {4g..4g+3, 16+4g..16+4g+3}.  The A operand V^T is read from the
//   row-major V tile with the LDS transpose read (ds_read_b64_tr_b16: in
//   each 16-lane group, lane j receives element j % 4 of the 8-byte words
//   addressed by lanes j/4, 4+j/4, 8+j/4, 12+j/4), so no transposed copy
//   of V is ever written.  K/V tiles are double- (128-row blocks: triple-)
//   buffered in LDS with one barrier per tile; the next tiles' global loads
//   are in flight while the current one is computed.  The tile loop runs
//   one step per buffer per trip, so every LDS read is a fixed register
//   plus an immediate offset, and the whole prefix tiles take a loop of
//   their own, without masks or row clamping.
//   Online softmax in fp32 registers with exp2
//   and a pre-multiplied log2(e) scale; the ancestor bitmask word of a tree
//   tile is tested per key in registers.  With S > 1 each split writes
//   (O, m, l) partials and a merge kernel combines them.
// fp32 path: plain per-row kernel (vector ALU), for fp32 inputs.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace et {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kt;
  const void* vt;
  const int32_t* prefix_len;
  const uint64_t* mask;
  const int32_t* n_kept;
  const int32_t* order;  // sequence of unit-sequence b0, or null (b = b0)
  int rank_inline;       // no order array: each wave ranks the batch (B <= 64);
                         // 1: keys below 2^20, 2: any keys, 0: off
  void* out;
  float* po;
  float* pm;
  float* pl;
  int B, T, Hq, Hkv, G, Pcap, W, nqb, S;
  int interleave;  // block qb holds row groups qb, qb + nqb, ... (WR = 1, S = 1)
  float scale, scale_log2;
};

// Global-memory (address space 1) vector types.
typedef __attribute__((address_space(1))) f32x4_t gmem_f32x4;
typedef __attribute__((address_space(1))) u32x2_t gmem_u32x2;

// Growth of a row's max (log2 units) tolerated before O is rescaled.
constexpr float kSlack = 8.0f;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint64_t pick_word(const uint64_t (&m)[4], int w) {
  return w == 0 ? m[0] : w == 1 ? m[1] : w == 2 ? m[2] : m[3];
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b16 at an LDS byte address plus an immediate offset.
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
  u32x2_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// s_waitcnt lgkmcnt(0) that the compiler sees as producing the values of
// the transpose reads issued before it.
__device__ __forceinline__ void lds_wait_all(u32x2_t (&x)[8], u32x2_t (&y)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]),
                 "+v"(x[5]), "+v"(x[6]), "+v"(x[7]), "+v"(y[0]), "+v"(y[1]),
                 "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]),
                 "+v"(y[7]));
}
__device__ __forceinline__ void lds_wait_all(u32x2_t (&x)[4], u32x2_t (&y)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(y[0]),
                 "+v"(y[1]), "+v"(y[2]), "+v"(y[3]));
}

// ds_read_b128 at an LDS byte address plus an immediate offset (assembly,
// like the transpose reads, so the compiler does not hold it behind the
// direct loads still filling another buffer).
template <int OFF>
__device__ __forceinline__ bf16x8_t ds_read_b128_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
// s_waitcnt lgkmcnt(0) that the compiler sees as producing the K fragments.
__device__ __forceinline__ void lds_wait_k(bf16x8_t (&x)[4][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]),
                 "+v"(x[2][0]), "+v"(x[2][1]), "+v"(x[3][0]), "+v"(x[3][1]));
}
__device__ __forceinline__ void lds_wait_k(bf16x8_t (&x)[2][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]));
}

// 16 bytes per lane from global memory straight into a 1 KB LDS slab
// (lane i writes bytes 16i..16i+15; `slab` must be wave-uniform).  A plain
// device function, so that kernel templates calling it still instantiate
// in the host pass.
__device__ __forceinline__ void load_lds16(const void* src, void* slab) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)slab, 16, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector memory loads are
// outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// Block index -> (unit, row block, split) with every block of a unit on
// XCD unit % 8.  Returns false for the padding blocks past the last unit.
__device__ __forceinline__ bool attn_block_coords(int i, int units, int per_unit,
                                                  int* unit, int* rem) {
  const int xcd = i & 7, j = i >> 3;
  const int u = xcd + 8 * (j / per_unit);
  *unit = u;
  *rem = j - (j / per_unit) * per_unit;
  return u < units;
}

// The sequence of rank r (0-based) when a batch of B <= 64 sequences, one
// per lane, is ordered by prefix length, longest first, ties by index: the
// (r + 1)-th largest of the distinct keys length * 64 + 63 - index, found
// bit by bit from the top with one ballot per bit.  NBITS: the keys'
// width (20 when every prefix length is below 2^14, else 32).  Whatever
// the lengths, the result is clamped to a lane below B.
template <int NBITS>
__device__ __forceinline__ int sequence_of_rank(const int32_t* prefix_len, int B, int r) {
  const int lane = threadIdx.x & 63;
  const uint32_t key = lane < B ? ((uint32_t)prefix_len[lane] << 6) | (uint32_t)(63 - lane) : 0u;
  uint32_t t = 0;
#pragma unroll
  for (int bit = NBITS - 1; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (__popcll(__ballot(key >= cand)) > r) t = cand;
  }
  return min(63 - (int)(t & 63u), B - 1);
}

__device__ __forceinline__ void barrier_no_fence() {
  // s_barrier alone: the direct loads still in flight into another buffer
  // need no fence here (each wave waits for its own loads with an explicit
  // vmcnt before the barrier that publishes them)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// NB LDS tile buffers, prefetch distance NB - 1.  NB = 2 halves the LDS
// so that two blocks share a compute unit (four waves per SIMD, which hide
// each other's LDS and matrix latencies) when the registers allow it.
template <int HD, int WR, int NB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NB == 2 ? 4 : 2)))
void tree_attn_bf16_kernel(AttnArgs a) {
  constexpr int KSTEPS = HD / 32;  // 32-wide d steps of K . Q^T
  constexpr int DT = HD / 16;      // 16-wide d tiles of O
  constexpr int TE = kAttnTile * HD;  // elements of one K (or V) tile
  constexpr int CPR = HD / 8;      // 16-byte chunks per key row
  constexpr int CH = kAttnTile * CPR / 64 / 8;  // 1 KB slabs per wave per tile
  constexpr int PD = NB - 1;       // prefetch distance
  constexpr int BR = 64 * WR;      // query rows per block
  // [K or V][buffer][tile]: the K tiles, then the V tiles, so that every
  // read of a buffer is one per-lane address plus an immediate offset
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2][NB][TE];
  __shared__ uint64_t sMask[4][BR];  // [tree tile][row of the block]

  // The arguments that pick the block's sequence in one round of scalar
  // loads, then its kept count and prefix length in one round (pointers
  // pass the asm as integers and come back as global-memory pointers).
  int nB = a.B, nHkv = a.Hkv, nqbs = a.nqb, nS = a.S, rank_inline = a.rank_inline;
  uint64_t u_order = (uint64_t)a.order, u_nk = (uint64_t)a.n_kept, u_pl = (uint64_t)a.prefix_len;
  asm volatile("" : "+s"(nB), "+s"(nHkv), "+s"(nqbs), "+s"(nS), "+s"(rank_inline), "+s"(u_order),
               "+s"(u_nk), "+s"(u_pl));
  int unit, rem;
  if (!attn_block_coords(blockIdx.x, nB * nHkv, nqbs * nS, &unit, &rem)) return;
  const int qb = rem / nS, split = rem - qb * nS;
  const int b0 = unit / nHkv, kvh = unit - b0 * nHkv;
  const int b = __builtin_amdgcn_readfirstlane(
      u_order ? ((const gmem_i32*)u_order)[b0]
              : rank_inline == 1 ? sequence_of_rank<20>(a.prefix_len, nB, b0)
              : rank_inline ? sequence_of_rank<32>(a.prefix_len, nB, b0) : b0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rg = wave & 3, kh = wave >> 2;  // row group, key half of a tile
  const int r16 = lane & 15, g = lane >> 4;
  int n = __builtin_amdgcn_readfirstlane(((const gmem_i32*)u_nk)[b]);
  int P = __builtin_amdgcn_readfirstlane(((const gmem_i32*)u_pl)[b]);
  asm volatile("" : "+s"(n), "+s"(P));
  const int R = (n + 1) * a.G;
  const int RT = a.T * a.G;
  const int row0 = qb * BR;
  // The unit row of the block's row rr (rr < BR).  Interleaved (64-row
  // blocks without key splits), block qb holds the 16-row groups qb,
  // qb + nqb, ...: the kept rows then spread evenly over a unit's blocks,
  // which walk its tiles at one pace and share them through the L2
  // (contiguous, a last block with few kept rows ran ahead of the others).
  const bool inter = a.interleave;
  auto row_of = [&](int rr) {
    return inter ? 16 * (qb + a.nqb * (rr >> 4)) + (rr & 15) : row0 + rr;
  };
  uint16_t* out = (uint16_t*)a.out;

  if (row_of(0) >= R) {
    // rows of unkept slots: zero output (the merge does it when S > 1)
    if (a.S == 1) {
      for (int e = tid; e < BR * (HD / 4); e += 512) {
        const int r = row_of(e / (HD / 4));
        if (r >= RT) break;
        const int slot = r / a.G, gg = r - slot * a.G;
        *(uint2*)(out + (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD +
                  (e % (HD / 4)) * 4) = make_uint2(0u, 0u);
      }
    }
    return;
  }

  const int tp = (P + kAttnTile - 1) / kAttnTile;
  const int tt = (n + 1 + kAttnTile - 1) / kAttnTile;
  const int tot = tp + tt;
  const int t_begin = (int)((int64_t)split * tot / a.S);
  const int cnt = (int)((int64_t)(split + 1) * tot / a.S) - t_begin;

  // Prologue loads are unconditional (row and key indexes are clamped to
  // valid data, whose results are then masked or never stored), so every
  // path into the tile loop has the same loads outstanding and the
  // compiler's wait counting adds no vmcnt(0) inside the loop.
  const int me = min(tid, 4 * BR - 1);  // mask word staged by this thread
  uint64_t mword;
  {
    const int rc = min(row_of(me % BR), R - 1);
    mword = a.mask[((int64_t)b * a.T + rc / a.G) * a.W + min(me / BR, a.W - 1)];
  }
  bf16x8_t qf[WR][KSTEPS];
#pragma unroll
  for (int w = 0; w < WR; ++w) {
    const int rc = min(row_of(rg * 16 * WR + w * 16 + r16), R - 1);
    const int slot = rc / a.G, gg = rc - slot * a.G;
    const uint16_t* qr = (const uint16_t*)a.q +
                         (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[w][kk] = *(const bf16x8_t*)(qr + kk * 32 + g * 8);
  }

  f32x4_t oacc[WR][DT];
#pragma unroll
  for (int w = 0; w < WR; ++w)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[w][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Row sums l ride on the matrix cores as well: ones . P^T adds the bf16
  // weights exactly as V^T . P^T uses them, replicated over the 16 d rows.
  // Per row: the running max m (scaled, log2 units), the exponent offset
  // -m (0 while m = -inf) and the raw tile max above which m is raised,
  // (m + kSlack) / c, all updated only when m is.
  f32x4_t lacc[WR];
  float m_run[WR], nmu[WR], raise_at[WR];
#pragma unroll
  for (int w = 0; w < WR; ++w) {
    lacc[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[w] = -INFINITY;
    nmu[w] = 0.f;
    raise_at[w] = -INFINITY;
  }
  bf16x8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const float c = a.scale_log2;

  const int64_t kvb = (int64_t)b * a.Hkv + kvh;
  const uint16_t* kcb = (const uint16_t*)a.kc + kvb * a.Pcap * HD;
  const uint16_t* vcb = (const uint16_t*)a.vc + kvb * a.Pcap * HD;
  const uint16_t* ktb = (const uint16_t*)a.kt + kvb * a.T * HD;
  const uint16_t* vtb = (const uint16_t*)a.vt + kvb * a.T * HD;

  // Tiles go straight from global memory to LDS (global_load_lds_dwordx4:
  // lane i of a wave writes bytes 16i..16i+15 of a 1 KB slab).  In LDS a
  // tile is row-major [key][d] with the 16-byte chunk c of row r stored at
  // chunk position c ^ (r % CPR): the direct loads cannot pad rows, and the
  // XOR swizzle keeps the K reads and V transpose reads free of bank
  // conflicts.  Keys past the end of the prefix, or past the last kept tree
  // slot, load the last valid row instead: finite values whose scores are
  // masked, so they add p = 0 times a finite V (tree rows past n_kept are
  // the caller's unwritten memory and are never read).
// A tile whose 64 rows all exist, from its first K and V rows.
#define ET_ISSUE_WHOLE(KT_, VT_, BUF_)                                        \
  do {                                                                        \
    const char* Kt_ = (const char*)(KT_);                                     \
    const char* Vt_ = (const char*)(VT_);                                     \
    _Pragma("unroll") for (int c_ = 0; c_ < CH; ++c_) {                       \
      const int slab = c_ * 8 + wave_u;                                       \
      const uint32_t bo_ = c_ * (512 / CPR) * HD * 2;                         \
      load_lds16(Kt_ + bo_ + tboff, &sKV[0][(BUF_)][slab * 512]);             \
      load_lds16(Vt_ + bo_ + tboff, &sKV[1][(BUF_)][slab * 512]);             \
    }                                                                         \
  } while (0)
#define ET_ISSUE_TILE(T_, BUF_)                                               \
  do {                                                                        \
    const int t_ = (T_);                                                      \
    const bool tr_ = t_ >= tp;                                                \
    const int k0_ = (tr_ ? t_ - tp : t_) * kAttnTile;                         \
    const int klast_ = (tr_ ? n + 1 : P) - 1;                                 \
    const uint16_t* Kg_ = tr_ ? ktb : kcb;                                    \
    const uint16_t* Vg_ = tr_ ? vtb : vcb;                                    \
    if (k0_ + kAttnTile <= klast_ + 1) {                                      \
      ET_ISSUE_WHOLE(Kg_ + (int64_t)k0_ * HD, Vg_ + (int64_t)k0_ * HD, (BUF_));  \
    } else {                                                                  \
      _Pragma("unroll") for (int c_ = 0; c_ < CH; ++c_) {                     \
        const int slab = c_ * 8 + wave_u;                                     \
        const int64_t go = (int64_t)min(k0_ + trow + c_ * (512 / CPR), klast_) * HD + tcol; \
        load_lds16(Kg_ + go, &sKV[0][(BUF_)][slab * 512]);                    \
        load_lds16(Vg_ + go, &sKV[1][(BUF_)][slab * 512]);                    \
      }                                                                       \
    }                                                                         \
  } while (0)

  // Per lane, the tile row it loads in its first slab and the swizzled
  // column, computed once (the wave index made uniform, so each slab's LDS
  // address is scalar arithmetic).  Slab c_ lies 512 / CPR rows further on,
  // with the same column (a multiple of CPR rows leaves the swizzle as is).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int trow = (wave_u * 64 + lane) / CPR;
  const int tcol = (((wave_u * 64 + lane) % CPR) ^ (trow & (CPR - 1))) * 8;
  const uint32_t tboff = (uint32_t)(trow * HD + tcol) * 2u;  // bytes, in a tile whose rows all exist
  static_assert((512 / CPR) % CPR == 0, "slabs keep the swizzle");
  if (cnt > 0) ET_ISSUE_TILE(t_begin, 0);
  if (PD > 1 && cnt > 1) ET_ISSUE_TILE(t_begin + 1, 1);
  // Q, the mask word and tile 0 have landed; tile 1 may still be in flight
  if (PD > 1 && cnt > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CH));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (tid < 4 * BR) {
    const int rr = me % BR, q = me / BR;
    sMask[q][rr] = (row_of(rr) < R && q < a.W) ? mword : 0ull;
  }
  __syncthreads();

  const int sw = r16 & (CPR - 1);  // swizzle of the K rows this lane reads
  // A row group whose rows all lie past the kept slots' rows (when the
  // unit's row count is not a multiple of the blocks') only helps stage the
  // tiles: its accumulators stay zero, which writes the zero output (or
  // empty partial) such rows get.
  const bool active = row_of(rg * 16 * WR) < R;  // wave-uniform
  // Per-lane LDS addresses of the K fragments and V transpose reads in
  // buffer 0; buffer `cur` adds cur * TE * 2 bytes (K) as an immediate
  // offset, and the V tiles lie NB * TE * 2 bytes further on.
  uint32_t ka0[KSTEPS], va0[DT];
  {
    const uint32_t kb = lds_addr(&sKV[0][0][0]) + (kh * 32 + r16) * (HD * 2);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) ka0[kk] = kb + (((kk * 4 + g) ^ sw) * 16);
    const int vrow = kh * 32 + g * 4 + (r16 >> 2);
    const uint32_t vbase = lds_addr(&sKV[1][0][vrow * HD]) + (r16 & 1) * 8;
    const int vsw = vrow & (CPR - 1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) va0[dt] = vbase + (((dt * 2 + ((r16 >> 1) & 1)) ^ vsw) * 16);
  }
  // One tile step on buffer CUR (a compile-time index: the loop below runs
  // NB steps per trip, so every LDS address is a fixed register plus an
  // immediate and no address is recomputed per tile).
  // FAST: the step's tile and the tile it issues are whole prefix tiles
  // (no clamped rows, no mask), which the caller has checked.
  auto tile_step = [&](auto CUR_, auto FAST_, const int it) {
    constexpr int cur = decltype(CUR_)::value;
    constexpr bool fast = decltype(FAST_)::value;
    constexpr int kofs = cur * TE * 2;  // byte offset of buffer cur
    // buffer (cur+PD) % NB was last read in step it-1, before its barrier
    if constexpr (fast) {
      const int64_t e0 = (int64_t)(t_begin + it + PD) * (kAttnTile * HD);
      ET_ISSUE_WHOLE(kcb + e0, vcb + e0, (cur + PD) % NB);
    } else if (it + PD < cnt) {
      ET_ISSUE_TILE(t_begin + it + PD, (cur + PD) % NB);
    }

    if (active) {
    const int t = t_begin + it;
    const bool tree = !fast && t >= tp;
    const int key0 = (tree ? t - tp : t) * kAttnTile;

    // S^T = K . Q^T over this wave's 32 keys: lane holds row r16 and keys
    // kh*32 + s2*16 + 4g + e.  Every K fragment of the tile is read before
    // one wait, then the matrix instructions run back to back, kk outermost
    // for independent accumulators.
    f32x4_t sacc[WR][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int w = 0; w < WR; ++w) sacc[w][s2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      bf16x8_t af[KSTEPS][2];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        af[kk][0] = ds_read_b128_at<kofs>(ka0[kk]);
        af[kk][1] = ds_read_b128_at<kofs + 16 * HD * 2>(ka0[kk]);  // 16 key rows below
      }
      lds_wait_k(af);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int w = 0; w < WR; ++w)
            sacc[w][s2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][s2], qf[w][kk], sacc[w][s2], 0, 0, 0);
    }

    // V^T by transpose reads, issued from inline assembly: the compiler
    // cannot tell them apart from the direct loads still filling another
    // buffer, and would otherwise wait for those loads (vmcnt(0)) before
    // each read.  The wait for them (lgkmcnt(0)) ties their registers, so
    // no use can be scheduled before it.  With three buffers (128-row
    // blocks, registers to spare) they are issued before the softmax, whose
    // vector work then hides their latency; 64-row blocks issue them after
    // it, keeping four waves per SIMD within the register budget.
    u32x2_t vlo[DT], vhi[DT];
    auto issue_v = [&]() {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // this lane's source word: key row vrow (+16), d = dt*16 + 4*(r16%4)
        vlo[dt] = ds_read_tr16_at<kofs>(va0[dt]);
        vhi[dt] = ds_read_tr16_at<kofs + 16 * HD * 2>(va0[dt]);  // 16 key rows below
      }
    };
    if constexpr (NB == 3) issue_v();

    // Softmax in base 2 on unscaled scores: p = 2^(s*c - m).  The running
    // max m is raised only when some row's tile max exceeds it by more
    // than kSlack (a wave-uniform branch), so the O rescale is rare; the
    // weights are then bounded by 2^kSlack, harmless in fp32 and bf16.
    const bool full = fast || (!tree && key0 + kAttnTile <= P);
    bf16x8_t pf[WR];
#pragma unroll
    for (int w = 0; w < WR; ++w) {
      float sv[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[s2][e] = sacc[w][s2][e];
      if (!full) {
        const uint64_t vm =
            (tree ? sMask[key0 >> 6][rg * 16 * WR + w * 16 + r16]
                  : (1ull << (P - key0)) - 1ull) >> (kh * 32 + g * 4);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!((vm >> (s2 * 16 + e)) & 1ull)) sv[s2][e] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sv[s2][e]);
      tmax = max_xor_rows<32>(max_xor_rows<16>(tmax));
      if (__ballot(tmax > raise_at[w]) != 0ull) {
        const float m_new = fmaxf(m_run[w], tmax * c);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[w] - m_new);
        m_run[w] = m_new;
        // a row that has seen no visible key keeps m = -inf and gets p = 0
        nmu[w] = m_new == -INFINITY ? 0.f : -m_new;
        raise_at[w] = (m_new + kSlack) / c;
        lacc[w] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[w][dt] *= alpha;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pf[w][s2 * 4 + e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[s2][e], c, nmu[w]));
    }

    if constexpr (NB != 3) issue_v();
    // O^T += V^T . P^T over the wave's 32 keys.
    lds_wait_all(vlo, vhi);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x8_t af;
      u32x2_t* afh = (u32x2_t*)&af;
      afh[0] = vlo[dt];
      afh[1] = vhi[dt];
#pragma unroll
      for (int w = 0; w < WR; ++w)
        oacc[w][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf[w], oacc[w][dt], 0, 0, 0);
    }
#pragma unroll
    for (int w = 0; w < WR; ++w)
      lacc[w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[w], lacc[w], 0, 0, 0);
    }  // active
    // tile it+1 must have landed before the barrier; tile it+2 may fly on
    if (PD > 1 && (fast || it + 2 < cnt)) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * CH));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    barrier_no_fence();
  };
  using fast_t = std::true_type;
  using gen_t = std::false_type;
  // Steps it < n_fast issue tile t_begin + it + PD below floor(P / 64):
  // it and every tile before it are whole prefix tiles.
  const int n_fast = max(0, min(cnt - PD, P / kAttnTile - t_begin - PD));
  int it = 0;
  for (; it + NB <= n_fast; it += NB) {
    tile_step(std::integral_constant<int, 0>{}, fast_t{}, it);
    tile_step(std::integral_constant<int, 1>{}, fast_t{}, it + 1);
    if constexpr (NB == 3) tile_step(std::integral_constant<int, NB - 1>{}, fast_t{}, it + 2);
  }
  for (; it < cnt; it += NB) {
    tile_step(std::integral_constant<int, 0>{}, gen_t{}, it);
    if (it + 1 < cnt) tile_step(std::integral_constant<int, 1>{}, gen_t{}, it + 1);
    if constexpr (NB == 3)
      if (it + 2 < cnt) tile_step(std::integral_constant<int, NB - 1>{}, gen_t{}, it + 2);
  }

  // Combine the two key halves of every row group: the kh = 1 waves
  // publish (m, l, O) in LDS (the tile buffers are idle now: every direct
  // load has landed and every read has returned), the kh = 0 waves merge.
  float* xo = (float*)&sKV[0][0][0];
  float* xm = xo + 4 * WR * DT * 64 * 4;
  float* xl = xm + 4 * WR * 16;
  static_assert((4 * WR * DT * 64 * 4 + 2 * 4 * WR * 16) * 4 <= NB * 2 * TE * 2,
                "the exchange fits in the tile buffers");
  if (kh == 1) {
#pragma unroll
    for (int w = 0; w < WR; ++w) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *(f32x4_t*)&xo[(((rg * WR + w) * DT + dt) * 64 + lane) * 4] = oacc[w][dt];
      if (g == 0) {
        xm[(rg * WR + w) * 16 + r16] = m_run[w];
        xl[(rg * WR + w) * 16 + r16] = lacc[w][0];
      }
    }
  }
  __syncthreads();
  if (kh == 1) return;

#pragma unroll
  for (int w = 0; w < WR; ++w) {
    const float m1 = xm[(rg * WR + w) * 16 + r16];
    const float l1 = xl[(rg * WR + w) * 16 + r16];
    const float m0 = m_run[w];
    const float m = fmaxf(m0, m1);
    const float f0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - m);
    const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    const float l = lacc[w][0] * f0 + l1 * f1;
    f32x4_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      o[dt] = oacc[w][dt] * f0 +
              *(const f32x4_t*)&xo[(((rg * WR + w) * DT + dt) * 64 + lane) * 4] * f1;
    const int rr = rg * 16 * WR + w * 16 + r16;
    const int r = row_of(rr);
    if (r >= RT) continue;
    if (a.S == 1) {
      const int slot = r / a.G, gg = r - slot * a.G;
      uint16_t* orow = out + (((int64_t)b * a.T + slot) * a.Hq + kvh * a.G + gg) * HD;
      const float inv = (r < R && l > 0.f) ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 wv;
        wv.x = (uint32_t)f32_to_bf16_rne(o[dt][0] * inv) |
               ((uint32_t)f32_to_bf16_rne(o[dt][1] * inv) << 16);
        wv.y = (uint32_t)f32_to_bf16_rne(o[dt][2] * inv) |
               ((uint32_t)f32_to_bf16_rne(o[dt][3] * inv) << 16);
        *(uint2*)(orow + dt * 16 + g * 4) = wv;
      }
    } else {
      const int64_t pr = ((int64_t)(unit * a.nqb + qb) * a.S + split) * BR + rr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(f32x4_t*)(a.po + pr * HD + dt * 16 + g * 4) = o[dt];
      if (g == 0) {
        a.pm[pr] = m;
        a.pl[pr] = l;
      }
    }
  }
}

#undef ET_ISSUE_TILE

// The batch's sequences ranked by descending prefix length (ties by
// index): order[r] is the sequence of rank r.  The attention grid then
// walks the longest sequences first, so that when a launch has more blocks
// than the chip holds at once the last blocks to start are short ones
// (longest-processing-time-first list scheduling).  One block; B is at
// most kAttnOrderMaxB.
__global__ __launch_bounds__(1024) void tree_attn_order_kernel(const int32_t* prefix_len, int B,
                                                          int32_t* order) {
  __shared__ int s_len[kAttnOrderMaxB];
  for (int i = threadIdx.x; i < B; i += blockDim.x) s_len[i] = prefix_len[i];
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += blockDim.x) {
    const int mine = s_len[t];
    int r = 0;
    for (int q = 0; q < B; ++q) {
      const int o = s_len[q];
      r += (o > mine || (o == mine && q < t)) ? 1 : 0;
    }
    order[r] = t;
  }
}

// Combine the S split partials: o = sum_i O_i 2^(m_i - m) / l.  A block
// covers RPB rows of one (unit, row block); thread = (row, 4 columns).
// Blocks map to XCDs like the main kernel.  Every load of a thread is
// independent and issued up front, for MS >= S splits (the smallest of 8,
// 16 and 32 that holds S: a short kernel for the common split counts).
template <int HD, int WR, int MS>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a) {
  static_assert(MS <= kAttnMaxSplits, "split bound");
  constexpr int TPR = HD / 4;     // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  constexpr int BR = 64 * WR;
  constexpr int MB = BR / RPB;    // merge blocks per (unit, row block)
  // The arguments in one round of scalar loads, then the kept count and
  // the split partials in one round of loads: the partials are read
  // whatever the count (rows past it hold unused workspace, replaced by
  // zeros at the end), so no load waits for another.
  // (Pointers pass the asm as integers and come back as global-memory
  // pointers, which keeps their loads global rather than flat.)
  int B = a.B, Hkv = a.Hkv, nqb = a.nqb, S = a.S, T = a.T, G = a.G, Hq = a.Hq;
  uint64_t u_nk = (uint64_t)a.n_kept, u_po = (uint64_t)a.po, u_pm = (uint64_t)a.pm,
           u_pl = (uint64_t)a.pl, u_out = (uint64_t)a.out;
  asm volatile("" : "+s"(B), "+s"(Hkv), "+s"(nqb), "+s"(S), "+s"(T), "+s"(G), "+s"(Hq),
               "+s"(u_nk), "+s"(u_po), "+s"(u_pm), "+s"(u_pl), "+s"(u_out));
  const gmem_i32* n_kept = (const gmem_i32*)u_nk;
  const gmem_f32 *po = (const gmem_f32*)u_po, *pm = (const gmem_f32*)u_pm,
                 *pl = (const gmem_f32*)u_pl;
  int unit, rem;
  if (!attn_block_coords(blockIdx.x, B * Hkv, nqb * MB, &unit, &rem)) return;
  const int qb = rem / MB, mb = rem - qb * MB;
  const int rr = mb * RPB + threadIdx.x / TPR;
  const int col = (threadIdx.x % TPR) * 4;
  const int b = unit / Hkv, kvh = unit - b * Hkv;
  const int r = qb * BR + rr;
  if (r >= T * G) return;
  const int R = (n_kept[b] + 1) * G;
  const int slot = r / G, gg = r - slot * G;
  gmem_u16* orow = (gmem_u16*)u_out + (((int64_t)b * T + slot) * Hq + kvh * G + gg) * HD + col;
  const int64_t base = (int64_t)(unit * nqb + qb) * S;
  float mi[MS], li[MS];
  float4 oi[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    mi[i] = -INFINITY;
    li[i] = 0.f;
    oi[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < S) {
      const int64_t pr = (base + i) * BR + rr;
      mi[i] = pm[pr];
      li[i] = pl[pr];
      const f32x4_t v = *(const gmem_f32x4*)(po + pr * HD + col);
      oi[i] = make_float4(v.x, v.y, v.z, v.w);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < MS; ++i) m = fmaxf(m, mi[i]);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const float f = mi[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi[i] - m);
    l += li[i] * f;
    acc.x += oi[i].x * f;
    acc.y += oi[i].y * f;
    acc.z += oi[i].z * f;
    acc.w += oi[i].w * f;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint2 w;
  w.x = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  w.y = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  if (r >= R) w = make_uint2(0u, 0u);  // rows of unkept slots
  *(gmem_u32x2*)orow = u32x2_t{w.x, w.y};
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

// 64-row blocks fit two per compute unit with two tile buffers (127
// registers, 66 KB of LDS); 128-row blocks need more registers than four
// waves per SIMD allow, so they keep three buffers and one block per CU.
#ifndef ET_ATTN_NB
#define ET_ATTN_NB(WR) ((WR) == 1 ? 2 : 3)
#endif
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
  a.order = nullptr;
  a.rank_inline = 0;
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
  a.interleave = p.attn_wr == 1 && p.attn_splits == 1 && p.attn_nqb > 1;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (p.qdt == ET_F32) {
    tree_attn_f32_kernel<<<dim3(p.T, p.Hq, p.B), 256, 0, s>>>(a, p.HD);
    return hipGetLastError();
  }
  const int units8 = (p.B * p.Hkv + 7) / 8 * 8;  // whole units per XCD
  const int blocks = units8 * p.attn_nqb * p.attn_splits;
  // More blocks than the chip holds at once (two per compute unit with two
  // tile buffers, one with three) and ragged prefixes: dispatch the
  // longest sequences first.  (Only without key splits: the split merge
  // maps units to sequences directly.)
  const int resident = 256 * (ET_ATTN_NB(p.attn_wr) == 2 ? 2 : 1);
  // Up to 64 sequences (lengths below 2^26) each wave ranks the batch
  // itself, one sequence per lane, instead of a launch of its own (over
  // 20-bit keys when the lengths are below 2^14).
  if (p.B > 1 && p.B <= 64 && p.Pcap < (1 << 26) && p.attn_splits == 1 && blocks > resident) {
    a.rank_inline = p.Pcap < (1 << 14) ? 1 : 2;
  } else if (p.B > 1 && p.B <= kAttnOrderMaxB && p.attn_splits == 1 && blocks > resident) {
    const int nt = p.B < 1024 ? (p.B + 63) / 64 * 64 : 1024;
    tree_attn_order_kernel<<<1, nt, 0, s>>>(prefix_len, p.B, w.order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.order = w.order;
  }
#define ET_ATTN(HD, WR)                                                          \
  do {                                                                           \
    tree_attn_bf16_kernel<HD, WR, ET_ATTN_NB(WR)><<<blocks, 512, 0, s>>>(a);     \
    hipError_t e = hipGetLastError();                                            \
    if (e != hipSuccess || p.attn_splits == 1) return e;                         \
    const dim3 mg(units8 * p.attn_nqb * (64 * WR / (256 / (HD / 4))));           \
    if (p.attn_splits <= 8) tree_attn_merge_kernel<HD, WR, 8><<<mg, 256, 0, s>>>(a);        \
    else if (p.attn_splits <= 16) tree_attn_merge_kernel<HD, WR, 16><<<mg, 256, 0, s>>>(a); \
    else tree_attn_merge_kernel<HD, WR, 32><<<mg, 256, 0, s>>>(a);               \
  } while (0)
  if (p.HD == 128) {
    if (p.attn_wr == 2) ET_ATTN(128, 2);
    else ET_ATTN(128, 1);
  } else {
    if (p.attn_wr == 2) ET_ATTN(64, 2);
    else ET_ATTN(64, 1);
  }
#undef ET_ATTN
  return hipGetLastError();
}

}  // namespace et
