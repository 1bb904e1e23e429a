// internal.h -- plan, workspace layout and kernel launchers of libeagletree.
//
// Workspace (device, caller-allocated, 256-byte aligned regions):
//   pool         SoA   token/parent/depth i32, conf/value f32  [B][cap]
//   pool_count, root_token                                     [B]
//   frontier     i32   [2][B][k] pool indices (and f32 values), double-
//                      buffered by step parity so a launch never reads
//                      what it writes
//   frontier_count i32 [2][B]
//   draft partials     per (row, chunk, wave): max, sum, top-k logit keys
//   draft rows         per row: max, fp64 sum, top-k logit keys
//   LM-head lists      per (row, 512-id vocab block): max, sum, top-k keys
//   accept partials    per (slot row, chunk, wave): argmax key (greedy) or
//                      (max, mass) of the wave's id range (sampled)
//   attention partials per (b, kv head, q block, split): O, m, l
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/eagletree.h"

namespace et {

constexpr int kMaxTopk = 16;
constexpr int kMaxDepth = 15;
constexpr int kMaxBudget = 255;
constexpr int kMaxVocab = 1 << 18;       // token id fits the 18-bit key field
constexpr int kMaxPool = 4095;           // pool index fits the 12-bit field
constexpr int kScanThreads = 256;        // threads per row-scan block
constexpr int kElemsBf16 = 32;           // bf16 elements per thread (4 x 16 B)
constexpr int kElemsF32 = 16;            // fp32 elements per thread (4 x 16 B)
// accept scan: 16K bf16 (8K fp32) elements per chunk, eight 16-byte loads
// in flight per thread
constexpr int kAccElemsBf16 = 64;
constexpr int kAccElemsF32 = 32;
constexpr int accept_chunk_elems(int dtype) {
  return kScanThreads * (dtype == ET_BF16 ? kAccElemsBf16 : kAccElemsF32);
}
// vocab elements per row-scan block for a logits dtype; wide chunks hold
// twice as many (eight 16-byte loads per thread)
constexpr int chunk_elems(int dtype, bool wide) {
  return kScanThreads * (dtype == ET_BF16 ? kElemsBf16 : kElemsF32) * (wide ? 2 : 1);
}
// Scan grids (draft and accept) above this many one-chunk blocks give
// each block several chunks of its row (the chip holds a few thousand
// blocks at once).
#ifndef ET_SCAN_TARGET_BLOCKS
#define ET_SCAN_TARGET_BLOCKS 6000
#endif
constexpr int kScanTargetBlocks = ET_SCAN_TARGET_BLOCKS;
// Draft scan grids above this many (narrow) blocks use wide chunks: a
// thread's fixed work per chunk (wave bound, candidate list, partial
// record) is then paid once per twice the elements, where the many waves
// per SIMD make the scan bound by instruction issue.
#ifndef ET_SCAN_WIDE_BLOCKS
#define ET_SCAN_WIDE_BLOCKS 2048
#endif
constexpr int kScanWideBlocks = ET_SCAN_WIDE_BLOCKS;
constexpr int kAttnTile = 64;            // keys per staged K/V tile
constexpr int kAttnMaxSplits = 32;       // key splits per (kv head, row block)
// Batches up to this size may have their attention blocks dispatched
// longest sequence first (one block ranks the prefix lengths).
constexpr int kAttnOrderMaxB = 1024;
#ifndef ET_ATTN_TARGET_BLOCKS
#define ET_ATTN_TARGET_BLOCKS 256
#endif
constexpr int kAttnTargetBlocks = ET_ATTN_TARGET_BLOCKS;  // blocks the split count aims for

struct DraftWs {
  int32_t* pool_token;    // [B][cap]
  int32_t* pool_parent;
  int32_t* pool_depth;
  float* pool_conf;
  float* pool_value;
  int32_t* pool_count;    // [B]
  int32_t* root_token;    // [B]
  int32_t* frontier;      // [2][B][k]
  float* frontier_val;    // [2][B][k] value of each frontier node
  int32_t* frontier_count;// [2][B]
  float* part_m;          // [B][k][lists] (lists = S, or S * waves)
  float* part_s;          // [B][k][lists]
  uint64_t* part_keys;    // [B][k][kMaxTopk][lists]: rank r of every list, contiguous
};

// Draft step from hidden states: level-1 lists, one per (row, kLmCols-id
// vocab block): max, sum of exp, top-k keys.
struct LmWs {
  float* m;               // [B][k][L1]
  float* s;               // [B][k][L1]
  uint64_t* keys;         // [B][k][L1][kMaxTopk]
};
#ifndef ET_LM_WAVES
#define ET_LM_WAVES 8
#endif
constexpr int kLmCols = ET_LM_WAVES * 64;  // vocab ids per LM-head block
constexpr int lm_lists1(int V) { return (V + kLmCols - 1) / kLmCols; }
constexpr int lm_lists2(int V) { return (lm_lists1(V) + 7) / 8; }

struct AcceptWs {
  uint64_t* part;         // [B][T][S][waves] (max logit, lowest id) keys, or
                          // double2 (max, mass) per id range when sampling
};

struct AttnWs {
  float* o;               // [B*Hkv][nqb][S][rows per block][d]
  float* m;               // [B*Hkv][nqb][S][rows per block]
  float* l;
  int32_t* order;         // [B] sequences by descending prefix length
};

struct Plan {
  et_config cfg;
  int B, V, k, D, N, T, W, cap;
  int Hq, Hkv, G, HD, Pcap;
  int ldt, qdt;           // et_dtype of logits and q/k/v
  int s_draft;            // vocab chunks per row
  int draft_cpb;          // chunks streamed by one draft scan block
  int draft_wide;         // draft scan chunks of twice the elements per thread
  int s_accept;           // target-row chunks per row
  int accept_cpb;         // chunks streamed by one accept scan block
  int attn_wr;            // 16-row groups per wave (rows per block 64*wr)
  int attn_nqb, attn_splits;
  // workspace layout
  size_t off[32];
  size_t ws_bytes;
  bool debug;             // ET_DEBUG set at plan creation: sync and check
  // call-order check
  const void* last_ws;
  int last_step;
  bool last_fixed;        // the steps so far followed the fixed shape
  // fixed tree shape (et_set_static_shape); static_m < 0: none
  int static_m;
  int static_nf[kMaxDepth + 2];                  // frontier rows at step l
  int32_t static_next[kMaxDepth + 1][kMaxTopk];  // step l: child j * k + r of each next-frontier node
  int32_t static_slot[kMaxBudget + 1];           // slot s >= 1: pool index | parent slot << 16
};

// The next frontier of one step under a fixed shape: node i is child ci[i]
// (j * k + r: rank r of the step's row j), for i < n.
struct FixedFrontier {
  int n;
  int32_t ci[kMaxTopk];
};
// A fixed tree's slots: slot s >= 1 is pool node slot[s] & 0xFFFF with
// parent slot slot[s] >> 16, for s <= m.
struct FixedSlots {
  int m;
  int32_t slot[kMaxBudget + 1];
};

DraftWs draft_ws(const Plan& p, void* ws);
LmWs lm_ws(const Plan& p, void* ws);
AcceptWs accept_ws(const Plan& p, void* ws);
AttnWs attn_ws(const Plan& p, void* ws);

// Launchers (return hipError_t of the launch).
// Where a rerank writes: the et_rerank outputs, and with the flatten the
// et_tree_mask outputs too.
struct RerankOut {
  int32_t* tokens;
  int32_t* parent_slot;
  float* conf;
  float* value;
  int32_t* n_kept;
  const int32_t* prefix_len;
  uint64_t* mask;
  int32_t* depth;
  int32_t* pos;
  int N, T, W;
};

// last: the step is the last one and its merge also reranks and flattens
// the tree into these outputs (et_draft_step_last); else null.
hipError_t launch_draft_step(const Plan& p, const DraftWs& w, int step,
                             const int32_t* root_tokens, const void* logits,
                             int64_t bstride, int64_t rstride, bool vec,
                             const FixedFrontier* fixed, int32_t* next_tokens,
                             int32_t* next_count, hipStream_t s,
                             const RerankOut* last = nullptr);
// The draft step's merge alone, over `parts` partial lists per row already
// in the workspace (fp32 logit keys).
hipError_t launch_draft_merge(const Plan& p, const DraftWs& w, int step,
                              const int32_t* root_tokens, int parts,
                              int32_t* next_tokens, int32_t* next_count, hipStream_t s);
hipError_t launch_draft_step_hidden(const Plan& p, const DraftWs& w, const LmWs& lm, int step,
                                    const int32_t* root_tokens, const void* hidden,
                                    int64_t hb, int64_t hr, const void* lm_head, int H,
                                    int32_t* next_tokens, int32_t* next_count,
                                    hipStream_t s);
hipError_t launch_rerank(const Plan& p, const DraftWs& w, int32_t* tokens,
                         int32_t* parent_slot, float* conf, float* value,
                         int32_t* n_kept, hipStream_t s);
hipError_t launch_rerank_mask(const Plan& p, const DraftWs& w, int32_t* tokens,
                              int32_t* parent_slot, float* conf, float* value,
                              int32_t* n_kept, const int32_t* prefix_len,
                              uint64_t* mask, int32_t* depth, int32_t* pos,
                              hipStream_t s);
hipError_t launch_static_tree(const Plan& p, const DraftWs& w, const FixedSlots& fs,
                              int32_t* tokens, int32_t* parent_slot, float* conf,
                              float* value, int32_t* n_kept, hipStream_t s);
hipError_t launch_tree_mask(const Plan& p, const int32_t* parent_slot,
                            const int32_t* n_kept, const int32_t* prefix_len,
                            uint64_t* mask, int32_t* depth, int32_t* pos,
                            hipStream_t s);
hipError_t launch_tree_attention(const Plan& p, const AttnWs& w,
                                 const void* q, const void* kc,
                                 const void* vc, const void* kt,
                                 const void* vt, const int32_t* prefix_len,
                                 const uint64_t* mask, const int32_t* n_kept,
                                 float scale, void* out, hipStream_t s);
hipError_t launch_accept(const Plan& p, const AcceptWs& w, const void* target,
                         int64_t bstride, int64_t rstride, bool vec,
                         const int32_t* tokens, const int32_t* parent_slot,
                         const int32_t* n_kept, int32_t* accept_len,
                         int32_t* path_slots, int32_t* out_tokens,
                         hipStream_t s);
hipError_t launch_accept_sample(const Plan& p, const AcceptWs& w, const void* target,
                                int64_t bstride, int64_t rstride, bool vec,
                                const int32_t* tokens, const int32_t* parent_slot,
                                const int32_t* n_kept, double c, const float* uniforms,
                                int32_t* accept_len, int32_t* path_slots,
                                int32_t* out_tokens, hipStream_t s);
hipError_t launch_kv_commit(const Plan& p, void* k_cache, void* v_cache,
                            const void* k_tree, const void* v_tree,
                            int32_t* prefix_len, const int32_t* path_slots,
                            const int32_t* accept_len, hipStream_t s);
hipError_t launch_pool_export(const Plan& p, const DraftWs& w, int32_t* token,
                              int32_t* parent, int32_t* depth, float* conf,
                              float* value, int32_t* pool_count,
                              int32_t* frontier, int32_t* frontier_count,
                              hipStream_t s);

}  // namespace et
