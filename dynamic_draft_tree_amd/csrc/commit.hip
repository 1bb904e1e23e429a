// commit.hip -- append the verified path's K/V to the prefix cache.
//
// EAGLE-2 summary page, s2.1: the accepted draft tokens extend the
// sequence in path order; s4.2: the one verify pass computed K/V for every
// tree slot.  The root (slot 0, the first token not yet cached) and the
// accepted slots follow the cached prefix, in path order.
#include "device.h"
#include "internal.h"

namespace et {

typedef uint32_t cu32x4_t __attribute__((ext_vector_type(4)));

// One block per sequence, so that every thread reads prefix_len[b] before
// it is advanced; (path row, kv head, 16-byte chunk) triples are spread
// over the threads.  Rows are copied bit for bit.  Slots and the prefix
// length are clamped into range, so a bad argument cannot address memory
// outside the buffers.
__global__ __launch_bounds__(256) void kv_commit_kernel(char* kc, char* vc, const char* kt,
                                                        const char* vt, int32_t* prefix_len,
                                                        const int32_t* path_slots,
                                                        const int32_t* accept_len, int T,
                                                        int Hkv, int Pcap, int D,
                                                        int row_bytes) {
  const int b = blockIdx.x;
  const int P = min(max(prefix_len[b], 0), Pcap);
  const int L = min(max(accept_len[b], 0), D);
  const int rows = min(L + 1, Pcap - P);
  const int cpr = row_bytes / 16;  // 16-byte chunks per row
  const int total = rows * Hkv * cpr;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int ch = e % cpr, hr = e / cpr;
    const int h = hr % Hkv, i = hr / Hkv;
    const int slot = min(max(path_slots[(int64_t)b * (D + 1) + i], 0), T - 1);
    const int64_t src = (((int64_t)b * Hkv + h) * T + slot) * row_bytes + ch * 16;
    const int64_t dst = (((int64_t)b * Hkv + h) * Pcap + P + i) * row_bytes + ch * 16;
    *(cu32x4_t*)(kc + dst) = *(const cu32x4_t*)(kt + src);
    *(cu32x4_t*)(vc + dst) = *(const cu32x4_t*)(vt + src);
  }
  __syncthreads();
  if (threadIdx.x == 0) prefix_len[b] = P + rows;
}

hipError_t launch_kv_commit(const Plan& p, void* k_cache, void* v_cache,
                            const void* k_tree, const void* v_tree,
                            int32_t* prefix_len, const int32_t* path_slots,
                            const int32_t* accept_len, hipStream_t s) {
  const int esz = p.qdt == ET_BF16 ? 2 : 4;
  kv_commit_kernel<<<p.B, 256, 0, s>>>((char*)k_cache, (char*)v_cache, (const char*)k_tree,
                                       (const char*)v_tree, prefix_len, path_slots,
                                       accept_len, p.T, p.Hkv, p.Pcap, p.D, p.HD * esz);
  return hipGetLastError();
}

}  // namespace et
