// launch_floor.hip -- the fixed cost of a draft step's two launches.
//
// A draft step is a scan launch (one block per 8K-element chunk of each
// frontier row) followed by a one-block-per-sequence merge launch.  This
// program replays, in HIP graphs, kernels with the same grids that do only
// the data movement of that pattern, and prints the time per step:
//   empty     two empty kernels with the scan's and the merge's grids;
//   pair      the scan grid loading 16 KB per block (four 16-byte loads
//             per thread, a wave maximum, one partial per wave stored),
//             then the merge block loading every partial and storing one
//             value: the floor under the two-launch design;
//   ticket    one launch: the scan grid publishing its partials with
//             agent-scope atomic stores, then an agent-scope arrival
//             counter; the last block to arrive loads every partial (the
//             single-launch alternative to the second launch).
// Buffers rotate over about 670 MB (at 160 blocks), so every step reads
// HBM, not the 256 MB MALL.
// Usage: launch_floor [scan_blocks [merge_threads]]   (defaults: 160, 640,
// the batch-1 Llama-3.1-8B draft step: 16 chunks x 10 rows, 10 waves).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CK(x)                                                               \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;                // scan block
constexpr int kVec = 4;                      // 16-byte loads per thread
constexpr int kBlockVecs = kThreads * kVec;  // 16 KB per block
constexpr int kSteps = 64;                   // steps per graph
constexpr int kGraphs = 4;                   // graphs, each on its own buffers

__global__ void empty_kernel() {}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
  return v;
}

__device__ __forceinline__ uint32_t block_chunk_max(const u32x4* src) {
  u32x4 r[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) r[i] = src[i * kThreads + threadIdx.x];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kVec; ++i) m = max(m, max(max(r[i][0], r[i][1]), max(r[i][2], r[i][3])));
  return wave_max(m);
}

// scan grid: block i reads chunk i of `buf` and stores its waves' maxima
__global__ __launch_bounds__(kThreads) void scan_kernel(const u32x4* buf, uint32_t* part) {
  const uint32_t m = block_chunk_max(buf + (size_t)blockIdx.x * kBlockVecs);
  if ((threadIdx.x & 63) == 0) part[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = m;
}

// merge: one block reads every partial and stores their maximum
__global__ __launch_bounds__(1024) void merge_kernel(const uint32_t* part, int n, uint32_t* out) {
  __shared__ uint32_t s_w[16];
  uint32_t v = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) v = max(v, part[i]);
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < (int)blockDim.x / 64; ++w) x = max(x, s_w[w]);
    out[0] = x;
  }
}

// one launch: partials by agent-scope atomic stores, an arrival counter,
// and the last block merges (it also resets the counter for the next step)
__global__ __launch_bounds__(kThreads) void ticket_kernel(const u32x4* buf, uint32_t* part,
                                                          int* ctr, uint32_t* out) {
  __shared__ int s_last;
  __shared__ uint32_t s_w[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t m = block_chunk_max(buf + (size_t)blockIdx.x * kBlockVecs);
  if (lane == 0)
    __hip_atomic_store(&part[blockIdx.x * (kThreads / 64) + wave], m, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();  // every wave's partial stored (and acknowledged)
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  const int n = gridDim.x * (kThreads / 64);
  uint32_t v = 0;
  for (int i = tid; i < n; i += kThreads)
    v = max(v, __hip_atomic_load(&part[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  v = wave_max(v);
  if (lane == 0) s_w[wave] = v;
  __syncthreads();
  if (tid == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kThreads / 64; ++w) x = max(x, s_w[w]);
    out[0] = x;
    __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int main(int argc, char** argv) {
  const int blocks = argc > 1 ? atoi(argv[1]) : 160;
  const int mthreads = argc > 2 ? atoi(argv[2]) : 640;
  if (blocks < 1 || blocks > 4096 || mthreads < 64 || mthreads > 1024 || mthreads % 64) {
    fprintf(stderr, "usage: launch_floor [scan_blocks 1..4096 [merge_threads 64..1024, x64]]\n");
    return 2;
  }
  // each step reads its own blocks * 16 KB; the buffers of all steps of
  // all graphs: kGraphs * kSteps * blocks * 16 KB (671 MB at 160 blocks)
  const size_t step_vecs = (size_t)blocks * kBlockVecs;
  const size_t nvec = step_vecs * kSteps * kGraphs;
  const int nparts = blocks * (kThreads / 64);
  u32x4* buf;
  uint32_t *part, *out;
  int* ctr;
  CK(hipMalloc(&buf, nvec * sizeof(u32x4)));
  CK(hipMalloc(&part, (size_t)nparts * 4));
  CK(hipMalloc(&out, 4));
  CK(hipMalloc(&ctr, 4));
  CK(hipMemset(buf, 1, nvec * sizeof(u32x4)));
  CK(hipMemset(part, 0, (size_t)nparts * 4));
  CK(hipMemset(ctr, 0, 4));
  CK(hipDeviceSynchronize());
  hipStream_t s;
  CK(hipStreamCreate(&s));

  auto time_mode = [&](int mode) {
    std::vector<hipGraphExec_t> ex(kGraphs);
    for (int g = 0; g < kGraphs; ++g) {
      hipGraph_t gr;
      CK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
      for (int st = 0; st < kSteps; ++st) {
        const u32x4* src = buf + ((size_t)g * kSteps + st) * step_vecs;
        if (mode == 0) {
          empty_kernel<<<blocks, kThreads, 0, s>>>();
          empty_kernel<<<1, mthreads, 0, s>>>();
        } else if (mode == 1) {
          scan_kernel<<<blocks, kThreads, 0, s>>>(src, part);
          merge_kernel<<<1, mthreads, 0, s>>>(part, nparts, out);
        } else {
          ticket_kernel<<<blocks, kThreads, 0, s>>>(src, part, ctr, out);
        }
      }
      CK(hipStreamEndCapture(s, &gr));
      CK(hipGraphInstantiate(&ex[g], gr, nullptr, nullptr, 0));
      CK(hipGraphDestroy(gr));
    }
    for (int g = 0; g < kGraphs; ++g) CK(hipGraphLaunch(ex[g], s));  // warm-up
    CK(hipStreamSynchronize(s));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    constexpr int kReps = 5;
    CK(hipEventRecord(e0, s));
    for (int r = 0; r < kReps; ++r)
      for (int g = 0; g < kGraphs; ++g) CK(hipGraphLaunch(ex[g], s));
    CK(hipEventRecord(e1, s));
    CK(hipEventSynchronize(e1));
    float ms;
    CK(hipEventElapsedTime(&ms, e0, e1));
    for (auto& e : ex) CK(hipGraphExecDestroy(e));
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
    return ms * 1e3 / (kReps * kGraphs * kSteps);
  };
  const double t_empty = time_mode(0), t_pair = time_mode(1), t_ticket = time_mode(2);
  printf("{\"scan_blocks\": %d, \"merge_threads\": %d, \"bytes_per_step\": %zu, "
         "\"us_per_step\": {\"empty\": %.3f, \"pair\": %.3f, \"ticket\": %.3f}}\n",
         blocks, mthreads, step_vecs * sizeof(u32x4), t_empty, t_pair, t_ticket);
  CK(hipFree(buf));
  CK(hipFree(part));
  CK(hipFree(out));
  CK(hipFree(ctr));
  return 0;
}
