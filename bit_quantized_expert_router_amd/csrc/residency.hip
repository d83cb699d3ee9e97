// Residency tier kernels: the usage histogram that decides which experts
// stay in device memory, and the update of the device slot map when the
// resident set changes ("RTX PRO 4500 单卡跑 125B MoE", lcz.me/topic/2169,
// section 最重要机制, item 2: the resident experts are swapped every few
// rounds for the ones the conversation has used most).
//
// The histogram adds integers with atomics, so the counts do not depend on
// the order in which blocks run.  Each block first counts its share of the
// ids in LDS and then adds its non-zero bins to the global counts, so the
// global atomics number at most E per block.
#include "launch.h"
#include "../../include/moe_q2.h"

namespace moeq2 {

namespace {

constexpr int kUsageThreads = 256;
constexpr int kUsageIdsPerBlock = 8192;

__global__ __launch_bounds__(kUsageThreads) void usage_update_kernel(const int32_t* __restrict__ ids,
                                                                     long long n, int E,
                                                                     unsigned long long* __restrict__ counts) {
  __shared__ uint32_t h[MOE_MAX_EXPERTS];
  for (int i = threadIdx.x; i < E; i += kUsageThreads) h[i] = 0u;
  __syncthreads();
  const long long step = static_cast<long long>(gridDim.x) * kUsageThreads;
  for (long long i = static_cast<long long>(blockIdx.x) * kUsageThreads + threadIdx.x; i < n; i += step) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kUsageThreads)
    if (h[i] != 0u) atomicAdd(&counts[i], static_cast<unsigned long long>(h[i]));
}

// One record per thread; the records of one launch name distinct experts.
__global__ __launch_bounds__(kMapRecs) void residency_map_kernel(int32_t* __restrict__ slot_of, MapRecs recs,
                                                                 int n) {
  const int i = threadIdx.x;
  if (i < n) {
    const uint32_t r = recs.rec[i];
    slot_of[r & 0xFFFFu] = static_cast<int32_t>(r >> 16) - 1;
  }
}

}  // namespace

hipError_t launch_usage_update(const int32_t* ids, long long n, int E, unsigned long long* counts,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long want = (n + kUsageIdsPerBlock - 1) / kUsageIdsPerBlock;
  const int blocks = static_cast<int>(want < 1024 ? want : 1024);
  return launch_kernel(K_USAGE_UPDATE, usage_update_kernel, dim3(blocks), dim3(kUsageThreads), 0, s, ids, n,
                       E, counts);
}

hipError_t launch_residency_map(int32_t* slot_of, const MapRecs& recs, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return launch_kernel(K_RESIDENCY_MAP, residency_map_kernel, dim3(1), dim3(kMapRecs), 0, s, slot_of, recs, n);
}

}  // namespace moeq2
