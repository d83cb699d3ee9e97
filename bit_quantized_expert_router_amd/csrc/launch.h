// Host-side launchers shared between the C-ABI layer (api.cpp) and the
// kernel translation units.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq2 {

// Kernel ids for the measurement hooks (order = moe_profile_kernel_name).
enum KernelId {
  K_ROUTE_TOPK = 0,
  K_ROUTE_SCAN,
  K_ROUTE_SCATTER,
  K_DECODE_GATEUP,
  K_DECODE_DOWN,
  K_PREFILL_PREP,
  K_PREFILL_GATEUP,
  K_PREFILL_DOWN,
  K_PREFILL_COMBINE,
  K_ROUTE_GEMV_TOPK,
  K_USAGE_UPDATE,
  K_RESIDENCY_MAP,
  K_NUM_KERNELS
};

// Start and stop events of one launch while the measurement hooks are on
// (both null otherwise).  hipExtLaunchKernel stamps them with the begin and
// end of the dispatch itself, so their difference is the kernel's execution
// time without the gap between launches.  Defined in api.cpp.
struct ProfileScope {
  explicit ProfileScope(int kernel_id);
  ~ProfileScope();
  void commit();  // the launch was enqueued: keep the pair for moe_profile_query
  int id;
  hipEvent_t ev0, ev1;
  bool committed;
};

// Every kernel of the library is enqueued through here.
template <typename F, typename... Args>
hipError_t launch_kernel(int kernel_id, F kernel, dim3 grid, dim3 block, uint32_t lds,
                         hipStream_t s, Args... args) {
  ProfileScope prof(kernel_id);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, prof.ev0, prof.ev1, 0u, args...);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) prof.commit();
  return e;
}

// ---------------------------------------------------------------- routing --
constexpr int kRouteMaxChunkTokens = 256;
// Tokens per routing workgroup (chunk): small chunks give more workgroups
// for the top-k, large ones fewer per-chunk counts to scan.
inline __host__ __device__ int route_chunk_tokens(int T) {
  return T <= 4096 ? 16 : (T <= 65536 ? 64 : 256);
}
// With rank, local_counts and the four histogram outputs given, and when
// route_histogram_fused(T, k) holds (one chunk of at most 16 tokens), the
// histogram is finished in this launch: the scan and scatter launches are
// then not needed.
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             int32_t* rank, int32_t* local_counts, hipStream_t s,
                             int32_t* counts = nullptr, int32_t* offsets = nullptr,
                             int32_t* sorted_pairs = nullptr, int32_t* pair_pos = nullptr);
// Whether launch_route_topk finishes the histogram itself for this shape.
bool route_histogram_fused(int T, int k);
// Router GEMV (fp64 accumulation, bf16 weight [E][H]) + top-k for T <= 4
// tokens in one kernel; `counter` is a zeroed word the kernel leaves zeroed.
hipError_t launch_route_gemv_topk(const void* x, int x_bf16, int T, const uint16_t* W, int E, int H,
                                  int k, float* logits, int32_t* ids, float* w, uint32_t* counter,
                                  hipStream_t s);
hipError_t launch_route_expert_scan(const int32_t* local_counts, int32_t* ebase, int E, int n_chunks,
                                    int32_t* counts, hipStream_t s);
hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* ebase,
                                const int32_t* counts, int E, int T, int k, int n_chunks,
                                int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                                hipStream_t s);

// ----------------------------------------------------------------- decode --
struct LayerArgs {
  const uint8_t* experts;   // all E experts, or (with slot_of) the S resident slots
  const uint8_t* shared;
  int64_t stride;
  int E, H, I;
  // residency tier (slot_of == nullptr otherwise): expert e is in slot
  // slot_of[e] of `experts` when that lies in [0, S), else at
  // arena + e * stride
  const int32_t* slot_of = nullptr;
  const uint8_t* arena = nullptr;
  int S = 0;
  // decode: += pairs routed to each expert (nullptr: not counted)
  unsigned long long* usage = nullptr;
};

// With `logits` non-null the routing (ids, w) is taken inside the gate/up
// kernel (ids_out / w_out, if non-null, receive it); otherwise ids and w are
// read.
hipError_t launch_decode(const LayerArgs& L, const void* x, int x_bf16, int T,
                         const int32_t* ids, const float* w, const float* logits,
                         int32_t* ids_out, float* w_out, int k, const void* residual,
                         void* out, int out_bf16, int prenorm, void* ws, hipStream_t s);
size_t decode_workspace_bytes(int T, int k, int H, int I);
// The device address of this GPU's static decode scratch (resolved once per
// device, with that device current) and its size.
hipError_t decode_static_scratch(void** ptr);
size_t decode_static_scratch_bytes();

// ---------------------------------------------------------------- prefill --
constexpr int kGroupRows = 64;          // rows (token-expert pairs) per work item

hipError_t launch_prefill(const LayerArgs& L, const void* x, int x_bf16, int T,
                          const int32_t* ids, const float* w, int k, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pairs,
                          const int32_t* pair_pos, const void* residual, void* out,
                          int out_bf16, int prenorm, void* ws, hipStream_t s);
size_t prefill_workspace_bytes(int T, int E, int k, int H, int I);

// ------------------------------------------------------------ residency --
// counts[e] += entries of ids[0..n) equal to e (others skipped).
hipError_t launch_usage_update(const int32_t* ids, long long n, int E, unsigned long long* counts,
                               hipStream_t s);
// Changes of the device slot map, carried as kernel arguments: entry i sets
// slot_of[rec & 0xFFFF] = (rec >> 16) - 1.
constexpr int kMapRecs = 256;
struct MapRecs {
  uint32_t rec[kMapRecs];
};
hipError_t launch_residency_map(int32_t* slot_of, const MapRecs& recs, int n, hipStream_t s);

}  // namespace moeq2
