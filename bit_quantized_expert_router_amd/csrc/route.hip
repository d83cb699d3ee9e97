// Router top-k + renormalised softmax weights, and the token->expert
// histogram with a stable (expert, pair-id) permutation.
//
// The router picks, per token, the experts whose ids the GPU hands to the
// expert compute ("RTX PRO 4500 单卡跑 125B MoE", lcz.me/topic/2169, section
// 最重要机制, item 1): 10 of 512 in the target model ("Strata 实测 ...",
// kefong.net, section 二, model table).  Prompt chunks are processed grouped
// by expert (strata-mlx README, section 它是什么), which needs the histogram and
// the permutation.
//
// Determinism: selection compares 64-bit keys (order-preserving float bits,
// then the inverted expert id), so equal logits go to the lower id and the
// result does not depend on reduction order.  The permutation is a counting
// sort: each 64-token chunk ranks its pairs in pair order inside one wave
// (so ranks are stable), a single-workgroup scan turns the per-chunk counts
// (laid out expert-major) into the base position of every (expert, chunk),
// and a scatter writes sorted_pairs / pair_pos.  Only integer arithmetic.
#include "launch.h"
#include "q2_device.h"
#include "../../include/moe_q2.h"

namespace moeq2 {

namespace {

constexpr int kSlotsPerLane = MOE_MAX_EXPERTS / kWave;   // 16

// Larger float -> larger key.  Adding +0.0f first maps -0.0 to +0.0, so the
// two zeros compare equal as they do in float32.
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ rank, int32_t* __restrict__ local_counts,
    int n_chunks) {
  __shared__ int32_t s_ids[kRouteChunkTokens * MOE_MAX_TOPK];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int chunk = blockIdx.x;
  const int t0 = chunk * kRouteChunkTokens;
  const int nt = min(kRouteChunkTokens, T - t0);
  const int nper = (E + kWave - 1) / kWave;

  if (rank) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  }

  for (int ti = wid; ti < nt; ti += blockDim.x / kWave) {
    const int t = t0 + ti;
    const float* row = logits + static_cast<size_t>(t) * E;
    uint64_t key[kSlotsPerLane];
#pragma unroll
    for (int s = 0; s < kSlotsPerLane; ++s) {
      const int e = lane + kWave * s;
      key[s] = 0;
      if (s < nper && e < E)
        key[s] = (static_cast<uint64_t>(float_key(row[e])) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
    }
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int s = 0; s < kSlotsPerLane; ++s) best = key[s] > best ? key[s] : best;
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const uint64_t other = shfl_xor_u64(best, o);
        best = other > best ? other : best;
      }
#pragma unroll
      for (int s = 0; s < kSlotsPerLane; ++s)
        if (key[s] == best) key[s] = 0;
      if (lane == j) my_e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    }
    // weights: softmax over the selected logits (slot 0 holds the maximum)
    const float l = (lane < k) ? row[my_e] : 0.0f;
    const float lmax = __shfl(l, 0, kWave);
    const float z = (lane < k) ? expf(l - lmax) : 0.0f;
    const float sum = wave_sum(z);
    if (lane < k) {
      ids[static_cast<size_t>(t) * k + lane] = my_e;
      w[static_cast<size_t>(t) * k + lane] = z / sum;
      s_ids[ti * k + lane] = my_e;
    }
  }
  if (!rank) return;
  __syncthreads();

  // Stable within-chunk rank of every pair (pair order = t*k + j), one wave.
  if (wid == 0) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const int np = nt * k;
    for (int p0 = 0; p0 < np; p0 += kWave) {
      const int p = p0 + lane;
      const bool active = p < np;
      const int e = active ? s_ids[p] : 0;
      uint64_t same = __ballot(active);
      for (int b = 0; b < nbits; ++b) {
        const int bit = (e >> b) & 1;
        const uint64_t bb = __ballot(active && bit);
        same &= bit ? bb : ~bb;
      }
      const int before = __popcll(same & ((1ull << lane) - 1ull));
      const int cnt = __popcll(same);
      const int base = active ? s_cnt[e] : 0;
      __builtin_amdgcn_wave_barrier();
      if (active) rank[static_cast<size_t>(t0) * k + p] = base + before;
      if (active && before == 0) s_cnt[e] = base + cnt;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    local_counts[static_cast<size_t>(e) * n_chunks + chunk] = s_cnt[e];
}

// One workgroup: exclusive scan of the expert-major [E][C] chunk counts.
__global__ __launch_bounds__(1024) void route_scan_kernel(
    const int32_t* __restrict__ local_counts, int32_t* __restrict__ base, int E, int C,
    int total, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t s_part[1024];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x;
  const int n = E * C;
  const int per = (n + 1023) / 1024;
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);
  int sum = 0;
  for (int i = beg; i < end; ++i) sum += local_counts[i];
  // inclusive scan inside the wave, then across the 16 waves
  const int lane = tid & 63, wid = tid >> 6;
  int v = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int x = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(x, o, kWave);
      if (lane >= o) x += u;
    }
    if (lane < 16) s_wave[lane] = x;
  }
  __syncthreads();
  int run = v - sum + (wid > 0 ? s_wave[wid - 1] : 0);
  for (int i = beg; i < end; ++i) {
    const int c = local_counts[i];
    base[i] = run;
    run += c;
  }
  (void)s_part;
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    int s = 0;
    for (int c = 0; c < C; ++c) s += local_counts[static_cast<size_t>(e) * C + c];
    counts[e] = s;
    offsets[e] = base[static_cast<size_t>(e) * C];
  }
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ base, int P, int k, int C, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  const int e = ids[p];
  const int c = (p / k) / kRouteChunkTokens;
  const int pos = base[static_cast<size_t>(e) * C + c] + rank[p];
  sorted_pairs[pos] = p;
  pair_pos[p] = pos;
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             int32_t* rank, int32_t* local_counts, hipStream_t s) {
  const int n_chunks = (T + kRouteChunkTokens - 1) / kRouteChunkTokens;
  ProfileScope prof(K_ROUTE_TOPK, s);
  hipLaunchKernelGGL(route_topk_kernel, dim3(n_chunks), dim3(256), 0, s, logits, T, E, k, ids, w,
                     rank, local_counts, n_chunks);
  return hipGetLastError();
}

hipError_t launch_route_scan(const int32_t* local_counts, int32_t* base, int E, int n_chunks,
                             int total_pairs, int32_t* counts, int32_t* offsets, hipStream_t s) {
  ProfileScope prof(K_ROUTE_SCAN, s);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, local_counts, base, E,
                     n_chunks, total_pairs, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* base,
                                int T, int k, int n_chunks, int32_t* sorted_pairs,
                                int32_t* pair_pos, hipStream_t s) {
  const int P = T * k;
  ProfileScope prof(K_ROUTE_SCATTER, s);
  hipLaunchKernelGGL(route_scatter_kernel, dim3((P + 255) / 256), dim3(256), 0, s, ids, rank,
                     base, P, k, n_chunks, sorted_pairs, pair_pos);
  return hipGetLastError();
}

}  // namespace moeq2
