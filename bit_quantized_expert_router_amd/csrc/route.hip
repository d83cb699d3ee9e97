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
// Determinism: selection compares order-preserving integer keys of the
// float32 logits; ties are broken by position (lowest expert id), so the
// result does not depend on reduction order.  The permutation is a counting
// sort: each chunk of 64 (or, above 4096 tokens, 256) tokens ranks its pairs
// in pair order inside one wave (so ranks are stable), a single-workgroup
// scan turns the per-chunk counts (laid out expert-major) into the base
// position of every (expert, chunk), and a scatter writes sorted_pairs and
// pair_pos.  Only integer arithmetic decides the order.
#include "launch.h"
#include "q2_device.h"
#include "../../include/moe_q2.h"


namespace moeq2 {

namespace {

// Larger float -> larger key.  Adding +0.0f first maps -0.0 to +0.0, so the
// two zeros compare equal as they do in float32.  Every finite value gets a
// key > 0, so 0 marks an empty or already selected slot.
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One token per wave.  Lane l holds experts l*per .. l*per+per-1, so a lower
// lane always holds lower ids: each round takes the wave maximum of the lanes'
// best keys (a DPP wavefront reduction), the lowest lane holding it wins, and
// inside that lane the lowest position holding it is taken -- together the
// lowest expert id among equal logits.  PER (>= per) is a compile-time bound;
// all loads are issued before any is used (clamped, so none is conditional).
template <int PER>
__device__ __forceinline__ void topk_one_token(const float* __restrict__ row, int E, int k,
                                               int lane, int& my_e, float& my_l) {
  const int per = (E + kWave - 1) / kWave;
  float lv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) lv[i] = row[min(lane * per + i, E - 1)];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * per + i;
    key[i] = (i < per && e < E) ? float_key(lv[i]) : 0u;
  }
  my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t gbest = __ockl_wfred_max_u32(best);
    const uint64_t holders = __ballot(best == gbest);
    const int winner = __builtin_ctzll(holders);
    int pick = PER - 1;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) pick = key[i] == gbest ? i : pick;
    if (lane == winner) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == pick) key[i] = 0u;
    }
    const int e = __shfl(lane * per + pick, winner, kWave);
    if (lane == j) my_e = e;
  }
  my_l = (lane < k) ? row[my_e] : 0.0f;
}

template <int PER>
__global__ __launch_bounds__(1024) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int chunk_tokens,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ rank,
    int32_t* __restrict__ local_counts, int n_chunks) {
  __shared__ int32_t s_ids[kRouteMaxChunkTokens * MOE_MAX_TOPK];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int chunk = blockIdx.x;
  const int t0 = chunk * chunk_tokens;
  const int nt = min(chunk_tokens, T - t0);

  if (rank) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  }
  for (int ti = wid; ti < nt; ti += nwaves) {
    const int t = t0 + ti;
    int my_e;
    float l;
    topk_one_token<PER>(logits + static_cast<size_t>(t) * E, E, k, lane, my_e, l);
    // weights: softmax over the selected logits (slot 0 holds the maximum)
    const float lmax = __shfl(l, 0, kWave);
    const float z = (lane < k) ? expf(l - lmax) : 0.0f;
    const float sum = wave_sum(z);
    if (lane < k) {
      ids[static_cast<size_t>(t) * k + lane] = my_e;
      w[static_cast<size_t>(t) * k + lane] = z / sum;
      if (rank) s_ids[ti * k + lane] = my_e;
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

// One workgroup: exclusive scan of the expert-major [E][C] chunk counts, in
// tiles of 4096 (4 consecutive elements per thread, coalesced 16-byte loads),
// then counts[e] and offsets[e] from the scanned array.
__global__ __launch_bounds__(1024) void route_scan_kernel(
    const int32_t* __restrict__ local_counts, int32_t* __restrict__ base, int E, int C,
    int total, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_carry;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int n = E * C;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int t0 = 0; t0 < n; t0 += 4096) {
    const int i0 = t0 + 4 * tid;
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (i0 + q < n) ? local_counts[i0 + q] : 0;
    const int sum = v[0] + v[1] + v[2] + v[3];
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(x, o, kWave);
      if (lane >= o) x += u;
    }
    if (lane == 63) s_wave[wid] = x;
    __syncthreads();
    if (wid == 0) {
      int y = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const int u = __shfl_up(y, o, kWave);
        if (lane >= o) y += u;
      }
      if (lane < 16) s_wave[lane] = y;
    }
    __syncthreads();
    int run = s_carry + x - sum + (wid > 0 ? s_wave[wid - 1] : 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q < n) base[i0 + q] = run;
      run += v[q];
    }
    __syncthreads();
    if (tid == 1023) s_carry = run;
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  for (int e = tid; e < E; e += 1024) {
    const int b0 = base[static_cast<size_t>(e) * C];
    const int b1 = (e + 1 < E) ? base[static_cast<size_t>(e + 1) * C] : total;
    counts[e] = b1 - b0;
    offsets[e] = b0;
  }
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ base, int P, int k, int C, int chunk_tokens,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  const int e = ids[p];
  const int c = (p / k) / chunk_tokens;
  const int pos = base[static_cast<size_t>(e) * C + c] + rank[p];
  sorted_pairs[pos] = p;
  pair_pos[p] = pos;
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             int32_t* rank, int32_t* local_counts, hipStream_t s) {
  const int ct = route_chunk_tokens(T);
  const int n_chunks = (T + ct - 1) / ct;
  const int threads = T <= 4 ? 64 * T : 1024;
  const int per = (E + kWave - 1) / kWave;
#define MOE_ROUTE_LAUNCH(P)                                                                 \
  launch_kernel(K_ROUTE_TOPK, route_topk_kernel<P>, dim3(n_chunks), dim3(threads), 0, s, logits, \
                T, E, k, ct, ids, w, rank, local_counts, n_chunks)
  if (per <= 1) return MOE_ROUTE_LAUNCH(1);
  if (per <= 2) return MOE_ROUTE_LAUNCH(2);
  if (per <= 4) return MOE_ROUTE_LAUNCH(4);
  if (per <= 8) return MOE_ROUTE_LAUNCH(8);
  return MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
}

hipError_t launch_route_scan(const int32_t* local_counts, int32_t* base, int E, int n_chunks,
                             int total_pairs, int32_t* counts, int32_t* offsets, hipStream_t s) {
  return launch_kernel(K_ROUTE_SCAN, route_scan_kernel, dim3(1), dim3(1024), 0, s, local_counts,
                       base, E, n_chunks, total_pairs, counts, offsets);
}

hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* base,
                                int T, int k, int n_chunks, int32_t* sorted_pairs,
                                int32_t* pair_pos, hipStream_t s) {
  const int P = T * k;
  return launch_kernel(K_ROUTE_SCATTER, route_scatter_kernel, dim3((P + 255) / 256), dim3(256), 0,
                       s, ids, rank, base, P, k, n_chunks, route_chunk_tokens(T), sorted_pairs,
                       pair_pos);
}

}  // namespace moeq2
