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
// sort: each chunk of 16, 64 or 256 tokens (by T) ranks its pairs in pair
// order inside one wave (so ranks are stable) and counts them per expert; one
// wave per expert scans that expert's per-chunk counts (laid out
// expert-major); a scatter kernel adds each expert's offset (every
// workgroup scans the E expert totals itself) and writes sorted_pairs and
// pair_pos.  When one chunk holds every token (T <= 16), its workgroup does
// the scan and the scatter itself and the other two kernels are not
// launched.  Only integer arithmetic decides the order.
#include "launch.h"
#include "q2_device.h"
#include "topk_device.h"
#include "../../include/moe_q2.h"


namespace moeq2 {

namespace {

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(x, o, kWave);
    if (lane >= o) x += u;
  }
  return x;
}

// fin (nullable): when one chunk holds every token, the same workgroup also
// finishes the histogram -- counts, offsets, sorted_pairs and pair_pos, the
// values the scan and scatter kernels would compute with a single chunk.
struct RouteFinish {
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pairs;
  int32_t* pair_pos;
};
constexpr int kRouteFusedPairs = 16 * MOE_MAX_TOPK;   // one chunk of at most 16 tokens

// WIDE: one token on 8 waves (topk_wave_select / topk_rank8): each wave
// selects from its slice of the logits, the candidates are ranked after a
// barrier, and wave 0 computes the weights from the ranked logits -- the
// ids, weights and histogram equal those of one wave taking the whole row.
template <int PER, bool WIDE>
__global__ __launch_bounds__(1024) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int chunk_tokens,
    int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ rank,
    int32_t* __restrict__ local_counts, int n_chunks, RouteFinish fin) {
  __shared__ int32_t s_ids[kRouteMaxChunkTokens * MOE_MAX_TOPK];
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ int32_t s_rank[kRouteFusedPairs];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS];
  __shared__ uint64_t s_cand[WIDE ? 8 : 1][kTopkCand];
  __shared__ int32_t s_wid[kTopkCand];
  __shared__ float s_wlg[kTopkCand];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  const int chunk = blockIdx.x;
  const int t0 = chunk * chunk_tokens;
  const int nt = min(chunk_tokens, T - t0);

  if (rank) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
  }
  if constexpr (WIDE) {
    // T = 1, one chunk, 8 waves
    static_assert(kTopkCand >= MOE_MAX_TOPK, "candidates per wave");
    constexpr int P8 = PER / 8 > 0 ? PER / 8 : 1;
    float lv[P8];
    topk_wave_load<P8>(logits, E, wid, lane, lv);
    topk_wave_select<P8>(lv, E, k, wid, lane, s_cand);
    __syncthreads();
    int r;
    uint64_t mc;
    topk_rank8(s_cand, wid, lane, r, mc);
    if (lane < k && r < k) {
      s_wid[r] = static_cast<int>(~static_cast<uint32_t>(mc));
      s_wlg[r] = key_float(static_cast<uint32_t>(mc >> 32));
    }
    __syncthreads();
    if (wid == 0) {
      const float l = lane < k ? s_wlg[lane] : 0.0f;
      const float wt = topk_weight(l, k, lane);
      if (lane < k) {
        const int e = s_wid[lane];
        ids[lane] = e;
        w[lane] = wt;
        if (rank) s_ids[lane] = e;
      }
    }
  } else {
    for (int ti = wid; ti < nt; ti += nwaves) {
      const int t = t0 + ti;
      int my_e;
      float l;
      topk_one_token<PER>(logits + static_cast<size_t>(t) * E, E, k, lane, my_e, l);
      const float wt = topk_weight(l, k, lane);
      if (lane < k) {
        ids[static_cast<size_t>(t) * k + lane] = my_e;
        w[static_cast<size_t>(t) * k + lane] = wt;
        if (rank) s_ids[ti * k + lane] = my_e;
      }
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
      if (fin.counts && active) s_rank[p] = base + before;
      if (active && before == 0) s_cnt[e] = base + cnt;
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  if (!fin.counts) {
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      local_counts[static_cast<size_t>(e) * n_chunks + chunk] = s_cnt[e];
    return;
  }
  // single chunk: offsets = exclusive scan of the counts (wave 0, 64 experts
  // at a time), then every pair's position (expert-major, stable)
  if (wid == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? s_cnt[e] : 0;
      const int incl = wave_incl_scan(v, lane);
      if (e < E) {
        fin.counts[e] = v;
        fin.offsets[e] = carry + incl - v;
        s_off[e] = carry + incl - v;
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) fin.offsets[E] = carry;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < nt * k; p += blockDim.x) {
    const int pos = s_off[s_ids[p]] + s_rank[p];
    fin.sorted_pairs[pos] = p;
    fin.pair_pos[p] = pos;
  }
}

// One wave per expert: the exclusive scan of its row of the expert-major
// [E][C] chunk counts gives, for every chunk, the number of the expert's
// pairs in earlier chunks (ebase); the row total is counts[e].
__global__ __launch_bounds__(1024) void route_expert_scan_kernel(
    const int32_t* __restrict__ local_counts, int32_t* __restrict__ ebase, int E, int C,
    int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 16 + static_cast<int>(threadIdx.x >> 6);
  if (e >= E) return;
  const int32_t* row = local_counts + static_cast<size_t>(e) * C;
  int32_t* out = ebase + static_cast<size_t>(e) * C;
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += kWave) {
    const int c = c0 + lane;
    const int v = c < C ? row[c] : 0;
    const int incl = wave_incl_scan(v, lane);
    if (c < C) out[c] = carry + incl - v;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) counts[e] = carry;
}

// One thread per pair: pos = offsets[e] + ebase[e][chunk] + rank.  Every
// workgroup derives offsets (the exclusive scan of counts over the E <= 1024
// experts) itself; workgroup 0 also writes them out.
__global__ __launch_bounds__(1024) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ ebase, const int32_t* __restrict__ counts, int E, int P, int k,
    int C, int chunk_tokens, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos) {
  __shared__ int32_t s_off[MOE_MAX_EXPERTS];
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  // this thread's pair first (independent of the scan)
  const int p = blockIdx.x * 1024 + tid;
  const int pc = min(p, P - 1);
  const int e = ids[pc];
  const int r = rank[pc];
  const int v = tid < E ? counts[tid] : 0;
  const int incl = wave_incl_scan(v, lane);
  if (lane == 63) s_wave[wid] = incl;
  __syncthreads();
  int wb = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) wb += (q < wid) ? s_wave[q] : 0;
  const int off = wb + incl - v;
  if (tid < E) {
    s_off[tid] = off;
    if (blockIdx.x == 0) offsets[tid] = off;
  }
  if (blockIdx.x == 0 && tid == 0) offsets[E] = P;
  __syncthreads();
  if (p < P) {
    const int c = (p / k) / chunk_tokens;
    const int pos = s_off[e] + ebase[static_cast<size_t>(e) * C + c] + r;
    sorted_pairs[pos] = p;
    pair_pos[p] = pos;
  }
}


// ------------------------------------------------- router GEMV + top-k --
// Router logits computed on the device and the top-k taken in the same
// kernel (decode, T <= 4): logits[t][e] = fp32(sum_h x[t][h] * W[e][h]),
// W the bf16 router weight [E][H].  Every product of a bf16 weight and a
// bf16 or fp32 activation is exact in fp64, and the sum is accumulated in
// fp64 (lane partial sums over fixed columns, then a fixed-order wavefront
// reduction) and rounded once to fp32, so the logits agree with a plain fp64
// dot product except when that one rounding falls within the fp64 summation
// error of an fp32 rounding boundary.  Each wave computes the logits of one
// expert for all T tokens.  With `ids` given, the last workgroup to finish
// (one agent-scope atomic per workgroup on a counter it then resets) selects
// the top-k from the logits written by all of them; no workgroup waits for
// another.  Without `ids` the kernel only writes the logits.
constexpr int kGemvWaves = 4;
constexpr int kGemvExpertsPerWave = 1;
constexpr int kGemvExpertsPerBlock = kGemvWaves * kGemvExpertsPerWave;

extern "C" __device__ double __ockl_wfred_add_f64(double);

// NC: 512-column chunks per lane (ceil(H / 512)); the router weight rows
// are read first (all of them in flight at once) while x is staged in LDS.
template <bool BF16X, int PER, int NC>
__global__ __launch_bounds__(64 * kGemvWaves) void route_gemv_topk_kernel(
    const void* __restrict__ x, int T, const uint16_t* __restrict__ W, int E, int H, int k,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w,
    uint32_t* __restrict__ counter) {
  extern __shared__ __align__(16) float s_x[];   // [T][H] as float32
  __shared__ uint32_t s_last;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int e0 = (blockIdx.x * kGemvWaves + wid) * kGemvExpertsPerWave;
  // weight rows: lane covers columns 8 * lane + 512 * c .. + 7 (clamped loads)
  u32x4 wr[NC][kGemvExpertsPerWave];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int q = 0; q < kGemvExpertsPerWave; ++q)
      wr[c][q] = *reinterpret_cast<const u32x4*>(
          W + static_cast<size_t>(min(e0 + q, E - 1)) * H + min(8 * lane + 512 * c, H - 8));
  // x into LDS as float32 (8 values per thread and step)
  for (int i = 8 * static_cast<int>(threadIdx.x); i < T * H; i += 8 * 64 * kGemvWaves) {
    f32x4 a, b;
    if (BF16X) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + i);
      a = f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xFFFF0000u),
                __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xFFFF0000u)};
      b = f32x4{__uint_as_float(r[2] << 16), __uint_as_float(r[2] & 0xFFFF0000u),
                __uint_as_float(r[3] << 16), __uint_as_float(r[3] & 0xFFFF0000u)};
    } else {
      a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + i);
      b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + i + 4);
    }
    *reinterpret_cast<f32x4*>(s_x + i) = a;
    *reinterpret_cast<f32x4*>(s_x + i + 4) = b;
  }
  __syncthreads();
  double acc[kGemvExpertsPerWave][MOE_MAX_GEMV_TOKENS];
#pragma unroll
  for (int q = 0; q < kGemvExpertsPerWave; ++q)
#pragma unroll
    for (int t = 0; t < MOE_MAX_GEMV_TOKENS; ++t) acc[q][t] = 0.0;
#pragma unroll
  for (int t = 0; t < MOE_MAX_GEMV_TOKENS; ++t) {
    if (t < T) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int c0 = 8 * lane + 512 * c;
        if (c0 < H) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(s_x + t * H + c0);
          const f32x4 b = *reinterpret_cast<const f32x4*>(s_x + t * H + c0 + 4);
          const double xv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
          for (int q = 0; q < kGemvExpertsPerWave; ++q) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const double wlo = static_cast<double>(__uint_as_float(wr[c][q][i] << 16));
              const double whi = static_cast<double>(__uint_as_float(wr[c][q][i] & 0xFFFF0000u));
              acc[q][t] = __builtin_fma(wlo, xv[2 * i], acc[q][t]);
              acc[q][t] = __builtin_fma(whi, xv[2 * i + 1], acc[q][t]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kGemvExpertsPerWave; ++q) {
#pragma unroll
    for (int t = 0; t < MOE_MAX_GEMV_TOKENS; ++t) {
      if (t < T) {
        const double sum = __ockl_wfred_add_f64(acc[q][t]);
        if (lane == 0 && e0 + q < E) logits[static_cast<size_t>(t) * E + e0 + q] = static_cast<float>(sum);
      }
    }
  }
  if (ids == nullptr) return;
  // Publish this workgroup's logits; the last workgroup selects.  The block
  // barrier completes every wave's stores (they are in this XCD's L2); thread
  // 0's arrival is a device-scope release (one L2 write-back per workgroup)
  // and, for the last workgroup, an acquire that invalidates this CU's and
  // XCD's stale lines before any wave reads the logits.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == gridDim.x - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  if (wid < T) {
    int my_e;
    float l;
    topk_one_token<PER>(logits + static_cast<size_t>(wid) * E, E, k, lane, my_e, l);
    const float wt = topk_weight(l, k, lane);
    if (lane < k) {
      ids[static_cast<size_t>(wid) * k + lane] = my_e;
      w[static_cast<size_t>(wid) * k + lane] = wt;
    }
  }
  if (threadIdx.x == 0) counter[0] = 0u;   // ready for the next call
}

}  // namespace

bool route_histogram_fused(int T, int k) {
  return (T + route_chunk_tokens(T) - 1) / route_chunk_tokens(T) == 1 && T * k <= kRouteFusedPairs;
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             int32_t* rank, int32_t* local_counts, hipStream_t s, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos) {
  const int ct = route_chunk_tokens(T);
  const int n_chunks = (T + ct - 1) / ct;
  // one chunk of at most 16 tokens: the histogram is finished in the same kernel
  const RouteFinish fin = (rank && counts && route_histogram_fused(T, k))
                              ? RouteFinish{counts, offsets, sorted_pairs, pair_pos}
                              : RouteFinish{nullptr, nullptr, nullptr, nullptr};
  // one token: 8 waves share its top-k; 2..4 tokens: one wave each
  const int threads = T == 1 ? 8 * kWave : T <= 4 ? 64 * T : 1024;
  const int per = (E + kWave - 1) / kWave;
#define MOE_ROUTE_LAUNCH(P)                                                                         \
  (T == 1 ? launch_kernel(K_ROUTE_TOPK, route_topk_kernel<P, true>, dim3(n_chunks), dim3(threads), 0, s, \
                          logits, T, E, k, ct, ids, w, rank, local_counts, n_chunks, fin)                  \
          : launch_kernel(K_ROUTE_TOPK, route_topk_kernel<P, false>, dim3(n_chunks), dim3(threads), 0, s, \
                          logits, T, E, k, ct, ids, w, rank, local_counts, n_chunks, fin))
  if (per <= 1) return MOE_ROUTE_LAUNCH(1);
  if (per <= 2) return MOE_ROUTE_LAUNCH(2);
  if (per <= 4) return MOE_ROUTE_LAUNCH(4);
  if (per <= 8) return MOE_ROUTE_LAUNCH(8);
  return MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
}

hipError_t launch_route_expert_scan(const int32_t* local_counts, int32_t* ebase, int E, int n_chunks,
                                    int32_t* counts, hipStream_t s) {
  return launch_kernel(K_ROUTE_SCAN, route_expert_scan_kernel, dim3((E + 15) / 16), dim3(1024), 0, s,
                       local_counts, ebase, E, n_chunks, counts);
}

hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* ebase,
                                const int32_t* counts, int E, int T, int k, int n_chunks,
                                int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                                hipStream_t s) {
  const int P = T * k;
  return launch_kernel(K_ROUTE_SCATTER, route_scatter_kernel, dim3((P + 1023) / 1024), dim3(1024), 0,
                       s, ids, rank, ebase, counts, E, P, k, n_chunks, route_chunk_tokens(T),
                       offsets, sorted_pairs, pair_pos);
}

hipError_t launch_route_gemv_topk(const void* x, int x_bf16, int T, const uint16_t* W, int E, int H,
                                  int k, float* logits, int32_t* ids, float* w, uint32_t* counter,
                                  hipStream_t s) {
  const dim3 grid((E + kGemvExpertsPerBlock - 1) / kGemvExpertsPerBlock), block(64 * kGemvWaves);
  const uint32_t lds = static_cast<uint32_t>(T) * H * 4u;
  const int per = (E + kWave - 1) / kWave;
  const int nc = (H + 511) / 512;
  // (x dtype, top-k lane bound, column chunks): the common shapes get exact
  // chunk counts, the rest the largest
#define MOE_GEMV_LAUNCH(XB, P, NC)                                                              \
  launch_kernel(K_ROUTE_GEMV_TOPK, route_gemv_topk_kernel<XB, P, NC>, grid, block, lds, s, x, T, W, \
                E, H, k, logits, ids, w, counter)
#define MOE_GEMV_NC(XB, P)                          \
  (nc <= 2 ? MOE_GEMV_LAUNCH(XB, P, 2)              \
           : nc <= 6 ? MOE_GEMV_LAUNCH(XB, P, 6) : MOE_GEMV_LAUNCH(XB, P, 16))
#define MOE_GEMV_PER(XB)                                                     \
  (per <= 1 ? MOE_GEMV_NC(XB, 1)                                             \
            : per <= 8 ? MOE_GEMV_NC(XB, 8) : MOE_GEMV_NC(XB, 16))
  return x_bf16 ? MOE_GEMV_PER(true) : MOE_GEMV_PER(false);
#undef MOE_GEMV_PER
#undef MOE_GEMV_NC
#undef MOE_GEMV_LAUNCH
}

}  // namespace moeq2
