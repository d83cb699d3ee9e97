// Router top-k of one token per wave, shared by the routing kernel and the
// decode kernels that route for themselves.
//
// The router selects, per token, the experts whose ids the GPU hands to the
// expert compute ("RTX PRO 4500 单卡跑 125B MoE", lcz.me/topic/2169, section
// 最重要机制, item 1).  Selection compares order-preserving integer keys of
// the float32 logits and breaks ties by the lowest expert id; the weights are
// the softmax over the selected logits (the full softmax renormalised over
// the selection).
#pragma once
#include "q2_device.h"

namespace moeq2 {

// Larger float -> larger key.  Adding +0.0f first maps -0.0 to +0.0, so the
// two zeros compare equal as they do in float32.  Every finite value gets a
// key > 0, so 0 marks an empty or already selected slot.
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_key (a zero comes back as +0.0).
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// b in the lanes whose bit is set in the (wave-uniform) mask, a elsewhere:
// one v_cndmask on a scalar lane mask.  Written out so that the compiler
// keeps the per-round list shift as a handful of selects instead of merging
// the rounds' selects into a position-tracking network.
__device__ __forceinline__ uint32_t select_lanes(uint32_t a, uint32_t b, uint64_t mask) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}

// Top-k of the (key, id) pairs a wave holds, PER per lane (a power of two;
// key 0 marks an empty entry; a lane's ids are id[0], id[0] + 1, ... and
// every id of a lower lane is lower).  Each lane
// first sorts its pairs into selection order (a bitonic network,
// compile-time indices only); then every round takes the wave maximum of the
// lanes' head keys (a DPP wavefront reduction), the lowest lane holding it
// wins -- its head is the lowest id among the equal keys -- and the winner
// shifts its list up by one.  Lane j < k receives the id and the key of
// round j.
template <int PER>
__device__ __forceinline__ void topk_select(uint32_t (&key)[PER], int (&id)[PER], int k, int lane,
                                            int& my_e, uint32_t& my_key) {
  static_assert((PER & (PER - 1)) == 0, "PER must be a power of two");
  // bitonic sort into selection order (position 0 first) on 64-bit words
  // (key, PER - 1 - position): one 64-bit compare per exchange, and since ids
  // ascend with the position inside a lane, the lower id first among equal
  // keys
  uint64_t kp[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) kp[i] = (static_cast<uint64_t>(key[i]) << 32) | (PER - 1 - i);
  const int id0 = id[0];
#pragma unroll
  for (int size = 2; size <= PER; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          // runs of `size` alternate direction; the last merge is forward
          const bool fwd = (i & size) == 0;
          const bool sw = fwd ? kp[j] > kp[i] : kp[i] > kp[j];
          const uint64_t a = kp[i], b = kp[j];
          kp[i] = sw ? b : a;
          kp[j] = sw ? a : b;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    key[i] = static_cast<uint32_t>(kp[i] >> 32);
    id[i] = id0 + (PER - 1 - static_cast<int>(kp[i] & 0xFFFFFFFFu));
  }
  my_e = 0;
  my_key = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t gbest = __ockl_wfred_max_u32(key[0]);
    const uint64_t holders = __ballot(key[0] == gbest);
    const int winner = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(holders)));
    const int e = __builtin_amdgcn_readlane(id[0], winner);
    const uint64_t wm = 1ull << winner;
#pragma unroll
    for (int i = 0; i + 1 < PER; ++i) {
      key[i] = select_lanes(key[i], key[i + 1], wm);
      id[i] = static_cast<int>(select_lanes(static_cast<uint32_t>(id[i]),
                                            static_cast<uint32_t>(id[i + 1]), wm));
    }
    key[PER - 1] = select_lanes(key[PER - 1], 0u, wm);
    if (lane == j) { my_e = e; my_key = gbest; }
  }
}

// One token per wave.  Lane l holds experts l*per .. l*per+per-1, so a lower
// lane always holds lower ids.  PER (>= per) is a compile-time bound; all
// loads are issued before any is used (clamped, so none is conditional).
// Lane j < k receives the id and the logit of round j.
template <int PER>
__device__ __forceinline__ void topk_one_token(const float* __restrict__ row, int E, int k,
                                               int lane, int& my_e, float& my_l) {
  const int per = (E + kWave - 1) / kWave;
  float lv[PER];
  if (PER >= 4 && E == PER * kWave && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    // whole 16-byte vectors per lane (E = 64 * PER)
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + lane * PER + i);
      lv[i] = v[0]; lv[i + 1] = v[1]; lv[i + 2] = v[2]; lv[i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) lv[i] = row[min(lane * per + i, E - 1)];
  }
  uint32_t key[PER];
  int id[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * per + i;
    key[i] = (i < per && e < E) ? float_key(lv[i]) : 0u;
    id[i] = e;
  }
  uint32_t my_key;
  topk_select<PER>(key, id, k, lane, my_e, my_key);
  my_l = key_float(my_key);
}

// Candidates kept per wave by topk_wave_select (at least the largest k).
constexpr int kTopkCand = 16;

// One token's top-k on the 8 waves of a workgroup (the routed workgroups of
// the one-token decode launch, and the one-token routing launch).  Wave w
// takes experts [w * 64 * P, (w + 1) * 64 * P), P per lane (lane l: ids
// w * 64 * P + l * P + i), and keeps its own top k: the keys above the
// wave's k-th largest key (found by bisection on the key bits, each step one
// compare and a population count of its ballot) and, among the keys equal to
// it, the lowest ids.  The union of the waves' own top k holds the global
// top k.  After a barrier, topk_rank8 counts for every candidate how many of
// the 8 * k beat it: that count is its rank in the global selection order.
// Candidates are kept as (key << 32) | ~id: a larger value is the better
// candidate (equal keys: the lower id), and no two are equal.  s_cand has
// 16 entries per wave; unused entries hold 0, which no candidate of a valid
// expert (key > 0) loses to.
template <int P>
__device__ __forceinline__ void topk_wave_load(const float* __restrict__ row, int E, int wid, int lane,
                                               float (&lv)[P]) {
  const int base = wid * kWave * P + lane * P;
#pragma unroll
  for (int i = 0; i < P; ++i) lv[i] = row[min(base + i, E - 1)];
}

template <int P>
__device__ __forceinline__ void topk_wave_select(const float (&lv)[P], int E, int k, int wid, int lane,
                                                 uint64_t (*s_cand)[kTopkCand]) {
  uint32_t key[P];
  const int base = wid * kWave * P + lane * P;
#pragma unroll
  for (int i = 0; i < P; ++i) key[i] = base + i < E ? float_key(lv[i]) : 0u;
  // tau = the largest value with at least k keys >= tau: the k-th largest key
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) cnt += __popcll(__ballot(key[i] >= c));
    tau = cnt >= k ? c : tau;
  }
  // fewer than k keys lie above tau; the rest of the k are the lowest ids
  // among the keys equal to tau (ids ascend with (lane, i))
  int n_gt = 0;
  uint64_t eq[P], gt[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    gt[i] = __ballot(key[i] > tau);
    eq[i] = __ballot(key[i] == tau);
    n_gt += __popcll(gt[i]);
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int ties_before = 0;     // keys equal to tau in lower lanes
#pragma unroll
  for (int i = 0; i < P; ++i) ties_before += __popcll(eq[i] & below);
  if (lane < kTopkCand && lane >= k) s_cand[wid][lane] = 0ull;
  {
    int gt_before = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) gt_before += __popcll(gt[i] & below);
    int t_lo = ties_before, g_lo = gt_before;   // counts of lower ids, then this lane's earlier entries
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool is_gt = key[i] > tau;
      const bool is_eq = key[i] == tau;
      const bool take = is_gt || (is_eq && t_lo < k - n_gt);
      // position: selected entries of lower ids (all the greater ones, and
      // the equal ones that are taken)
      const int pos = g_lo + min(t_lo, k - n_gt);
      if (take) s_cand[wid][pos] = (static_cast<uint64_t>(key[i]) << 32) | static_cast<uint32_t>(~(base + i));
      g_lo += is_gt ? 1 : 0;
      t_lo += is_eq ? 1 : 0;
    }
  }
}

// Ranks of the candidates: each lane holds two of the 128 entries (waves
// 0..3 and 4..7); for each of its wave's 16 entries (read from LDS by every
// lane) a wave counts the entries that beat it with two ballots, the counts
// independent of each other, and lane j (< 16) gets entry j's count in rank
// and the entry itself in mc (entries past k hold 0 and rank last).
__device__ __forceinline__ void topk_rank8(const uint64_t (*s_cand)[kTopkCand], int wid, int lane,
                                           int& rank, uint64_t& mc) {
  static_assert(8 * kTopkCand == 2 * kWave, "two entries per lane");
  const uint64_t* flat = &s_cand[0][0];
  const uint64_t c0 = flat[lane], c1 = flat[kWave + lane];
  mc = s_cand[wid][lane & (kTopkCand - 1)];
  uint64_t mj[kTopkCand];
#pragma unroll
  for (int j = 0; j < kTopkCand; ++j) mj[j] = s_cand[wid][j];
  rank = kTopkCand;
#pragma unroll
  for (int j = 0; j < kTopkCand; ++j) {
    const int r = __popcll(__ballot(c0 > mj[j])) + __popcll(__ballot(c1 > mj[j]));
    rank = lane == j ? r : rank;
  }
}

// Weight of slot `lane` (< k) of a token whose selected logits sit in lanes
// 0..k-1 in descending order: exp(l - l_0) / sum over the k slots.
__device__ __forceinline__ float topk_weight(float l, int k, int lane) {
  const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
  const float z = (lane < k) ? expf(l - lmax) : 0.0f;
  const float sum = wave_sum(z);
  return z / sum;
}

}  // namespace moeq2
