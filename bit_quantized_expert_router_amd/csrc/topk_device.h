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

// One token per wave.  Lane l holds experts l*per .. l*per+per-1, so a lower
// lane always holds lower ids: each round takes the wave maximum of the lanes'
// best keys (a DPP wavefront reduction), the lowest lane holding it wins, and
// inside that lane the lowest position holding it is taken -- together the
// lowest expert id among equal logits.  PER (>= per) is a compile-time bound;
// all loads are issued before any is used (clamped, so none is conditional).
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
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane * per + i;
    key[i] = (i < per && e < E) ? float_key(lv[i]) : 0u;
  }
  my_e = 0;
  uint32_t my_key = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
    int pick = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i) {
      const bool gt = key[i] > best;   // strict: the first position wins ties
      best = gt ? key[i] : best;
      pick = gt ? i : pick;
    }
    const uint32_t gbest = __ockl_wfred_max_u32(best);
    const uint64_t holders = __ballot(best == gbest);
    const int winner = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(holders)));
    const int e = __builtin_amdgcn_readlane(lane * per + pick, winner);
    if (lane == winner) {
#pragma unroll
      for (int i = 0; i < PER; ++i) key[i] = (i == pick) ? 0u : key[i];
    }
    if (lane == j) { my_e = e; my_key = gbest; }
  }
  my_l = key_float(my_key);
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
