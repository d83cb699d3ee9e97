// Device-side building blocks for gfx950 (CDNA4, wave64).
//
// Numeric scheme of the expert kernels
//   * Weights: a tile lane's 32-bit code word holds 8 codes of block 2i and 8
//     of block 2i+1 (two bits per nibble).  w & 0x33333333 leaves each code
//     of block 2i alone in a nibble, i.e. an fp4 (e2m1) number q/2, and
//     (w >> 2) & 0x33333333 does the same for block 2i+1.  The gfx950
//     scaled fp4->fp16 conversion with scale 2.0 turns two such nibbles into
//     two fp16 values q, and one packed fp16 fma q*d - d gives d*(q-1)
//     exactly (fp16 holds -d, 0, d and 2d exactly).  So each weight costs
//     about 1.2 VALU operations and the MFMA B operand is the exact weight.
//   * Activations enter the MFMA as fp16: per token x_hat is multiplied by a
//     power of two s_t so that max|x_hat*s_t| lies in [0.5, 1); the fp32
//     accumulators are multiplied back by 1/s_t (exact).
//   * v_mfma_f32_16x16x32_f16: lane l supplies A[i = l%16][k = 8(l/16) + e]
//     and B[k = 8(l/16) + e][j = l%16] for e = 0..7 and receives
//     D[4(l/16) + r][l%16] in accumulator element r.  A and B use the same
//     (lane group, element) -> k assignment, so the dot products do not
//     depend on how the hardware orders k inside the instruction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;
constexpr int kTileCols = 256;
constexpr int kTileBytes = 1280;
constexpr int kCodeBytes = 1024;
constexpr int kWave = 64;

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four consecutive fp4 code pairs of one nibble word -> 8 fp16 weights d*(q-1).
__device__ __forceinline__ f16x8 nibbles_to_weights(uint32_t nib, f16x2 dd) {
  f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 0);
  f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 1);
  f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 2);
  f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 2.0f, 3);
  f16x2 nd = -dd;
  q0 = __builtin_elementwise_fma(q0, dd, nd);
  q1 = __builtin_elementwise_fma(q1, dd, nd);
  q2 = __builtin_elementwise_fma(q2, dd, nd);
  q3 = __builtin_elementwise_fma(q3, dd, nd);
  f16x8 r;
  r[0] = q0[0]; r[1] = q0[1]; r[2] = q1[0]; r[3] = q1[1];
  r[4] = q2[0]; r[5] = q2[1]; r[6] = q3[0]; r[7] = q3[1];
  return r;
}

// Scale of block j (0..7) of the lane's row, from the row's 16 scale bytes,
// duplicated into both halves with integer operations.  (Letting the packed
// fma broadcast one half through its operand-select bits instead gave wrong
// products on gfx950 in a direct comparison, so that form is not used.)
__device__ __forceinline__ f16x2 scale_pair(const u32x4& s, int j) {
  uint32_t w = s[j >> 1];
  uint32_t h = (j & 1) ? (w >> 16) : (w & 0xFFFFu);
  uint32_t p = h | (h << 16);
  return __builtin_bit_cast(f16x2, p);
}

// B fragment of block j of a tile for this lane: code words `c`, scales `s`.
__device__ __forceinline__ f16x8 tile_block_weights(const u32x4& c, const u32x4& s, int j) {
  uint32_t w = c[j >> 1];
  uint32_t nib = (j & 1) ? ((w >> 2) & 0x33333333u) : (w & 0x33333333u);
  return nibbles_to_weights(nib, scale_pair(s, j));
}

// Loads of one tile record for this lane (n = lane % 16, g = lane / 16).
__device__ __forceinline__ u32x4 load_codes(const uint8_t* rec, int lane) {
  return *reinterpret_cast<const u32x4*>(rec + 16 * lane);
}
__device__ __forceinline__ u32x4 load_scales(const uint8_t* rec, int lane) {
  return *reinterpret_cast<const u32x4*>(rec + kCodeBytes + 16 * (lane & 15));
}

// The same loads through a buffer resource: `base` (wave-uniform) is one
// expert, `rec_off` (wave-uniform) the byte offset of the record in it, so
// the address is a scalar base + scalar offset + a per-lane constant (no
// 64-bit vector address arithmetic).  `bytes` bounds the resource: a load
// past it returns zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t expert_rsrc(const uint8_t* base, uint32_t bytes) {
  // the caller guarantees uniformity; readfirstlane lets the compiler keep
  // the resource in scalar registers
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  uint8_t* p = reinterpret_cast<uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 load_codes(__amdgpu_buffer_rsrc_t r, uint32_t rec_off, int lane) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, rec_off, 0);
}
__device__ __forceinline__ u32x4 load_scales(__amdgpu_buffer_rsrc_t r, uint32_t rec_off, int lane) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, kCodeBytes + 16 * (lane & 15), rec_off, 0);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// Per-token power-of-two normaliser of the activations: returns s = 2^-e
// with max_abs * s in [0.5, 1) (s = 1 for an all-zero token), e clamped to
// [-60, 60] so that s and 1/s stay normal float32 numbers.  A token whose
// largest |x_hat| is beyond 2^60 has outputs (degree 2 in x) beyond float32.
__device__ __forceinline__ float pow2_normaliser(float max_abs) {
  if (!(max_abs > 0.0f)) return 1.0f;
  int e;
  frexpf(max_abs, &e);
  e = e < -60 ? -60 : (e > 60 ? 60 : e);
  return ldexpf(1.0f, -e);
}

// Exponent of a block of intermediate values (h or y rows): e with
// max_abs * 2^-e in [0.5, 1), so the block stored as fp16 v * 2^-e lies in
// (-1, 1) and cannot overflow; clamped to [-120, 127].  An all-zero block
// gets kZeroExp, below every other exponent, so it never sets a maximum.
constexpr int kZeroExp = -128;
__device__ __forceinline__ int block_exponent(float max_abs) {
  if (!(max_abs > 0.0f)) return kZeroExp;
  int e;
  frexpf(max_abs, &e);
  return e < -120 ? -120 : (e > 127 ? 127 : e);
}

// Maximum over the 16 lanes of this lane's DPP row (lanes 16r..16r+15),
// returned in every lane of the row; all 16 lanes must be active.
__device__ __forceinline__ float row16_max(float v) {
  int x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false)));  // quad [1,0,3,2]
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false)));  // quad [2,3,0,1]
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false))); // half-row mirror
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false))); // row mirror
  return v;
}

// fp16 bits of 2^d in both halves of a word, d <= 0: a normal number for
// d >= -14, a subnormal for -24 <= d < -14, zero below.  Built with integer
// operations so that the multiply takes it as an ordinary register operand
// (a half-word broadcast through the packed instruction's operand-select
// bits gave wrong products on gfx950 in a direct comparison).
__device__ __forceinline__ uint32_t pow2_f16x2_bits(int d) {
  const uint32_t b = d >= -14 ? static_cast<uint32_t>(d + 15) << 10
                              : (d >= -24 ? 1u << (d + 24) : 0u);
  return b | (b << 16);
}

// 8 fp16 values times 2^d for d <= 0 (exact unless the result is subnormal;
// below 2^-24 of the input the values become zero).
__device__ __forceinline__ f16x8 scale_pow2(const f16x8& a, int d) {
  const f16x2 s = __builtin_bit_cast(f16x2, pow2_f16x2_bits(d));
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 v = {a[2 * i], a[2 * i + 1]};
    const f16x2 p = v * s;
    r[2 * i] = p[0];
    r[2 * i + 1] = p[1];
  }
  return r;
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);   // round to nearest even (finite inputs)
  return static_cast<uint16_t>(u >> 16);
}

}  // namespace moeq2

// Wavefront reductions of the ROCm device library (DPP based, fixed order).
extern "C" __device__ float __ockl_wfred_add_f32(float);
extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);

namespace moeq2 {

__device__ __forceinline__ float wave_sum(float v) { return __ockl_wfred_add_f32(v); }
__device__ __forceinline__ float wave_max(float v) { return __ockl_wfred_max_f32(v); }

// Bit mask of the lanes (among `active`) whose value equals this lane's;
// values must be < 2^nbits.  nbits ballots, no shuffles.
__device__ __forceinline__ uint64_t match_lanes(int v, bool active, int nbits) {
  uint64_t same = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (v >> b) & 1;
    const uint64_t bb = __ballot(active && bit);
    same &= bit ? bb : ~bb;
  }
  return same;
}

// Wave-uniform integer broadcast helper.
__device__ __forceinline__ int first_lane_value(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace moeq2
