// Prefill-time expert layer: a chunk of T tokens (1024 or 32768 in the
// target workloads), grouped by expert from the routing histogram.
//
// Prompt chunks are read expert block by expert block (strata-mlx README,
// section 它是什么); larger chunks spread each expert's weight read over more
// tokens ("Strata 实测 ...", kefong.net, section 四, change 4).  Here every
// expert's rows (its token-expert pairs, in the stable sorted order from the
// router) are cut into work items of up to 64 rows; the shared expert is one
// more "expert" whose rows are all T tokens, with weight 1.
//
// Kernels (all enqueued on the caller's stream, no host round trip):
//   prep     token t: x_hat = x (* rsqrt(mean x^2 + 1e-6)), times a power of
//            two s_t (max |x_hat s_t| in [0.5, 1)), stored fp16 [T][H]; one
//            workgroup turns `counts` into the work-item list, the others
//            write each sorted row's token and routing weight.
//   gateup   work item x 128-row block of I, 8 waves (one 16-row tile of
//            gate and of up each; two of each and 256-row blocks for chunks
//            of more than 8192 tokens): A = the item's gathered x rows (fp16,
//            staged in LDS, double buffered per 256-column K tile), B = the
//            expert's gate and up tiles dequantized in registers (each weight
//            is dequantized once per item and used by every M tile; two
//            register sets keep the next K tile's weights in flight while
//            one is multiplied),
//            v_mfma_f32_16x16x32_f16, SwiGLU epilogue: h = w * silu(g) * u
//            in float32, stored (sorted-row order) as fp16 h * 2^-e with one
//            exponent e per (row, 16-row tile of I) in a byte array, so that
//            |h~| < 1 and fp16 cannot overflow whatever the weights' scales.
//   down     A = h rows rescaled to one exponent per row (the row's
//            largest) while they are moved into LDS, B = down tiles, 8 waves x
//            2 row tiles of H; y = acc * 2^E_row, stored as fp16 y * 2^-F
//            with one exponent F per (row, 8 columns): each wave turns its
//            accumulators around through LDS so that a lane holds 8
//            consecutive columns of one row.  For I <= 768 the item's h rows
//            stay in LDS while the workgroup runs three 256-row chunks of H
//            (half items of 32 rows for chunks of up to 4096 tokens, so that
//            two workgroups fit on a CU); wider I stages h per K tile for
//            each 256-row block.
//   combine  token t: out = sum_j y~[pair_pos[t,j]] * 2^F + y~[shared row]
//            * 2^F (+ residual), j ascending: fixed order, no atomics.
// Workgroup ids are remapped so that every XCD gets an equal share of the
// real work and the row blocks of one work item (which read the same A rows)
// run on the same XCD and share its L2.  Chunks of up to 4096 tokens list
// the items by size (longest first) and deal them to the XCDs in turn;
// longer chunks list them in expert order and give each XCD one contiguous
// range, so that an expert's items share its weights in one L2.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "launch.h"
#include "q2_device.h"
#include "../../include/moe_q2.h"

namespace moeq2 {

namespace {

constexpr int kGemmWaves = 8;               // waves per GEMM workgroup
constexpr int kThreads = 64 * kGemmWaves;
constexpr int kDownRTW = kGemmWaves == 16 ? 1 : 2;          // 16-row tiles of H per wave
constexpr int kGateupRowsPerBlock = 16 * kGemmWaves;        // 16 rows of I (gate and up) per wave
constexpr int kDownRowsPerBlock = 16 * kDownRTW * kGemmWaves;
constexpr int kGateupRing = 2;              // K tiles of weights in flight per wave
constexpr int kDownRing = 2;

struct PrefillWs {
  int32_t* hdr;        // [0] = number of work items
  int4* items;         // {expert, row0, nrows, slot: the expert itself, or its residency slot, -1 = arena}
  float* unscale;      // [T]  1 / s_t
  int32_t* row_tok;    // [rows] token of each sorted row
  float* row_w;        // [rows] routing weight of each sorted row (1 for the shared expert)
  _Float16* x16;       // [T][H]
  _Float16* h;         // [rows][I]     h * 2^-hexp
  _Float16* y;         // [rows][H]     y * 2^-yexp
  int8_t* hexp;        // [rows][I/16]  exponent of each 16-row tile of I
  int8_t* yexp;        // [rows][H/8]   exponent of each 8 columns of H
};
constexpr int kYGroup = 8;                   // columns of y per exponent (one 16-byte chunk)

__host__ __device__ inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

__host__ __device__ inline int max_items(int T, int E, int k) {
  const long long P = static_cast<long long>(T) * k;
  return static_cast<int>((P + kGroupRows - 1) / kGroupRows + E + (T + kGroupRows - 1) / kGroupRows + 1);
}

__host__ __device__ inline PrefillWs carve(void* base, int T, int E, int k, int H, int I) {
  uint8_t* p = static_cast<uint8_t*>(base);
  const size_t rows = static_cast<size_t>(T) * k + T;
  PrefillWs w;
  w.hdr = reinterpret_cast<int32_t*>(p); p += 256;
  w.items = reinterpret_cast<int4*>(p); p += align256(sizeof(int4) * max_items(T, E, k));
  w.unscale = reinterpret_cast<float*>(p); p += align256(sizeof(float) * T);
  w.row_tok = reinterpret_cast<int32_t*>(p); p += align256(sizeof(int32_t) * rows);
  w.row_w = reinterpret_cast<float*>(p); p += align256(sizeof(float) * rows);
  w.x16 = reinterpret_cast<_Float16*>(p); p += align256(sizeof(_Float16) * static_cast<size_t>(T) * H);
  w.h = reinterpret_cast<_Float16*>(p); p += align256(sizeof(_Float16) * rows * I);
  w.y = reinterpret_cast<_Float16*>(p); p += align256(sizeof(_Float16) * rows * H);
  w.hexp = reinterpret_cast<int8_t*>(p); p += align256(rows * (I / kTileRows));
  w.yexp = reinterpret_cast<int8_t*>(p);
  return w;
}

// Work unit of a block, or -1.  Blocks are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8); the n real units (known only on the device)
// are split into 8 contiguous ranges, one per XCD, so every XCD gets the
// same share and consecutive units (the row blocks of one work item, which
// read the same activation rows) share an XCD's L2.  The grid is sized for
// the largest possible n; blocks beyond the work return at once.
__device__ __forceinline__ int xcd_unit(int bid, int n) {
  const int per = (n + 7) / 8;
  const int i = bid / 8;
  const int u = (bid % 8) * per + i;
  return (i < per && u < n) ? u : -1;
}

// Work item and row block of a GEMM block (item -1: none).  hdr[1] = 0:
// units item * RB + rb in contiguous ranges per XCD (xcd_unit); hdr[1] = 1:
// item i on XCD i % 8, the XCD's items in list order, each item's RB row
// blocks in a row.  The grid covers 8 * ceil(items / 8) * RB blocks.
__device__ __forceinline__ int2 work_unit(int bid, const int32_t* hdr, int RB) {
  const int n = hdr[0];
  if (hdr[1]) {
    const int j = bid >> 3;
    const int item = (bid & 7) + 8 * (j / RB);
    return item < n ? make_int2(item, j % RB) : make_int2(-1, 0);
  }
  const int u = xcd_unit(bid, n * RB);
  return u < 0 ? make_int2(-1, 0) : make_int2(u / RB, u % RB);
}

// Where a work item's expert sits: the w field holds its slot (the expert
// itself without the residency tier; -1 = in the arena), set by prep.
__device__ __forceinline__ int item_slot(const LayerArgs& L, int e) {
  if (e >= L.E || !L.slot_of) return e;
  const int s = L.slot_of[e];
  return s >= 0 && s < L.S ? s : -1;
}
__device__ __forceinline__ const uint8_t* expert_base(const LayerArgs& L, const int4& it) {
  if (it.x >= L.E) return L.shared;
  return it.w >= 0 ? L.experts + static_cast<int64_t>(it.w) * L.stride
                   : L.arena + static_cast<int64_t>(it.x) * L.stride;
}

// --------------------------------------------------------------------- prep --
constexpr int kPrepTokensPerBlock = 4;                // one wave per token
constexpr int kSizeOrderMaxTokens = 4096;             // chunks up to this long: items by size, dealt round robin

// One x row as 8-element chunks (16 bytes of bf16 or 32 of fp32); lane l
// holds chunks l, l + 64, ... (at most NCL of them) in registers, so the row
// is read once.
template <bool BF16>
__device__ __forceinline__ void load_x_chunk(const void* x, size_t e0, u32x4 (&r)[2]) {
  if constexpr (BF16) {
    r[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + e0);
    r[0] = p[0];
    r[1] = p[1];
  }
}

template <bool BF16>
__device__ __forceinline__ float x_chunk_elem(const u32x4 (&r)[2], int i) {
  if constexpr (BF16) {
    const uint32_t w = r[0][i >> 1];   // element 2j is the low half of word j
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return __uint_as_float(r[i >> 2][i & 3]);
  }
}

// x_hat_t = x_t (* rsqrt(mean x_t^2 + 1e-6)) times the power of two s_t that
// puts max |x_hat_t s_t| in [0.5, 1), stored fp16; unscale[t] = 1 / s_t.
template <bool BF16, int NCL>
__device__ void prep_token(const void* __restrict__ x, int t, int H, int prenorm, const PrefillWs& ws) {
  const int lane = threadIdx.x & 63;
  const int nch = H >> 3;
  u32x4 r[NCL][2];
#pragma unroll
  for (int i = 0; i < NCL; ++i)
    if (64 * i + lane < nch) load_x_chunk<BF16>(x, static_cast<size_t>(t) * H + 8 * (64 * i + lane), r[i]);
  float ss = 0.0f, mx = 0.0f;
#pragma unroll
  for (int i = 0; i < NCL; ++i) {
    if (64 * i + lane < nch) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = x_chunk_elem<BF16>(r[i], j);
        ss += v * v;
        mx = fmaxf(mx, fabsf(v));
      }
    }
  }
  ss = wave_sum(ss);
  mx = wave_max(mx);
  const float rn = prenorm ? 1.0f / sqrtf(ss / static_cast<float>(H) + 1e-6f) : 1.0f;
  const float sc = pow2_normaliser(mx * rn);
#pragma unroll
  for (int i = 0; i < NCL; ++i) {
    if (64 * i + lane < nch) {
      f16x8 h;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = static_cast<_Float16>((x_chunk_elem<BF16>(r[i], j) * rn) * sc);
      *reinterpret_cast<f16x8*>(ws.x16 + static_cast<size_t>(t) * H + 8 * (64 * i + lane)) = h;
    }
  }
  if (lane == 0) ws.unscale[t] = 1.0f / sc;
}

// Blocks [0, TB): x_hat of 4 tokens each (TB = ceil(T / 4)); block TB: the
// work-item list; blocks after it: token and weight of 256 sorted rows each.
template <bool XBF16, int NCL>
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    LayerArgs L, const void* __restrict__ x, int T, int k, int prenorm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pairs, const float* __restrict__ topk_w, int item_cap,
    PrefillWs ws) {
  __shared__ int s_scan[256];
  __shared__ uint64_t s_scan64[256];
  const int H = L.H, E = L.E;
  const int P = T * k;
  const int TB = (T + kPrepTokensPerBlock - 1) / kPrepTokensPerBlock;
  if (blockIdx.x < TB) {
    const int t = blockIdx.x * kPrepTokensPerBlock + (threadIdx.x >> 6);
    if (t < T) prep_token<XBF16, NCL>(x, t, H, prenorm, ws);
    return;
  }
  if (blockIdx.x > TB) {
    // token and weight of every sorted row (an invalid entry contributes nothing)
    const int r = (blockIdx.x - TB - 1) * 256 + threadIdx.x;
    if (r < P) {
      const int p = sorted_pairs[r];
      const bool ok = p >= 0 && p < P;
      ws.row_tok[r] = ok ? p / k : 0;
      ws.row_w[r] = ok ? topk_w[p] : 0.0f;
    } else if (r < P + T) {
      ws.row_tok[r] = r - P;
      ws.row_w[r] = 1.0f;
    }
    return;
  }
  // ---- work items from the histogram -----------------------------------
  // (rows of expert e: [offsets[e], offsets[e] + counts[e]) clipped to
  // [0, T*k), so inconsistent histogram arrays cannot send any later kernel
  // outside its buffers)
  const int nexp = E + (L.shared ? 1 : 0);
  const int per = (nexp + 255) / 256;
  auto rows_of = [&](int e, int& r0, int& n) {
    if (e < E) {
      r0 = min(max(offsets[e], 0), P);
      n = min(max(counts[e], 0), P - r0);
    } else {
      r0 = P;
      n = T;
    }
  };
  if (T <= kSizeOrderMaxTokens) {
    // Short chunks: items ordered by size class (M tiles: 4, 3, 2, 1), each
    // class in expert order; the GEMM kernels deal them to the XCDs round
    // robin, so every XCD gets the same mix of long and short items and
    // starts with the long ones.  Per-thread counts of the four classes are
    // scanned together, 16 bits each (every total is below 2^16 here).
    auto cls = [](int rows) { return 4 - (rows + 15) / 16; };   // 0 = four M tiles
    uint64_t local = 0;
    for (int q = 0; q < per; ++q) {
      const int e = threadIdx.x * per + q;
      if (e < nexp) {
        int r0, n;
        rows_of(e, r0, n);
        if (n > 0) {
          const int full = (n - 1) / kGroupRows;                       // 64-row items before the last
          local += static_cast<uint64_t>(full);
          local += 1ull << (16 * cls(n - full * kGroupRows));
        }
      }
    }
    s_scan64[threadIdx.x] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const uint64_t v = threadIdx.x >= o ? s_scan64[threadIdx.x - o] : 0ull;
      __syncthreads();
      s_scan64[threadIdx.x] += v;
      __syncthreads();
    }
    const uint64_t tot = s_scan64[255];
    const uint64_t excl = s_scan64[threadIdx.x] - local;
    int pos[4];
    int base = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pos[c] = base + static_cast<int>((excl >> (16 * c)) & 0xFFFFu);
      base += static_cast<int>((tot >> (16 * c)) & 0xFFFFu);
    }
    for (int q = 0; q < per; ++q) {
      const int e = threadIdx.x * per + q;
      if (e < nexp) {
        int r0, n;
        rows_of(e, r0, n);
        const int slot = n > 0 ? item_slot(L, e) : 0;
        for (int g = 0; g * kGroupRows < n; ++g) {
          const int rows = min(kGroupRows, n - g * kGroupRows);
          const int at = pos[cls(rows)]++;
          if (at < item_cap) ws.items[at] = make_int4(e, r0 + g * kGroupRows, rows, slot);
        }
      }
    }
    if (threadIdx.x == 255) {
      ws.hdr[0] = min(base, item_cap);
      ws.hdr[1] = 1;
    }
    return;
  }
  // Long chunks: items in expert order; the GEMM kernels give each XCD one
  // contiguous range of units, so an expert's items share an L2.
  int local = 0;
  for (int q = 0; q < per; ++q) {
    const int e = threadIdx.x * per + q;
    if (e < nexp) {
      int r0, n;
      rows_of(e, r0, n);
      local += (n + kGroupRows - 1) / kGroupRows;
    }
  }
  s_scan[threadIdx.x] = local;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = threadIdx.x >= o ? s_scan[threadIdx.x - o] : 0;
    __syncthreads();
    s_scan[threadIdx.x] += v;
    __syncthreads();
  }
  int pos = s_scan[threadIdx.x] - local;
  for (int q = 0; q < per; ++q) {
    const int e = threadIdx.x * per + q;
    if (e < nexp) {
      int r0, n;
      rows_of(e, r0, n);
      const int slot = n > 0 ? item_slot(L, e) : 0;
      for (int g = 0; g * kGroupRows < n && pos < item_cap; ++g)
        ws.items[pos++] = make_int4(e, r0 + g * kGroupRows, min(kGroupRows, n - g * kGroupRows), slot);
    }
  }
  if (threadIdx.x == 255) {
    ws.hdr[0] = min(s_scan[255], item_cap);
    ws.hdr[1] = 0;
  }
}

// A tile staging, fragment-major: the MFMA A fragment of (block j, M tile
// mt) -- 64 lanes x 8 halves, lane = m + 16 g holding row 16 mt + m, columns
// 32 j + 8 g .. + 7 of the K tile -- is stored as 1 KB of consecutive 16-byte
// slots at ((4 j + mt) * 64 + lane) * 16 bytes.  Wave w loads block j = w
// (8 waves = 8 blocks of a 256-column K tile), one 16-byte global load per
// M tile, and stores it to its own slot, so the stores and the fragment reads
// are both conflict-free and need no padding.  The rows are read through a
// buffer resource over the activation array: each lane's byte offsets (one
// per M tile) are fixed for the whole K loop and the K tile is a scalar
// offset; rows at or beyond nrows repeat the last row (their outputs are
// never written).
constexpr int kFragHalves = 64 * 8;                 // one fragment
constexpr int kATileHalves = 8 * 4 * kFragHalves;   // 8 blocks x 4 M tiles = 32 KB

// With 16 waves, wave w loads block j = w % 8 and the M tiles w / 8,
// w / 8 + 2, ... (clamped to the last one: a wave with nothing left repeats
// a fragment, writing the same bytes to the same place).
template <int NMT>
struct ATile {
  static constexpr int NR = kGemmWaves == 16 ? (NMT + 1) / 2 : NMT;   // fragments per wave
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[NR];
  int slot[NR];      // fragment index 4 j + mt
  u32x4 r[2][NR];    // two register sets: a tile is loaded two K steps before it is stored
  // row_byte(i): byte offset of item row i in the resource
  template <typename RowByte>
  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t rsrc, RowByte row_byte, int nrows) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = w & 7, m = lane & 15, g = lane >> 4;
    rs = rsrc;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int mt = kGemmWaves == 16 ? min((w >> 3) + 2 * i, NMT - 1) : i;
      slot[i] = 4 * j + mt;
      off[i] = row_byte(min(mt * 16 + m, nrows - 1)) + 2u * static_cast<uint32_t>(32 * j + 8 * g);
    }
  }
  template <int SET>
  __device__ __forceinline__ void load(int kt) {
    const uint32_t k0 = static_cast<uint32_t>(kt) * (2 * kTileCols);
#pragma unroll
    for (int i = 0; i < NR; ++i)
      r[SET][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], k0, 0);
  }
  template <int SET>
  __device__ __forceinline__ void store(_Float16* buf, int /*kt*/) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      *reinterpret_cast<u32x4*>(buf + (slot[i] * 64 + lane) * 8) = r[SET][i];
  }
};

__device__ __forceinline__ f16x8 a_frag(const _Float16* buf, int j, int mt, int lane) {
  return *reinterpret_cast<const f16x8*>(buf + ((4 * j + mt) * 64 + lane) * 8);
}

// A tile staging of the down GEMM: the item's h rows, laid out as ATile,
// but each fragment (8 values of one row inside one 16-row tile of I) is
// rescaled from its tile's exponent to the row's exponent E_row on its way
// into LDS, so every MFMA row shares one scale.  The exponents come from the
// item's table in LDS, tile-major (s_hx[tile * 64 + row]), so that each
// lane's lookups are one base address plus compile-time offsets; s_erow
// holds E_row.  Rows at or beyond nrows hold stale exponents: their MFMA
// rows are never stored.
template <int NMT>
struct HTile {
  static constexpr int NR = NMT;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off0;     // byte offset of this lane's fragment in row m; row i*16 + m adds i*16 rows
  uint32_t row_bytes;
  int last;          // the last row: rows at or beyond nrows repeat it
  u32x4 r[2][NR];
  const int8_t* s_hx;
  const int* s_erow;
  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t hrsrc, uint32_t row_bytes_, int nrows,
                                       const int8_t* hx, const int* erow) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = w & 7, m = lane & 15, g = lane >> 4;
    rs = hrsrc;
    row_bytes = row_bytes_;
    last = nrows - 1;
    off0 = 2u * static_cast<uint32_t>(32 * j + 8 * g);
    s_hx = hx + (2 * j + (g >> 1)) * kGroupRows + m;     // tile 2j + g/2 of K tile 0, row m
    s_erow = erow + m;
  }
  template <int SET>
  __device__ __forceinline__ void load(int kt) {
    const int m = threadIdx.x & 15;
    const uint32_t k0 = static_cast<uint32_t>(kt) * (2 * kTileCols);
#pragma unroll
    for (int i = 0; i < NR; ++i)
      r[SET][i] = __builtin_amdgcn_raw_buffer_load_b128(
          rs, static_cast<uint32_t>(min(i * 16 + m, last)) * row_bytes + off0, k0, 0);
  }
  template <int SET>
  __device__ __forceinline__ void store(_Float16* buf, int kt) const {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = w & 7;
    const int8_t* hx = s_hx + kt * (kTileCols / kTileRows) * kGroupRows;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int d = static_cast<int>(hx[i * 16]) - s_erow[i * 16];
      *reinterpret_cast<f16x8*>(buf + ((4 * j + i) * 64 + lane) * 8) =
          scale_pow2(__builtin_bit_cast(f16x8, r[SET][i]), min(d, 0));
    }
  }
};

// One K tile of the gate/up product for NMT 16-row M tiles and RTW row
// tiles of gate and of up: each activation fragment read from LDS feeds
// 2 * RTW MFMAs.
template <int NMT, int RTW>
__device__ __forceinline__ void gateup_ktile(const u32x4 (&b)[4 * RTW], const _Float16* abuf, int lane,
                                             f32x4 (&acc_g)[RTW][4], f32x4 (&acc_u)[RTW][4]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16x8 bg[RTW], bu[RTW];
#pragma unroll
    for (int q = 0; q < RTW; ++q) {
      bg[q] = tile_block_weights(b[4 * q], b[4 * q + 1], j);
      bu[q] = tile_block_weights(b[4 * q + 2], b[4 * q + 3], j);
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const f16x8 a = a_frag(abuf, j, mt, lane);
#pragma unroll
      for (int q = 0; q < RTW; ++q) {
        acc_g[q][mt] = mfma16(a, bg[q], acc_g[q][mt]);
        acc_u[q][mt] = mfma16(a, bu[q], acc_u[q][mt]);
      }
    }
  }
}

// The K loop shared by both GEMMs.  Tile kt's weights live in register set
// kt % RING, so while one tile is multiplied the next RING - 1 tiles' weights
// are in flight, without register copies (which would force early waits).
// Activation tiles go global -> registers -> LDS (double buffered): tile
// kt + 2 is loaded during step kt (register set kt % 2) and published into
// LDS at the end of step kt + 1, so each load has two steps to arrive.
// Each step: load activation tile kt + 2, multiply tile kt, refill the
// weight set RING tiles ahead (only while such a tile exists), publish
// activation tile kt + 1, barrier.  Full groups of RING steps run in a loop;
// the last one or two groups are unrolled with uniform conditions, so no
// weight load past the last tile is issued.  The caller has published tile 0
// into s_a[0] and loaded tile 1 into activation register set 1.
template <int RING, int NB, typename LoadB, typename ATileT, typename Mul>
__device__ __forceinline__ void k_loop(int KT, u32x4 (&b)[RING][NB], LoadB load_b, ATileT& A,
                                       _Float16 (*s_a)[kATileHalves], Mul mul) {
  static_assert(RING % 2 == 0, "the activation double buffer alternates every step");
  auto step = [&](auto par, u32x4 (&bs)[NB], int kt, bool refill) {
    constexpr int P = decltype(par)::value;          // kt % 2
    A.template load<P>(min(kt + 2, KT - 1));
    __builtin_amdgcn_sched_barrier(0);
    mul(bs, s_a[P]);
    __builtin_amdgcn_sched_barrier(0);
    if (refill) load_b(bs, kt + RING);
    A.template store<P ^ 1>(s_a[P ^ 1], min(kt + 1, KT - 1));
    __syncthreads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int kt = 0;
  for (; kt + 2 * RING <= KT; kt += RING) {
#pragma unroll
    for (int u = 0; u < RING; u += 2) {
      step(P0{}, b[u], kt + u, true);
      step(P1{}, b[u + 1], kt + u + 1, true);
    }
  }
#pragma unroll
  for (int u = 0; u < RING; u += 2) {
    if (kt + u < KT) step(P0{}, b[u], kt + u, kt + u + RING < KT);
    if (kt + u + 1 < KT) step(P1{}, b[u + 1], kt + u + 1, kt + u + 1 + RING < KT);
  }
#pragma unroll
  for (int u = 0; u < RING - 1; u += 2) {
    if (kt + RING + u < KT) step(P0{}, b[u], kt + RING + u, false);
    if (u + 1 < RING - 1 && kt + RING + u + 1 < KT) step(P1{}, b[u + 1], kt + RING + u + 1, false);
  }
}

// The same K loop for a K tile count fixed at compile time, fully unrolled:
// every wait the compiler inserts then counts exactly the loads issued since
// the one it waits for (a runtime loop makes it merge the loop-entry and
// back-edge states conservatively, which drains the weight prefetch once per
// iteration).
template <int KTC, int RING, int NB, typename LoadB, typename ATileT, typename Mul, int... KS>
__device__ __forceinline__ void k_loop_fixed(u32x4 (&b)[RING][NB], LoadB load_b, ATileT& A,
                                             _Float16 (*s_a)[kATileHalves], Mul mul,
                                             std::integer_sequence<int, KS...>) {
  static_assert(RING % 2 == 0, "the activation double buffer alternates every step");
  auto step = [&](auto ktc) {
    constexpr int kt = decltype(ktc)::value;
    constexpr int P = kt & 1;
    if constexpr (kt + 2 < KTC) A.template load<P>(kt + 2);
    __builtin_amdgcn_sched_barrier(0);
    mul(b[kt % RING], s_a[P]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kt + RING < KTC) load_b(b[kt % RING], kt + RING);
    if constexpr (kt + 1 < KTC) {
      A.template store<P ^ 1>(s_a[P ^ 1], kt + 1);
      __syncthreads();
    }
  };
  (step(std::integral_constant<int, KS>{}), ...);
}

// ------------------------------------------------------------------ gate/up --
// Row tiles of gate (and of up) per wave for a chunk of T tokens.
inline int gateup_row_tiles_per_wave(int T) { return T > 2 * kSizeOrderMaxTokens ? 2 : 1; }

// Wave w of row block rb takes the RTW row tiles rt0 .. rt0 + RTW - 1 of
// gate and of up, rt0 = (rb * kGemmWaves + w) * RTW.
template <int NMT, int RING, int KTC, int RTW>
__device__ __forceinline__ void gateup_body(const LayerArgs& L, const PrefillWs& ws, int T, const uint8_t* wb,
                                            int row0, int nrows, int rt0,
                                            _Float16 (*s_a)[kATileHalves], const uint32_t* s_off,
                                            const float* s_w, const float* s_u) {
  const int H = L.H, I = L.I;
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int KT = H / kTileCols;
  const uint32_t mat = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<int64_t>(I) * H * 5 / 16)));
  const __amdgpu_buffer_rsrc_t rs = expert_rsrc(wb, 3 * mat);
  const uint32_t gate = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(rt0)) * KT * kTileBytes;
  const uint32_t tile_row = static_cast<uint32_t>(KT) * kTileBytes;     // one row tile, all K tiles
  auto load_b = [&](u32x4 (&b)[4 * RTW], int kt) {
    const uint32_t o = gate + static_cast<uint32_t>(min(kt, KT - 1)) * kTileBytes;
#pragma unroll
    for (int q = 0; q < RTW; ++q) {
      b[4 * q] = load_codes(rs, o + q * tile_row, lane);
      b[4 * q + 1] = load_scales(rs, o + q * tile_row, lane);
      b[4 * q + 2] = load_codes(rs, o + q * tile_row + mat, lane);
      b[4 * q + 3] = load_scales(rs, o + q * tile_row + mat, lane);
    }
  };
  u32x4 b[RING][4 * RTW];
#pragma unroll
  for (int u = 0; u < RING; ++u) load_b(b[u], u);   // clamped: no tile past the last is read
  ATile<NMT> A;
  A.init(expert_rsrc(reinterpret_cast<const uint8_t*>(ws.x16),
                     static_cast<uint32_t>(T) * static_cast<uint32_t>(H) * 2u),
         [&](int i) { return s_off[i]; }, nrows);
  A.template load<0>(0);
  A.template load<1>(min(1, KT - 1));
  A.template store<0>(s_a[0], 0);
  __syncthreads();

  f32x4 acc_g[RTW][4], acc_u[RTW][4];
#pragma unroll
  for (int q = 0; q < RTW; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) { acc_g[q][i] = f32x4{0.f, 0.f, 0.f, 0.f}; acc_u[q][i] = acc_g[q][i]; }

  auto mul = [&](const u32x4 (&bs)[4 * RTW], const _Float16* abuf) {
    gateup_ktile<NMT, RTW>(bs, abuf, lane, acc_g, acc_u);
  };
  if constexpr (KTC > 0)
    k_loop_fixed<KTC, RING>(b, load_b, A, s_a, mul, std::make_integer_sequence<int, KTC>{});
  else
    k_loop<RING>(KT, b, load_b, A, s_a, mul);

  // h rows of this wave's 16-row tiles of I: one exponent per (row, tile)
  const int RTI = I / kTileRows;
#pragma unroll
  for (int q = 0; q < RTW; ++q) {
    const int rt = rt0 + q;
    const int col = rt * 16 + m;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = mt * 16 + 4 * g + r;            // uniform in each 16-lane row
        const bool ok = rl < nrows;
        const float u = ok ? s_u[rl] : 1.0f;
        const float h = ok ? s_w[rl] * silu(acc_g[q][mt][r] * u) * (acc_u[q][mt][r] * u) : 0.0f;
        const int e = block_exponent(row16_max(fabsf(h)));
        if (ok) {
          ws.h[static_cast<size_t>(row0 + rl) * I + col] = static_cast<_Float16>(ldexpf(h, -e));
          if (m == 0) ws.hexp[static_cast<size_t>(row0 + rl) * RTI + rt] = static_cast<int8_t>(e);
        }
      }
    }
  }
}

// KTC: the number of 256-column K tiles (H / 256) when fixed at compile
// time, 0 for the runtime loop.  RTW: row tiles of gate and of up per wave
// (a block covers 16 * kGemmWaves * RTW rows of I).
template <int KTC, int RTW>
__global__ __launch_bounds__(kThreads) void prefill_gateup_kernel(LayerArgs L, PrefillWs ws, int T) {
  __shared__ __align__(16) _Float16 s_a[2][kATileHalves];
  __shared__ uint32_t s_off[kGroupRows];
  __shared__ float s_w[kGroupRows];
  __shared__ float s_u[kGroupRows];
  const int RB = L.I / (kGateupRowsPerBlock * RTW);
  const int2 wu = work_unit(blockIdx.x, ws.hdr, RB);
  if (wu.x < 0) return;
  const int item = wu.x;
  const int rb = wu.y;
  const int4 it = ws.items[item];
  const uint8_t* wb = expert_base(L, it);
  const int row0 = it.y, nrows = it.z;
  if (threadIdx.x < nrows) {
    const int t = ws.row_tok[row0 + threadIdx.x];
    s_off[threadIdx.x] = static_cast<uint32_t>(t) * static_cast<uint32_t>(L.H) * 2u;   // bytes
    s_w[threadIdx.x] = ws.row_w[row0 + threadIdx.x];
    s_u[threadIdx.x] = ws.unscale[t];
  }
  __syncthreads();
  const int rt0 = (rb * kGemmWaves + static_cast<int>(threadIdx.x >> 6)) * RTW;
  switch ((nrows + 15) / 16) {
    case 1: gateup_body<1, kGateupRing, KTC, RTW>(L, ws, T, wb, row0, nrows, rt0, s_a, s_off, s_w, s_u); break;
    case 2: gateup_body<2, kGateupRing, KTC, RTW>(L, ws, T, wb, row0, nrows, rt0, s_a, s_off, s_w, s_u); break;
    case 3: gateup_body<3, kGateupRing, KTC, RTW>(L, ws, T, wb, row0, nrows, rt0, s_a, s_off, s_w, s_u); break;
    default: gateup_body<4, kGateupRing, KTC, RTW>(L, ws, T, wb, row0, nrows, rt0, s_a, s_off, s_w, s_u); break;
  }
}

// --------------------------------------------------------------------- down --
// Per block: both row tiles' weights dequantized first, then one activation
// fragment at a time (fewer live registers than holding every M tile's
// fragment).
template <int NMT>
__device__ __forceinline__ void down_ktile(const u32x4 (&b)[2 * kDownRTW], const _Float16* abuf, int lane,
                                           f32x4 (&acc)[kDownRTW][4]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f16x8 bq[kDownRTW];
#pragma unroll
    for (int q = 0; q < kDownRTW; ++q) bq[q] = tile_block_weights(b[2 * q], b[2 * q + 1], j);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const f16x8 a = a_frag(abuf, j, mt, lane);
#pragma unroll
      for (int q = 0; q < kDownRTW; ++q) acc[q][mt] = mfma16(a, bq[q], acc[q][mt]);
    }
  }
}

template <int NMT, int RING, int KTC>
__device__ __forceinline__ void down_body(const LayerArgs& L, const PrefillWs& ws, const uint8_t* wb, int row0,
                                          int nrows, int rt0, _Float16 (*s_a)[kATileHalves],
                                          int* s_erow, int8_t* s_hx) {
  const int H = L.H, I = L.I;
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int KT = I / kTileCols;
  const int RTI = I / kTileRows;
  const uint32_t mat = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<int64_t>(I) * H * 5 / 16)));
  const __amdgpu_buffer_rsrc_t rs = expert_rsrc(wb, 3 * mat);
  const uint32_t down = 2 * mat + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(rt0)) * KT * kTileBytes;
  constexpr int NB = 2 * kDownRTW;   // codes and scales of each row tile
  auto load_b = [&](u32x4 (&b)[NB], int kt) {
    const uint32_t o = down + static_cast<uint32_t>(min(kt, KT - 1)) * kTileBytes;
#pragma unroll
    for (int q = 0; q < kDownRTW; ++q) {
      b[2 * q] = load_codes(rs, o + q * KT * kTileBytes, lane);
      b[2 * q + 1] = load_scales(rs, o + q * KT * kTileBytes, lane);
    }
  };
  // the item's tile exponents are requested first: they are waited for
  // first, and loads complete in issue order (RTI / 16 = KT vectors per row)
  constexpr int kEPre = 4;
  const u32x4* ev_src = reinterpret_cast<const u32x4*>(
      ws.hexp + static_cast<size_t>(row0 + min(static_cast<int>(threadIdx.x), nrows - 1)) * RTI);
  u32x4 ev[kEPre];
#pragma unroll
  for (int q = 0; q < kEPre; ++q) ev[q] = ev_src[min(q, KT - 1)];
  u32x4 b[RING][NB];
#pragma unroll
  for (int u = 0; u < RING; ++u) load_b(b[u], u);
  HTile<NMT> A;   // the item's h rows are consecutive: a resource over just them
  const uint32_t row_bytes = static_cast<uint32_t>(I) * 2u;
  A.init(expert_rsrc(reinterpret_cast<const uint8_t*>(ws.h + static_cast<size_t>(row0) * I),
                     static_cast<uint32_t>(nrows) * row_bytes),
         row_bytes, nrows, s_hx, s_erow);
  A.template load<0>(0);
  A.template load<1>(min(1, KT - 1));
  // the item's tile exponents into LDS, tile-major (its rows are consecutive
  // in hexp, RTI a multiple of 16), and E_row, the largest exponent of each row
  if (static_cast<int>(threadIdx.x) < nrows) {
    const int row = threadIdx.x;
    int mx = kZeroExp;
    auto take = [&](int q, const u32x4& wv) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ex = static_cast<int8_t>(wv[c] >> (8 * s));
          s_hx[(16 * q + 4 * c + s) * kGroupRows + row] = static_cast<int8_t>(ex);
          mx = max(mx, ex);
        }
    };
#pragma unroll
    for (int q = 0; q < kEPre; ++q)
      if (q < KT) take(q, ev[q]);
    for (int q = kEPre; q < KT; ++q) take(q, ev_src[q]);
    s_erow[row] = mx;
  }
  __syncthreads();
  A.template store<0>(s_a[0], 0);
  __syncthreads();

  f32x4 acc[kDownRTW][4];
#pragma unroll
  for (int q = 0; q < kDownRTW; ++q)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mul = [&](const u32x4 (&bs)[NB], const _Float16* abuf) {
    down_ktile<NMT>(bs, abuf, lane, acc);
  };
  if constexpr (KTC > 0)
    k_loop_fixed<KTC, RING>(b, load_b, A, s_a, mul, std::make_integer_sequence<int, KTC>{});
  else
    k_loop<RING>(KT, b, load_b, A, s_a, mul);

  // y = acc * 2^E_row, one exponent per (row, 8 columns).  The wave's
  // accumulators (its rows x 32 columns, fp32) go through its own 8 KB of
  // the A tile buffer (free after the K loop) so that a lane then holds 8
  // consecutive columns of one row: the block maximum needs no cross-lane
  // step and the store is one 16-byte write.  Rows are 32 floats; the 8-float
  // chunks of row r sit at chunk ^ ((r >> 2) & 3), which spreads the four
  // lane groups of an accumulator write over all 32 chunk positions.
  static_assert(kDownRTW == 2 && 8 * kGroupRows * 32 * 4 == sizeof(_Float16) * 2 * kATileHalves,
                "one wave's rows x 32 fp32 columns fill an eighth of the A tile buffer");
  __syncthreads();                                   // every wave is done with the A tiles
  float* tb = reinterpret_cast<float*>(&s_a[0][0]) + (threadIdx.x >> 6) * (kGroupRows * 32);
  auto at = [](int row, int col) { return row * 32 + ((((col >> 3) ^ (row >> 2)) & 3) << 3) + (col & 7); };
#pragma unroll
  for (int q = 0; q < kDownRTW; ++q)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tb[at(mt * 16 + 4 * g + r, q * 16 + m)] = acc[q][mt][r];
  __builtin_amdgcn_wave_barrier();
  const int NYG = H / kYGroup;
#pragma unroll
  for (int it = 0; it < NMT; ++it) {                 // 16 rows x 4 chunks per step
    const int rl = it * 16 + (lane >> 2), ch = lane & 3;
    if (rl < nrows) {
      const f32x4* src4 = reinterpret_cast<const f32x4*>(tb + at(rl, 8 * ch));
      const f32x4 lo = src4[0], hi = src4[1];
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fmaxf(fabsf(lo[i]), fabsf(hi[i])));
      // y = acc * 2^E_row = y~ * 2^F, F = exponent of the chunk's largest |y|
      const int er = s_erow[rl];
      const int f = block_exponent(mx);
      const int F = f == kZeroExp ? kZeroExp : max(-126, min(127, f + er));
      f16x8 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = static_cast<_Float16>(ldexpf(lo[i], er - F));
        o[4 + i] = static_cast<_Float16>(ldexpf(hi[i], er - F));
      }
      const int col = rt0 * 16 + ch * 8;
      *reinterpret_cast<f16x8*>(ws.y + static_cast<size_t>(row0 + rl) * H + col) = o;
      ws.yexp[static_cast<size_t>(row0 + rl) * NYG + col / kYGroup] = static_cast<int8_t>(F);
    }
  }
}

template <int KTC>   // I / 256 when fixed at compile time, else 0
__global__ __launch_bounds__(kThreads) void prefill_down_kernel(LayerArgs L, PrefillWs ws) {
  __shared__ __align__(16) _Float16 s_a[2][kATileHalves];
  __shared__ int s_erow[kGroupRows];
  extern __shared__ __align__(16) int8_t s_hx[];     // [kGroupRows][I/16] tile exponents
  const int RB = L.H / kDownRowsPerBlock;
  const int2 wu = work_unit(blockIdx.x, ws.hdr, RB);
  if (wu.x < 0) return;
  const int item = wu.x;
  const int rb = wu.y;
  const int4 it = ws.items[item];
  const uint8_t* wb = expert_base(L, it);
  const int row0 = it.y, nrows = it.z;
  const int rt0 = (rb * kGemmWaves + static_cast<int>(threadIdx.x >> 6)) * kDownRTW;
  switch ((nrows + 15) / 16) {
    case 1: down_body<1, kDownRing, KTC>(L, ws, wb, row0, nrows, rt0, s_a, s_erow, s_hx); break;
    case 2: down_body<2, kDownRing, KTC>(L, ws, wb, row0, nrows, rt0, s_a, s_erow, s_hx); break;
    case 3: down_body<3, kDownRing, KTC>(L, ws, wb, row0, nrows, rt0, s_a, s_erow, s_hx); break;
    default: down_body<4, kDownRing, KTC>(L, ws, wb, row0, nrows, rt0, s_a, s_erow, s_hx); break;
  }
}

// --------------------------------------------------------- down, A resident --
// For I <= 768 (at most three 256-column K tiles of h): the block stages its
// item's h rows, rescaled to the row exponents, into LDS once and then runs
// NCB chunks of 256 output rows of H one after the other (wave w: the two
// 16-row tiles 2 (8 c + w) and 2 (8 c + w) + 1 of chunk c).  With A resident
// the chunk loop needs no block barrier: a wave issues the weight loads of
// chunk i + 2 as soon as chunk i's registers are free, and its epilogue goes
// through a transposition buffer of its own.  So one staging of A, and one
// exponent table, serve NCB times the work of the per-chunk kernel above.
constexpr int kDownResMaxKT = 3;
constexpr int kDownChunkRows = 16 * kDownRTW * kGemmWaves;   // 256
static_assert(kDownRTW == 2, "two row tiles per wave and chunk");

// f(integral_constant<int, i>) for i = IS... in order.
template <typename F, int... IS>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, IS...>) {
  (f(std::integral_constant<int, IS>{}), ...);
}

// Row r, column c (0..15) of a wave's 64 x 16 fp32 transposition buffer:
// the two 8-float halves of a row swap places every four rows, which spreads
// an accumulator write (rows 4g + r of 16 columns) over both halves.
__device__ __forceinline__ int res_at(int row, int col) {
  return row * 16 + ((((col >> 3) ^ (row >> 2)) & 1) << 3) + (col & 7);
}

// MT: M tiles the LDS holds (4, or 2 for half items); PF: chunks of weights
// in flight per wave (2: the next-but-one chunk is requested as soon as a
// chunk's registers are free; 1: the next chunk, fewer registers).
template <int NMT, int KT, int NCB, int MT, int PF>
__device__ __forceinline__ void down_res_body(const LayerArgs& L, const PrefillWs& ws, const uint8_t* wb,
                                              int row0, int nrows, int c0, _Float16* s_a,
                                              float* s_t, int* s_erow, int8_t* s_hx) {
  static_assert(NMT <= MT, "an item part fits the LDS tiles");
  constexpr int AH = 8 * MT * kFragHalves;        // halves of one K tile of A
  constexpr int MR = MT * 16;                     // rows of the exponent table and the buffer
  const int H = L.H, I = L.I;                     // I == 256 * KT
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  constexpr int RTI = KT * (kTileCols / kTileRows);
  const uint32_t mat = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<int64_t>(I) * H * 5 / 16)));
  const __amdgpu_buffer_rsrc_t rs = expert_rsrc(wb, 3 * mat);
  constexpr int NB = 2 * kDownRTW * KT;           // codes and scales of the wave's tiles, all K tiles
  // the wave's two row tiles are consecutive, and so are their K tiles
  auto load_chunk = [&](u32x4 (&b)[NB], int c) {
    const uint32_t o = 2 * mat + static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
                                     (c * kGemmWaves + w) * kDownRTW)) * KT * kTileBytes;
#pragma unroll
    for (int t = 0; t < kDownRTW * KT; ++t) {
      b[2 * t] = load_codes(rs, o + t * kTileBytes, lane);
      b[2 * t + 1] = load_scales(rs, o + t * kTileBytes, lane);
    }
  };
  // requests in the order they are waited for: the item's tile exponents,
  // the first PF chunks' weights, the h fragments
  const u32x4* ev_src = reinterpret_cast<const u32x4*>(
      ws.hexp + static_cast<size_t>(row0 + min(static_cast<int>(threadIdx.x), nrows - 1)) * RTI);
  u32x4 ev[KT];
#pragma unroll
  for (int q = 0; q < KT; ++q) ev[q] = ev_src[q];
  u32x4 b[PF][NB];
  load_chunk(b[0], c0);
  if constexpr (PF > 1 && NCB > 1) load_chunk(b[1], c0 + 1);
  const uint32_t row_bytes = static_cast<uint32_t>(I) * 2u;
  const __amdgpu_buffer_rsrc_t hr = expert_rsrc(reinterpret_cast<const uint8_t*>(ws.h + static_cast<size_t>(row0) * I),
                                                static_cast<uint32_t>(nrows) * row_bytes);
  u32x4 ar[KT][NMT];           // fragment (kt, block j = w, M tile mt) of the item's h rows
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      ar[kt][mt] = __builtin_amdgcn_raw_buffer_load_b128(
          hr, static_cast<uint32_t>(min(mt * 16 + m, nrows - 1)) * row_bytes + 2u * static_cast<uint32_t>(32 * w + 8 * g),
          static_cast<uint32_t>(kt) * (2 * kTileCols), 0);
  // the tile exponents into LDS, tile-major, and E_row, each row's largest
  if (static_cast<int>(threadIdx.x) < nrows) {
    const int row = threadIdx.x;
    int mx = kZeroExp;
#pragma unroll
    for (int q = 0; q < KT; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          const int ex = static_cast<int8_t>(ev[q][c] >> (8 * sb));
          s_hx[(16 * q + 4 * c + sb) * MR + row] = static_cast<int8_t>(ex);
          mx = max(mx, ex);
        }
    s_erow[row] = mx;
  }
  __syncthreads();
  // every fragment rescaled from its tile's exponent to its row's; rows at or
  // beyond nrows repeat the last row with stale exponents and are never stored
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int d = static_cast<int>(s_hx[(kt * 16 + 2 * w + (g >> 1)) * MR + mt * 16 + m]) -
                    s_erow[mt * 16 + m];
      *reinterpret_cast<f16x8*>(&s_a[kt * AH + ((MT * w + mt) * 64 + lane) * 8]) =
          scale_pow2(__builtin_bit_cast(f16x8, ar[kt][mt]), min(d, 0));
    }
  __syncthreads();

  float* tb = s_t + w * (MR * 16);
  const int NYG = H / kYGroup;
  auto chunk = [&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const u32x4 (&bs)[NB] = b[i % PF];
    f32x4 acc[kDownRTW][4];
#pragma unroll
    for (int q = 0; q < kDownRTW; ++q)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f16x8 bq[kDownRTW];
#pragma unroll
        for (int q = 0; q < kDownRTW; ++q) bq[q] = tile_block_weights(bs[2 * (q * KT + kt)], bs[2 * (q * KT + kt) + 1], j);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(s_a + kt * AH + ((MT * j + mt) * 64 + lane) * 8);
#pragma unroll
          for (int q = 0; q < kDownRTW; ++q) acc[q][mt] = mfma16(a, bq[q], acc[q][mt]);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (i + PF < NCB) load_chunk(b[i % PF], c0 + i + PF);
    __builtin_amdgcn_sched_barrier(0);
    // y = acc * 2^E_row, one exponent per (row, 8 columns), one row tile at
    // a time through the wave's buffer: a lane then holds 8 consecutive
    // columns of one row
    const int rt0 = ((c0 + i) * kGemmWaves + w) * kDownRTW;
#pragma unroll
    for (int q = 0; q < kDownRTW; ++q) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tb[res_at(mt * 16 + 4 * g + r, m)] = acc[q][mt][r];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int st = 0; st < (NMT * 16 + 31) / 32; ++st) {      // 32 rows x 2 halves per step
        const int rl = st * 32 + (lane >> 1), ch = lane & 1;
        if (rl < nrows && rl < NMT * 16) {
          const f32x4* src4 = reinterpret_cast<const f32x4*>(tb + res_at(rl, 8 * ch));
          const f32x4 lo = src4[0], hi = src4[1];
          float mx = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(lo[e]), fabsf(hi[e])));
          const int er = s_erow[rl];
          const int f = block_exponent(mx);
          const int F = f == kZeroExp ? kZeroExp : max(-126, min(127, f + er));
          f16x8 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = static_cast<_Float16>(ldexpf(lo[e], er - F));
            o[4 + e] = static_cast<_Float16>(ldexpf(hi[e], er - F));
          }
          const int col = (rt0 + q) * 16 + ch * 8;
          *reinterpret_cast<f16x8*>(ws.y + static_cast<size_t>(row0 + rl) * H + col) = o;
          ws.yexp[static_cast<size_t>(row0 + rl) * NYG + col / kYGroup] = static_cast<int8_t>(F);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  };
  for_each_index(chunk, std::make_integer_sequence<int, NCB>{});
}

// HALVES = 2: a work unit takes 32 rows of an item (MT = 2), so the
// resident h tiles take half the LDS and two workgroups fit on a CU.
template <int KT, int NCB, int MT, int PF, int HALVES>
__global__ __launch_bounds__(kThreads) void prefill_down_res_kernel(LayerArgs L, PrefillWs ws) {
  static_assert(MT * 16 * HALVES == kGroupRows, "the parts of an item cover its rows");
  __shared__ __align__(16) _Float16 s_a[KT * 8 * MT * kFragHalves];
  __shared__ __align__(16) float s_t[kGemmWaves * MT * 16 * 16];
  __shared__ int8_t s_hx[MT * 16 * KT * (kTileCols / kTileRows)];
  __shared__ int s_erow[MT * 16];
  const int RB = L.H / (kDownChunkRows * NCB);
  const int2 wu = work_unit(blockIdx.x, ws.hdr, RB * HALVES);
  if (wu.x < 0) return;
  const int4 it = ws.items[wu.x];
  const int part = wu.y / RB;
  const int row0 = it.y + part * MT * 16;
  const int nrows = min(it.z - part * MT * 16, MT * 16);
  if (nrows <= 0) return;
  const uint8_t* wb = expert_base(L, it);
  const int c0 = (wu.y % RB) * NCB;
  switch ((nrows + 15) / 16) {
    case 1: down_res_body<1, KT, NCB, MT, PF>(L, ws, wb, row0, nrows, c0, s_a, s_t, s_erow, s_hx); break;
    case 2: down_res_body<2, KT, NCB, MT, PF>(L, ws, wb, row0, nrows, c0, s_a, s_t, s_erow, s_hx); break;
    case 3:
      if constexpr (MT >= 3) down_res_body<3, KT, NCB, MT, PF>(L, ws, wb, row0, nrows, c0, s_a, s_t, s_erow, s_hx);
      break;
    default:
      if constexpr (MT >= 4) down_res_body<4, KT, NCB, MT, PF>(L, ws, wb, row0, nrows, c0, s_a, s_t, s_erow, s_hx);
      break;
  }
}

// ------------------------------------------------------------------ combine --
// One thread per (token, 8-column chunk): the token's k rows of y~ (and the
// shared row) are all requested before the first is summed, in 16-byte loads,
// with each row's exponent for these columns; the sum runs over j ascending,
// then the shared row, in fp32.
__global__ __launch_bounds__(256) void prefill_combine_kernel(
    int T, int H, int k, int has_shared, const int32_t* __restrict__ pair_pos,
    const void* residual, void* out, int out_bf16, PrefillWs ws) {   // residual may alias out
  const int nch = H >> 3;
  const long long g = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= static_cast<long long>(T) * nch) return;
  const int t = static_cast<int>(g / nch);
  const int c = static_cast<int>(g - static_cast<long long>(t) * nch);
  const int P = T * k;
  const int NYG = H / kYGroup;
  const int yg = c;                                   // one exponent per 8-column chunk
  int pos[MOE_MAX_TOPK + 1];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    pos[j] = j < k ? min(max(pair_pos[static_cast<size_t>(t) * k + j], 0), P - 1) : 0;
  pos[MOE_MAX_TOPK] = P + t;
  f16x8 v[MOE_MAX_TOPK + 1];
  int f[MOE_MAX_TOPK + 1];
#pragma unroll
  for (int j = 0; j <= MOE_MAX_TOPK; ++j) {
    if (j < k || (j == MOE_MAX_TOPK && has_shared)) {
      v[j] = *reinterpret_cast<const f16x8*>(ws.y + static_cast<size_t>(pos[j]) * H + 8 * c);
      f[j] = ws.yexp[static_cast<size_t>(pos[j]) * NYG + yg];
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j <= MOE_MAX_TOPK; ++j) {
    if (j < k || (j == MOE_MAX_TOPK && has_shared)) {
      const float sc = ldexpf(1.0f, f[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += static_cast<float>(v[j][i]) * sc;
    }
  }
  const size_t o = static_cast<size_t>(t) * H + 8 * c;
  if (out_bf16) {
    u32x4 rs = {0u, 0u, 0u, 0u}, w;
    if (residual) rs = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(residual) + o);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo = acc[2 * q], hi = acc[2 * q + 1];
      if (residual) {
        lo += __uint_as_float(rs[q] << 16);
        hi += __uint_as_float(rs[q] & 0xFFFF0000u);
      }
      w[q] = static_cast<uint32_t>(float_to_bf16(lo)) | (static_cast<uint32_t>(float_to_bf16(hi)) << 16);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o) = w;
  } else {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = acc[i]; b[i] = acc[4 + i]; }
    if (residual) {
      const f32x4* rp = reinterpret_cast<const f32x4*>(static_cast<const float*>(residual) + o);
      a += rp[0];
      b += rp[1];
    }
    f32x4* op = reinterpret_cast<f32x4*>(static_cast<float*>(out) + o);
    op[0] = a;
    op[1] = b;
  }
}

}  // namespace

size_t prefill_workspace_bytes(int T, int E, int k, int H, int I) {
  const size_t rows = static_cast<size_t>(T) * k + T;
  return 256 + align256(sizeof(int4) * max_items(T, E, k)) + align256(sizeof(float) * T) +
         align256(sizeof(int32_t) * rows) + align256(sizeof(float) * rows) +
         align256(sizeof(_Float16) * static_cast<size_t>(T) * H) + align256(sizeof(_Float16) * rows * I) +
         align256(sizeof(_Float16) * rows * H) + align256(rows * (I / kTileRows)) +
         align256(rows * (H / kYGroup));
}

hipError_t launch_prefill(const LayerArgs& L, const void* x, int x_bf16, int T,
                          const int32_t* ids, const float* w, int k, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pairs,
                          const int32_t* pair_pos, const void* residual, void* out,
                          int out_bf16, int prenorm, void* wsp, hipStream_t s) {
  (void)ids;
  const PrefillWs ws = carve(wsp, T, L.E, k, L.H, L.I);
  const int nitems = max_items(T, L.E, k);   // capacity of the item list
  const long long rows = static_cast<long long>(T) * k + T;
  // the GEMM grids cover at most one item per row (every item has a row):
  // far fewer than the list capacity for short chunks
  const int grid_items = static_cast<int>(std::min<long long>(nitems, rows));
  hipError_t e;
  {
    const int grid = (T + kPrepTokensPerBlock - 1) / kPrepTokensPerBlock + 1 + static_cast<int>((rows + 255) / 256);
    // chunks of 8 elements per lane: H / 512, rounded up to a kernel variant
    const int ncl = (L.H / 8 + 63) / 64;
    auto prep = [&](auto xbf16, auto n) {
      return launch_kernel(K_PREFILL_PREP, prefill_prep_kernel<decltype(xbf16)::value, decltype(n)::value>,
                           dim3(grid), dim3(256), 0, s, L, x, T, k, prenorm, counts, offsets, sorted_pairs,
                           w, nitems, ws);
    };
    using B1 = std::true_type;
    using B0 = std::false_type;
    using N2 = std::integral_constant<int, 2>;
    using N6 = std::integral_constant<int, 6>;
    using N16 = std::integral_constant<int, MOE_MAX_DIM / 512>;
    if (ncl <= 2) e = x_bf16 ? prep(B1{}, N2{}) : prep(B0{}, N2{});
    else if (ncl <= 6) e = x_bf16 ? prep(B1{}, N6{}) : prep(B0{}, N6{});
    else e = x_bf16 ? prep(B1{}, N16{}) : prep(B0{}, N16{});
  }
  if (e != hipSuccess) return e;
  {
    // long chunks (full 64-row items): two row tiles per wave, so each
    // activation fragment read from LDS feeds four MFMAs; I is a multiple of
    // 256, so the wider row block divides it
    const int rtw = gateup_row_tiles_per_wave(T);
    const long long nb = (static_cast<long long>(grid_items) + 7) / 8 * 8 * (L.I / (kGateupRowsPerBlock * rtw));
    const int grid = static_cast<int>(nb);
    const dim3 g(grid), b(kThreads);
    auto gu = [&](auto ktc, auto rtwc) {
      return launch_kernel(K_PREFILL_GATEUP,
                           prefill_gateup_kernel<decltype(ktc)::value, decltype(rtwc)::value>, g, b, 0, s, L,
                           ws, T);
    };
    auto by_width = [&](auto rtwc) {
      switch (L.H / kTileCols) {   // fully unrolled K loops for the common widths
        case 4: return gu(std::integral_constant<int, 4>{}, rtwc);
        case 8: return gu(std::integral_constant<int, 8>{}, rtwc);
        case 12: return gu(std::integral_constant<int, 12>{}, rtwc);
        case 16: return gu(std::integral_constant<int, 16>{}, rtwc);
        default: return gu(std::integral_constant<int, 0>{}, rtwc);
      }
    };
    e = rtw == 2 ? by_width(std::integral_constant<int, 2>{}) : by_width(std::integral_constant<int, 1>{});
  }
  if (e != hipSuccess) return e;
  const int ktd = L.I / kTileCols;
  const int nc = L.H / kDownChunkRows;
  if (ktd <= kDownResMaxKT) {
    // A resident: chunks per block, 3 where they divide H / 256 (then 2, 1).
    // Chunks up to kSizeOrderMaxTokens (mostly short items): half items, two
    // workgroups per CU
    const int ncb = nc % 3 == 0 ? 3 : (nc % 2 == 0 ? 2 : 1);
    const bool halves = T <= kSizeOrderMaxTokens;
    const long long nb = (static_cast<long long>(grid_items) + 7) / 8 * 8 * (nc / ncb) * (halves ? 2 : 1);
    const dim3 g(static_cast<int>(nb)), b(kThreads);
    auto dr = [&](auto ktc, auto ncbc) {
      constexpr int KTv = decltype(ktc)::value, NCBv = decltype(ncbc)::value;
      return halves ? launch_kernel(K_PREFILL_DOWN, prefill_down_res_kernel<KTv, NCBv, 2, 1, 2>, g, b, 0, s, L, ws)
                    : launch_kernel(K_PREFILL_DOWN, prefill_down_res_kernel<KTv, NCBv, 4, 2, 1>, g, b, 0, s, L, ws);
    };
    auto by_ncb = [&](auto ktc) {
      if (ncb == 3) return dr(ktc, std::integral_constant<int, 3>{});
      if (ncb == 2) return dr(ktc, std::integral_constant<int, 2>{});
      return dr(ktc, std::integral_constant<int, 1>{});
    };
    if (ktd == 1) e = by_ncb(std::integral_constant<int, 1>{});
    else if (ktd == 2) e = by_ncb(std::integral_constant<int, 2>{});
    else e = by_ncb(std::integral_constant<int, 3>{});
  } else {
    const long long nb = (static_cast<long long>(grid_items) + 7) / 8 * 8 * (L.H / kDownRowsPerBlock);
    const int grid = static_cast<int>(nb);
    const dim3 g(grid), b(kThreads);
    const uint32_t lds = static_cast<uint32_t>(kGroupRows * (L.I / kTileRows));   // tile-exponent table
    switch (L.I / kTileCols) {
      case 1: e = launch_kernel(K_PREFILL_DOWN, prefill_down_kernel<1>, g, b, lds, s, L, ws); break;
      case 2: e = launch_kernel(K_PREFILL_DOWN, prefill_down_kernel<2>, g, b, lds, s, L, ws); break;
      case 3: e = launch_kernel(K_PREFILL_DOWN, prefill_down_kernel<3>, g, b, lds, s, L, ws); break;
      case 4: e = launch_kernel(K_PREFILL_DOWN, prefill_down_kernel<4>, g, b, lds, s, L, ws); break;
      default: e = launch_kernel(K_PREFILL_DOWN, prefill_down_kernel<0>, g, b, lds, s, L, ws); break;
    }
  }
  if (e != hipSuccess) return e;
  const long long nthr = static_cast<long long>(T) * (L.H / 8);
  return launch_kernel(K_PREFILL_COMBINE, prefill_combine_kernel, dim3(static_cast<int>((nthr + 255) / 256)),
                       dim3(256), 0, s, T,
                       L.H, k, L.shared ? 1 : 0, pair_pos, residual, out, out_bf16, ws);
}

}  // namespace moeq2
