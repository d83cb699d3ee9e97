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
//            two s_t (max |x_hat s_t| in [0.5, 1)), stored fp16 [T][H]; the
//            last workgroup turns `counts` into the work-item list.
//   gateup   work item x 64-row block of I: A = the item's gathered x rows
//            (fp16, staged in LDS, double buffered per 256-column K tile), B =
//            the expert's gate and up tiles dequantized in registers (each
//            weight is dequantized once per item and used by every M tile),
//            v_mfma_f32_16x16x32_f16, SwiGLU epilogue:
//            h~[row] = w * silu(g) * u * s_t^2  (fp16, sorted-row order).
//   down     work item x 256-row block of H: A = h~ rows (LDS), B = down
//            tiles; y~[row] = W_down h~ (fp16).
//   combine  token t: out = (sum_j y~[pair_pos[t,j]] + y~[shared row]) / s_t^2
//            (+ residual), j ascending: fixed order, no atomics.
// Workgroup ids are remapped so that consecutive logical ids (the row blocks
// of one work item, which read the same A rows) run on the same XCD and
// share its L2.
#include "launch.h"
#include "q2_device.h"
#include "../../include/moe_q2.h"

namespace moeq2 {

namespace {

constexpr int kLdsStride = kTileCols + 8;   // halves per LDS row (pad: no bank conflicts)
constexpr int kGateupRowsPerBlock = 64;     // 4 waves x 16 rows of I (gate and up)
constexpr int kDownRowsPerBlock = 256;      // 4 waves x 4 x 16 rows of H

struct PrefillWs {
  int32_t* hdr;        // [0] = number of work items
  int4* items;         // {expert, row0, nrows, 0}
  float* unscale;      // [T]  1 / s_t
  _Float16* x16;       // [T][H]
  _Float16* h;         // [rows][I]
  _Float16* y;         // [rows][H]
};

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
  w.x16 = reinterpret_cast<_Float16*>(p); p += align256(sizeof(_Float16) * static_cast<size_t>(T) * H);
  w.h = reinterpret_cast<_Float16*>(p); p += align256(sizeof(_Float16) * rows * I);
  w.y = reinterpret_cast<_Float16*>(p);
  return w;
}

__device__ __forceinline__ int xcd_logical(int bid, int nblocks) {
  const int per = nblocks / 8;
  return (bid % 8) * per + bid / 8;
}

__device__ __forceinline__ const uint8_t* expert_base(const LayerArgs& L, int e) {
  return e >= L.E ? L.shared : L.experts + static_cast<int64_t>(e) * L.stride;
}

// --------------------------------------------------------------------- prep --
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    LayerArgs L, const void* __restrict__ x, int x_bf16, int T, int k, int prenorm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int item_cap,
    PrefillWs ws) {
  __shared__ float s_a[4], s_b[4];
  __shared__ int s_scan[256];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int H = L.H, E = L.E;
  if (blockIdx.x < T) {
    const int t = blockIdx.x;
    float ss = 0.0f, mx = 0.0f;
    for (int i = threadIdx.x; i < H; i += 256) {
      const size_t o = static_cast<size_t>(t) * H + i;
      const float v = x_bf16 ? bf16_to_float(static_cast<const uint16_t*>(x)[o]) : static_cast<const float*>(x)[o];
      ss += v * v;
      mx = fmaxf(mx, fabsf(v));
    }
    ss = wave_sum(ss);
    mx = wave_max(mx);
    if (lane == 0) { s_a[wid] = ss; s_b[wid] = mx; }
    __syncthreads();
    ss = s_a[0] + s_a[1] + s_a[2] + s_a[3];
    mx = fmaxf(fmaxf(s_b[0], s_b[1]), fmaxf(s_b[2], s_b[3]));
    const float r = prenorm ? 1.0f / sqrtf(ss / static_cast<float>(H) + 1e-6f) : 1.0f;
    const float s = pow2_normaliser(mx * r);
    for (int i = threadIdx.x; i < H; i += 256) {
      const size_t o = static_cast<size_t>(t) * H + i;
      const float v = x_bf16 ? bf16_to_float(static_cast<const uint16_t*>(x)[o]) : static_cast<const float*>(x)[o];
      ws.x16[o] = static_cast<_Float16>((v * r) * s);
    }
    if (threadIdx.x == 0) ws.unscale[t] = 1.0f / s;
    return;
  }
  // ---- last workgroup: work items from the histogram --------------------
  // (rows of expert e: [offsets[e], offsets[e] + counts[e]) clipped to
  // [0, T*k), so inconsistent histogram arrays cannot send any later kernel
  // outside its buffers)
  const int P = T * k;
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
      for (int g = 0; g * kGroupRows < n && pos < item_cap; ++g) {
        ws.items[pos++] = make_int4(e, r0 + g * kGroupRows, min(kGroupRows, n - g * kGroupRows), 0);
      }
    }
  }
  if (threadIdx.x == 255) ws.hdr[0] = min(s_scan[255], item_cap);
}

// ------------------------------------------------------------------ gate/up --
__global__ __launch_bounds__(256) void prefill_gateup_kernel(
    LayerArgs L, int T, int k, const int32_t* __restrict__ sorted_pairs,
    const float* __restrict__ topk_w, PrefillWs ws) {
  __shared__ __align__(16) _Float16 s_a[2][kGroupRows * kLdsStride];
  __shared__ int s_tok[kGroupRows];
  __shared__ float s_w[kGroupRows];
  __shared__ float s_u[kGroupRows];
  const int H = L.H, I = L.I, E = L.E;
  const int RB = I / kGateupRowsPerBlock;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int item = logical / RB;
  const int rb = logical % RB;
  if (item >= ws.hdr[0]) return;
  const int4 it = ws.items[item];
  const int e = it.x, row0 = it.y, nrows = it.z;
  const int P = T * k;
  if (threadIdx.x < nrows) {
    const int r = row0 + threadIdx.x;
    int t;
    float wt;
    if (e < E) {
      const int p = sorted_pairs[r];
      const bool ok = p >= 0 && p < P;   // an invalid entry contributes nothing
      t = ok ? p / k : 0;
      wt = ok ? topk_w[p] : 0.0f;
    } else {
      t = r - P;
      wt = 1.0f;
    }
    s_tok[threadIdx.x] = t;
    s_w[threadIdx.x] = wt;
    s_u[threadIdx.x] = ws.unscale[t];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int nmt = (nrows + 15) / 16;
  const int KT = H / kTileCols;
  const int rt = rb * 4 + wid;
  const int64_t mat = static_cast<int64_t>(I) * H * 5 / 16;
  const uint8_t* gate = expert_base(L, e) + static_cast<int64_t>(rt) * KT * kTileBytes;
  const uint8_t* up = gate + mat;

  // A tile staging: 64 rows x 32 chunks of 8 halves; thread owns 8 chunks
  u32x4 areg[8];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 5, c8 = c & 31;
      if (row < nrows)
        areg[i] = *reinterpret_cast<const u32x4*>(ws.x16 + static_cast<size_t>(s_tok[row]) * H + kt * kTileCols + c8 * 8);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 5, c8 = c & 31;
      if (row < nrows) *reinterpret_cast<u32x4*>(&s_a[buf][row * kLdsStride + c8 * 8]) = areg[i];
    }
  };

  u32x4 cg, sg, cu, su, ncg, nsg, ncu, nsu;
  load_a(0);
  cg = load_codes(gate, lane); sg = load_scales(gate, lane);
  cu = load_codes(up, lane); su = load_scales(up, lane);
  store_a(0);
  __syncthreads();

  f32x4 acc_g[4], acc_u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { acc_g[i] = f32x4{0.f, 0.f, 0.f, 0.f}; acc_u[i] = acc_g[i]; }

  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1);
      const uint8_t* gn = gate + (kt + 1) * kTileBytes;
      const uint8_t* un = up + (kt + 1) * kTileBytes;
      ncg = load_codes(gn, lane); nsg = load_scales(gn, lane);
      ncu = load_codes(un, lane); nsu = load_scales(un, lane);
    }
    const _Float16* abuf = s_a[kt & 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16x8 bg = tile_block_weights(cg, sg, j);
      const f16x8 bu = tile_block_weights(cu, su, j);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < nmt) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(abuf + (mt * 16 + m) * kLdsStride + 32 * j + 8 * g);
          acc_g[mt] = mfma16(a, bg, acc_g[mt]);
          acc_u[mt] = mfma16(a, bu, acc_u[mt]);
        }
      }
    }
    if (more) {
      store_a((kt + 1) & 1);
      cg = ncg; sg = nsg; cu = ncu; su = nsu;
    }
    __syncthreads();
  }

  const int col = rt * 16 + m;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = mt * 16 + 4 * g + r;
        if (rl < nrows) {
          const float u = s_u[rl];
          const float s = 1.0f / u;
          const float gv = acc_g[mt][r] * u, uv = acc_u[mt][r] * u;
          const float h = s_w[rl] * silu(gv) * uv * (s * s);
          ws.h[static_cast<size_t>(row0 + rl) * I + col] = static_cast<_Float16>(h);
        }
      }
    }
  }
}

// --------------------------------------------------------------------- down --
__global__ __launch_bounds__(256) void prefill_down_kernel(LayerArgs L, PrefillWs ws) {
  __shared__ __align__(16) _Float16 s_a[2][kGroupRows * kLdsStride];
  const int H = L.H, I = L.I;
  const int RB = H / kDownRowsPerBlock;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int item = logical / RB;
  const int rb = logical % RB;
  if (item >= ws.hdr[0]) return;
  const int4 it = ws.items[item];
  const int e = it.x, row0 = it.y, nrows = it.z;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int nmt = (nrows + 15) / 16;
  const int KT = I / kTileCols;
  const int64_t mat = static_cast<int64_t>(I) * H * 5 / 16;
  const int rt0 = rb * 16 + wid * 4;
  const uint8_t* down = expert_base(L, e) + 2 * mat + static_cast<int64_t>(rt0) * KT * kTileBytes;

  u32x4 areg[8];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 5, c8 = c & 31;
      if (row < nrows)
        areg[i] = *reinterpret_cast<const u32x4*>(ws.h + static_cast<size_t>(row0 + row) * I + kt * kTileCols + c8 * 8);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int row = c >> 5, c8 = c & 31;
      if (row < nrows) *reinterpret_cast<u32x4*>(&s_a[buf][row * kLdsStride + c8 * 8]) = areg[i];
    }
  };

  u32x4 c[4], sc[4], nc[4], nsc[4];
  load_a(0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint8_t* rec = down + static_cast<int64_t>(q) * KT * kTileBytes;
    c[q] = load_codes(rec, lane);
    sc[q] = load_scales(rec, lane);
  }
  store_a(0);
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint8_t* rec = down + (static_cast<int64_t>(q) * KT + kt + 1) * kTileBytes;
        nc[q] = load_codes(rec, lane);
        nsc[q] = load_scales(rec, lane);
      }
    }
    const _Float16* abuf = s_a[kt & 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16x8 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        if (mt < nmt) a[mt] = *reinterpret_cast<const f16x8*>(abuf + (mt * 16 + m) * kLdsStride + 32 * j + 8 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f16x8 b = tile_block_weights(c[q], sc[q], j);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (mt < nmt) acc[q][mt] = mfma16(a[mt], b, acc[q][mt]);
      }
    }
    if (more) {
      store_a((kt + 1) & 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = nc[q]; sc[q] = nsc[q]; }
    }
    __syncthreads();
  }

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = (rt0 + q) * 16 + m;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < nmt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = mt * 16 + 4 * g + r;
          if (rl < nrows) ws.y[static_cast<size_t>(row0 + rl) * H + col] = static_cast<_Float16>(acc[q][mt][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine --
__global__ __launch_bounds__(256) void prefill_combine_kernel(
    int T, int H, int k, int has_shared, const int32_t* __restrict__ pair_pos,
    const void* __restrict__ residual, void* __restrict__ out, int out_bf16, PrefillWs ws) {
  const int t = blockIdx.x;
  const int P = T * k;
  const float u = ws.unscale[t];
  const float u2 = u * u;
  for (int c8 = threadIdx.x; c8 < H / 8; c8 += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int pos = min(max(pair_pos[static_cast<size_t>(t) * k + j], 0), P - 1);
      const f16x8 v = *reinterpret_cast<const f16x8*>(ws.y + static_cast<size_t>(pos) * H + c8 * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += static_cast<float>(v[i]);
    }
    if (has_shared) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(ws.y + static_cast<size_t>(P + t) * H + c8 * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += static_cast<float>(v[i]);
    }
    const size_t o = static_cast<size_t>(t) * H + c8 * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = acc[i] * u2;
      if (out_bf16) {
        if (residual) v += bf16_to_float(static_cast<const uint16_t*>(residual)[o + i]);
        static_cast<uint16_t*>(out)[o + i] = float_to_bf16(v);
      } else {
        if (residual) v += static_cast<const float*>(residual)[o + i];
        static_cast<float*>(out)[o + i] = v;
      }
    }
  }
}

}  // namespace

size_t prefill_workspace_bytes(int T, int E, int k, int H, int I) {
  const size_t rows = static_cast<size_t>(T) * k + T;
  return 256 + align256(sizeof(int4) * max_items(T, E, k)) + align256(sizeof(float) * T) +
         align256(sizeof(_Float16) * static_cast<size_t>(T) * H) + align256(sizeof(_Float16) * rows * I) +
         align256(sizeof(_Float16) * rows * H);
}

hipError_t launch_prefill(const LayerArgs& L, const void* x, int x_bf16, int T,
                          const int32_t* ids, const float* w, int k, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pairs,
                          const int32_t* pair_pos, const void* residual, void* out,
                          int out_bf16, int prenorm, void* wsp, hipStream_t s) {
  (void)ids;
  const PrefillWs ws = carve(wsp, T, L.E, k, L.H, L.I);
  const int nitems = max_items(T, L.E, k);
  hipError_t e;
  {
    ProfileScope prof(K_PREFILL_PREP, s);
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(T + 1), dim3(256), 0, s, L, x, x_bf16, T, k,
                       prenorm, counts, offsets, nitems, ws);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const long long nb = static_cast<long long>(nitems) * (L.I / kGateupRowsPerBlock);
    const int grid = static_cast<int>((nb + 7) / 8 * 8);
    ProfileScope prof(K_PREFILL_GATEUP, s);
    hipLaunchKernelGGL(prefill_gateup_kernel, dim3(grid), dim3(256), 0, s, L, T, k, sorted_pairs, w, ws);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const long long nb = static_cast<long long>(nitems) * (L.H / kDownRowsPerBlock);
    const int grid = static_cast<int>((nb + 7) / 8 * 8);
    ProfileScope prof(K_PREFILL_DOWN, s);
    hipLaunchKernelGGL(prefill_down_kernel, dim3(grid), dim3(256), 0, s, L, ws);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    ProfileScope prof(K_PREFILL_COMBINE, s);
    hipLaunchKernelGGL(prefill_combine_kernel, dim3(T), dim3(256), 0, s, T, L.H, k,
                       L.shared ? 1 : 0, pair_pos, residual, out, out_bf16, ws);
  }
  return hipGetLastError();
}

}  // namespace moeq2
