// C-ABI entry points: argument validation (everything is checked before the
// first enqueue), workspace sizing, launch, status codes and the optional
// hipEvent measurement hooks.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_q2.h"
#include "launch.h"

namespace moeq2 {
namespace {

thread_local std::string g_last_error;

__attribute__((format(printf, 2, 3))) int fail(int status, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Whether the byte ranges [a, a + an) and [b, b + bn) share a byte.
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return an > 0 && bn > 0 && x < y + bn && y < x + an;
}

// ------------------------------------------------------ measurement hooks --
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[K_NUM_KERNELS];
  int64_t launches[K_NUM_KERNELS] = {};
  double total_ms[K_NUM_KERNELS] = {};
  std::vector<hipEvent_t> pool;

  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain(int id) {
    for (auto& pr : pending[id]) {
      float ms = 0.0f;
      if (hipEventSynchronize(pr.second) == hipSuccess &&
          hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) {
        total_ms[id] += ms;
        launches[id] += 1;
      }
      pool.push_back(pr.first);
      pool.push_back(pr.second);
    }
    pending[id].clear();
  }
};

Profiler& prof() {
  static Profiler p;
  return p;
}

const char* const kKernelNames[K_NUM_KERNELS] = {
    "route_topk_kernel",     "route_scan_kernel",     "route_scatter_kernel",
    "decode_gateup_kernel",  "decode_down_kernel",    "prefill_prep_kernel",
    "prefill_gateup_kernel", "prefill_down_kernel",   "prefill_combine_kernel",
    "route_gemv_topk_kernel", "usage_update_kernel",  "residency_map_kernel"};

bool valid_dtype(int d) { return d == MOE_F32 || d == MOE_BF16; }

int check_layer(const moe_q2_layer* L, int k) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "layer descriptor is NULL");
  if (!L->experts) return fail(MOE_ERR_INVALID_ARG, "layer->experts is NULL");
  if (L->num_experts < 1) return fail(MOE_ERR_INVALID_ARG, "num_experts must be >= 1");
  if (L->num_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "num_experts > 1024");
  if (L->hidden < 256 || L->inter < 256 || L->hidden % 256 || L->inter % 256)
    return fail(MOE_ERR_INVALID_ARG, "hidden and inter must be positive multiples of 256");
  if (L->hidden > MOE_MAX_DIM || L->inter > MOE_MAX_DIM)
    return fail(MOE_ERR_UNSUPPORTED, "hidden and inter must be <= 8192");
  const int64_t need = 3LL * L->hidden * L->inter * 5 / 16;
  if (L->expert_stride < need || L->expert_stride % 256)
    return fail(MOE_ERR_INVALID_ARG, "expert_stride must be >= 3*H*I*5/16 and a multiple of 256");
  if (!aligned(L->experts, 256) || (L->shared && !aligned(L->shared, 256)))
    return fail(MOE_ERR_INVALID_ARG, "expert weights must be 256-byte aligned");
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k must be >= 1");
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k must be <= 16");
  if (k > L->num_experts) return fail(MOE_ERR_INVALID_ARG, "k must be <= num_experts");
  return MOE_OK;
}

LayerArgs layer_args(const moe_q2_layer* L) {
  LayerArgs a;
  a.experts = static_cast<const uint8_t*>(L->experts);
  a.shared = static_cast<const uint8_t*>(L->shared);
  a.stride = L->expert_stride;
  a.E = L->num_experts;
  a.H = L->hidden;
  a.I = L->inter;
  return a;
}

size_t route_workspace(int T, int E, int k) {
  const size_t chunks = (static_cast<size_t>(T) + route_chunk_tokens(T) - 1) / route_chunk_tokens(T);
  const size_t rank = (static_cast<size_t>(T) * k * 4 + 255) / 256 * 256;
  const size_t cnt = (chunks * E * 4 + 255) / 256 * 256;
  return rank + 2 * cnt;
}

}  // namespace

ProfileScope::ProfileScope(int kernel_id)
    : id(kernel_id), ev0(nullptr), ev1(nullptr), committed(false) {
  Profiler& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> g(p.mu);
  ev0 = p.get();
  ev1 = ev0 ? p.get() : nullptr;
  if (!ev1 && ev0) { p.pool.push_back(ev0); ev0 = nullptr; }
}

void ProfileScope::commit() { committed = ev0 != nullptr; }

ProfileScope::~ProfileScope() {
  if (!ev0) return;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (committed) {
    p.pending[id].emplace_back(ev0, ev1);
  } else {
    p.pool.push_back(ev0);
    p.pool.push_back(ev1);
  }
}

}  // namespace moeq2

using namespace moeq2;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_bytes(int32_t op, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  if (T < 1 || E < 1 || k < 1 || T > MOE_MAX_TOKENS || k > MOE_MAX_TOPK || E > MOE_MAX_EXPERTS)
    return 0;
  switch (op) {
    case MOE_OP_ROUTE: return route_workspace(T, E, k);
    case MOE_OP_DECODE:
      if (T > MOE_MAX_DECODE_TOKENS || H < 256 || I < 256) return 0;
      return decode_workspace_bytes(T, k, H, I);
    case MOE_OP_PREFILL:
      if (H < 256 || I < 256) return 0;
      return prefill_workspace_bytes(T, E, k, H, I);
    case MOE_OP_ROUTE_GEMV:
      if (T > MOE_MAX_GEMV_TOKENS) return 0;
      return 256 + (static_cast<size_t>(T) * E * 4 + 255) / 256 * 256;
    default: return 0;
  }
}

int moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                   float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                   int32_t* pair_pos, void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID_ARG, "logits, topk_ids and topk_w are required");
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1");
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k must be >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k must be <= 16");
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k must be <= E");
  if (T > MOE_MAX_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "T must be <= 2^17");
  const int nhist = (counts != nullptr) + (offsets != nullptr) + (sorted_pairs != nullptr) + (pair_pos != nullptr);
  if (nhist != 0 && nhist != 4)
    return fail(MOE_ERR_INVALID_ARG, "counts, offsets, sorted_pairs and pair_pos: all or none");
  const bool hist = nhist == 4;
  if (hist) {
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is required for the histogram");
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < route_workspace(T, E, k))
      return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)route_workspace(T, E, k));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!hist) {
    e = launch_route_topk(logits, T, E, k, topk_ids, topk_w, nullptr, nullptr, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "route_topk launch");
  }
  const int chunks = (T + route_chunk_tokens(T) - 1) / route_chunk_tokens(T);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* rank = reinterpret_cast<int32_t*>(ws);
  const size_t rank_b = (static_cast<size_t>(T) * k * 4 + 255) / 256 * 256;
  const size_t cnt_b = (static_cast<size_t>(chunks) * E * 4 + 255) / 256 * 256;
  int32_t* local = reinterpret_cast<int32_t*>(ws + rank_b);
  int32_t* base = reinterpret_cast<int32_t*>(ws + rank_b + cnt_b);
  if (route_histogram_fused(T, k)) {   // one chunk: the histogram in the same launch
    e = launch_route_topk(logits, T, E, k, topk_ids, topk_w, rank, local, s, counts, offsets,
                          sorted_pairs, pair_pos);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "route_topk launch");
  }
  if ((e = launch_route_topk(logits, T, E, k, topk_ids, topk_w, rank, local, s)) != hipSuccess)
    return hip_fail(e, "route_topk launch");
  if ((e = launch_route_expert_scan(local, base, E, chunks, counts, s)) != hipSuccess)
    return hip_fail(e, "route_scan launch");
  if ((e = launch_route_scatter(topk_ids, rank, base, counts, E, T, k, chunks, offsets, sorted_pairs,
                                pair_pos, s)) != hipSuccess)
    return hip_fail(e, "route_scatter launch");
  return MOE_OK;
}

int moe_route_topk_gemv(const void* x, int32_t x_dtype, int32_t T, const uint16_t* router_w,
                        int32_t E, int32_t H, int32_t k, float* logits, int32_t* topk_ids,
                        float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !router_w) return fail(MOE_ERR_INVALID_ARG, "x and router_w are required");
  if ((topk_ids == nullptr) != (topk_w == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "topk_ids and topk_w: both or neither");
  const bool select = topk_ids != nullptr;
  if (!select && !logits) return fail(MOE_ERR_INVALID_ARG, "logits is required without topk_ids");
  if (!valid_dtype(x_dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1");
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (k < 1) return fail(MOE_ERR_INVALID_ARG, "k must be >= 1");
  if (H < 256 || H % 256) return fail(MOE_ERR_INVALID_ARG, "H must be a positive multiple of 256");
  if (T > MOE_MAX_GEMV_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "at most 4 tokens");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k must be <= 16");
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "k must be <= E");
  if (H > MOE_MAX_DIM) return fail(MOE_ERR_UNSUPPORTED, "H must be <= 8192");
  if (!aligned(x, 16) || !aligned(router_w, 16) || (logits && !aligned(logits, 4)) ||
      (select && (!aligned(topk_ids, 4) || !aligned(topk_w, 4))))
    return fail(MOE_ERR_INVALID_ARG, "x and router_w must be 16-byte aligned, the outputs 4-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (select) {   // the counter (and the logits when not requested) live in the workspace
    if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is required");
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t need = moe_workspace_bytes(MOE_OP_ROUTE_GEMV, T, E, k, H, 0);
    if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)need);
  }
  float* lg = logits ? logits : reinterpret_cast<float*>(ws + 256);
  const hipError_t e = launch_route_gemv_topk(x, x_dtype == MOE_BF16, T, router_w, E, H, k, lg, topk_ids,
                                             topk_w, select ? reinterpret_cast<uint32_t*>(ws) : nullptr,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "route_gemv_topk launch");
}

// Every argument of a forward call except the workspace.
static int check_forward_args(const moe_q2_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                              const int32_t* ids, const float* w, int32_t k, const void* residual,
                              const void* out, int32_t out_dtype, uint32_t flags) {
  int st = check_layer(layer, k);
  if (st) return st;
  if (!x || !ids || !w || !out) return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_w and out are required");
  if (!valid_dtype(x_dtype) || !valid_dtype(out_dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (flags & ~MOE_FLAG_PRENORM_RMS) return fail(MOE_ERR_INVALID_ARG, "unknown flag");
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1");
  {
    // out must not share a byte with x; residual is either out itself or
    // disjoint from it
    const size_t n = static_cast<size_t>(T) * static_cast<size_t>(layer->hidden);
    const size_t xb = n * (x_dtype == MOE_BF16 ? 2 : 4), ob = n * (out_dtype == MOE_BF16 ? 2 : 4);
    if (overlaps(x, xb, out, ob)) return fail(MOE_ERR_INVALID_ARG, "out must not overlap x");
    if (residual && residual != out && overlaps(residual, ob, out, ob))
      return fail(MOE_ERR_INVALID_ARG, "residual must be out itself or not overlap it");
  }
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(residual, 16) || !aligned(ids, 4) || !aligned(w, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "x, out and residual must be 16-byte aligned, topk_ids and topk_w 4-byte aligned");
  return MOE_OK;
}

static int check_workspace(void* workspace) {
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is required");
  if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return MOE_OK;
}

static int check_forward(const moe_q2_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                         const int32_t* ids, const float* w, int32_t k, const void* residual, const void* out,
                         int32_t out_dtype, uint32_t flags, void* workspace) {
  int st = check_forward_args(layer, x, x_dtype, T, ids, w, k, residual, out, out_dtype, flags);
  return st ? st : check_workspace(workspace);
}

// The arguments of the routed decode call except the workspace.
static int check_routed_args(const moe_q2_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                             const float* logits, int32_t k, const int32_t* topk_ids, const float* topk_w,
                             const void* residual, const void* out, int32_t out_dtype, uint32_t flags) {
  if (!logits) return fail(MOE_ERR_INVALID_ARG, "logits is required");
  if ((topk_ids == nullptr) != (topk_w == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "topk_ids and topk_w: both or neither");
  if (!aligned(logits, 4) || (topk_ids && (!aligned(topk_ids, 4) || !aligned(topk_w, 4))))
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_ids and topk_w must be 4-byte aligned");
  // the routing outputs are optional here, so check the rest with stand-ins
  int st = check_forward_args(layer, x, x_dtype, T, reinterpret_cast<const int32_t*>(logits), logits, k,
                              residual, out, out_dtype, flags);
  if (st) return st;
  if (T > MOE_MAX_DECODE_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "decode takes at most 8 tokens");
  return MOE_OK;
}

static int launch_routed(const moe_q2_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                         const float* logits, int32_t k, int32_t* topk_ids, float* topk_w,
                         const void* residual, void* out, int32_t out_dtype, uint32_t flags,
                         void* workspace, void* stream) {
  const hipError_t e = launch_decode(layer_args(layer), x, x_dtype == MOE_BF16, T, nullptr, nullptr,
                                     logits, topk_ids, topk_w, k, residual, out,
                                     out_dtype == MOE_BF16, (flags & MOE_FLAG_PRENORM_RMS) ? 1 : 0,
                                     workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "decode launch");
}

int moe_expert_forward_decode(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                              int32_t T, const int32_t* topk_ids, const float* topk_w, int32_t k,
                              const void* residual, void* out, int32_t out_dtype, uint32_t flags,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_forward(layer, x, x_dtype, T, topk_ids, topk_w, k, residual, out, out_dtype, flags, workspace);
  if (st) return st;
  if (T > MOE_MAX_DECODE_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "decode takes at most 8 tokens");
  const size_t need = decode_workspace_bytes(T, k, layer->hidden, layer->inter);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)need);
  const hipError_t e = launch_decode(layer_args(layer), x, x_dtype == MOE_BF16, T, topk_ids, topk_w,
                                     nullptr, nullptr, nullptr, k, residual, out,
                                     out_dtype == MOE_BF16, (flags & MOE_FLAG_PRENORM_RMS) ? 1 : 0,
                                     workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "decode launch");
}

int moe_expert_forward_decode_routed(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                                     int32_t T, const float* logits, int32_t k, int32_t* topk_ids,
                                     float* topk_w, const void* residual, void* out,
                                     int32_t out_dtype, uint32_t flags, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  int st = check_routed_args(layer, x, x_dtype, T, logits, k, topk_ids, topk_w, residual, out, out_dtype, flags);
  if (st || (st = check_workspace(workspace))) return st;
  const size_t need = decode_workspace_bytes(T, k, layer->hidden, layer->inter);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)need);
  return launch_routed(layer, x, x_dtype, T, logits, k, topk_ids, topk_w, residual, out, out_dtype, flags,
                       workspace, stream);
}

int moe_expert_forward_decode_routed_noalloc(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                                             int32_t T, const float* logits, int32_t k,
                                             int32_t* topk_ids, float* topk_w, const void* residual,
                                             void* out, int32_t out_dtype, uint32_t flags, void* stream) {
  int st = check_routed_args(layer, x, x_dtype, T, logits, k, topk_ids, topk_w, residual, out, out_dtype, flags);
  if (st) return st;
  const size_t need = decode_workspace_bytes(T, k, layer->hidden, layer->inter);
  if (need > decode_static_scratch_bytes())
    return fail(MOE_ERR_UNSUPPORTED, "the call needs %lld bytes of scratch, the static scratch holds %lld",
                (long long)need, (long long)decode_static_scratch_bytes());
  void* scratch = nullptr;
  const hipError_t e = decode_static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "static decode scratch");
  return launch_routed(layer, x, x_dtype, T, logits, k, topk_ids, topk_w, residual, out, out_dtype, flags,
                       scratch, stream);
}

static int check_prefill(const moe_q2_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                         const int32_t* topk_ids, const float* topk_w, int32_t k, const int32_t* counts,
                         const int32_t* offsets, const int32_t* sorted_pairs, const int32_t* pair_pos,
                         const void* residual, const void* out, int32_t out_dtype, uint32_t flags,
                         void* workspace, size_t workspace_bytes) {
  int st = check_forward(layer, x, x_dtype, T, topk_ids, topk_w, k, residual, out, out_dtype, flags, workspace);
  if (st) return st;
  if (!counts || !offsets || !sorted_pairs || !pair_pos)
    return fail(MOE_ERR_INVALID_ARG, "counts, offsets, sorted_pairs and pair_pos are required");
  if (T > MOE_MAX_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "T must be <= 2^17");
  const size_t need = prefill_workspace_bytes(T, layer->num_experts, k, layer->hidden, layer->inter);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)need);
  return MOE_OK;
}

int moe_expert_forward_prefill(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                               int32_t T, const int32_t* topk_ids, const float* topk_w, int32_t k,
                               const int32_t* counts, const int32_t* offsets,
                               const int32_t* sorted_pairs, const int32_t* pair_pos,
                               const void* residual, void* out, int32_t out_dtype, uint32_t flags,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_prefill(layer, x, x_dtype, T, topk_ids, topk_w, k, counts, offsets, sorted_pairs, pair_pos,
                              residual, out, out_dtype, flags, workspace, workspace_bytes);
  if (st) return st;
  const hipError_t e = launch_prefill(layer_args(layer), x, x_dtype == MOE_BF16, T, topk_ids, topk_w, k,
                                      counts, offsets, sorted_pairs, pair_pos, residual, out,
                                      out_dtype == MOE_BF16, (flags & MOE_FLAG_PRENORM_RMS) ? 1 : 0,
                                      workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "prefill launch");
}

// ------------------------------------------------------------- residency --

int moe_expert_usage_update(const int32_t* ids, int64_t n, int32_t E, uint64_t* counts, void* stream) {
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
  if (n < 0 || n > 0x7FFFFFFFLL) return fail(MOE_ERR_INVALID_ARG, "n must be in 0..2^31-1");
  if (n > 0 && (!ids || !counts)) return fail(MOE_ERR_INVALID_ARG, "ids and counts are required");
  if (!aligned(ids, 4) || !aligned(counts, 8))
    return fail(MOE_ERR_INVALID_ARG, "ids must be 4-byte and counts 8-byte aligned");
  const hipError_t e = launch_usage_update(ids, n, E, reinterpret_cast<unsigned long long*>(counts),
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "usage update launch");
}

namespace {

// Occupants of S slots: each -1 or an expert in [0, E), no expert twice.
// slot_of (E entries) receives the inverse map.
int check_occupants(const int32_t* occ, int32_t E, int32_t S, std::vector<int32_t>& slot_of, const char* name) {
  slot_of.assign(static_cast<size_t>(E), -1);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t e = occ[s];
    if (e < -1 || e >= E) return fail(MOE_ERR_INVALID_ARG, "%s[%d] = %d is not -1 or an expert", name, s, e);
    if (e >= 0) {
      if (slot_of[e] >= 0) return fail(MOE_ERR_INVALID_ARG, "%s holds expert %d twice", name, e);
      slot_of[e] = s;
    }
  }
  return MOE_OK;
}

}  // namespace

int moe_residency_plan(const uint64_t* counts, int32_t E, int32_t S, const int32_t* expert_of_slot,
                       int32_t* new_expert_of_slot, int32_t* slot_of, int32_t* n_changed) {
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
  if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARG, "S must be in 0..E");
  if (!counts) return fail(MOE_ERR_INVALID_ARG, "counts is required");
  if (S > 0 && (!expert_of_slot || !new_expert_of_slot))
    return fail(MOE_ERR_INVALID_ARG, "expert_of_slot and new_expert_of_slot are required");
  std::vector<int32_t> cur_slot;
  const std::vector<int32_t> cur(expert_of_slot, expert_of_slot + S);
  int st = check_occupants(cur.data(), E, S, cur_slot, "expert_of_slot");
  if (st) return st;
  // the S largest counts, ties to the lower id
  std::vector<int32_t> order(static_cast<size_t>(E));
  for (int32_t e = 0; e < E; ++e) order[e] = e;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return counts[a] != counts[b] ? counts[a] > counts[b] : a < b;
  });
  std::vector<char> chosen(static_cast<size_t>(E), 0);
  for (int32_t i = 0; i < S; ++i) chosen[order[i]] = 1;
  // chosen experts already held stay where they are
  std::vector<int32_t> next(static_cast<size_t>(S), -1);
  for (int32_t s = 0; s < S; ++s)
    if (cur[s] >= 0 && chosen[cur[s]]) next[s] = cur[s];
  // the others, in ascending id, into the free slots, lowest first
  int32_t free_slot = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (!chosen[e] || cur_slot[e] >= 0) continue;
    while (next[free_slot] >= 0) ++free_slot;
    next[free_slot] = e;
  }
  int32_t changed = 0;
  for (int32_t s = 0; s < S; ++s) changed += next[s] != cur[s];
  std::copy(next.begin(), next.end(), new_expert_of_slot);
  if (slot_of) {
    for (int32_t e = 0; e < E; ++e) slot_of[e] = -1;
    for (int32_t s = 0; s < S; ++s) slot_of[next[s]] = s;
  }
  if (n_changed) *n_changed = changed;
  return MOE_OK;
}

int moe_residency_apply(const void* arena, int64_t expert_stride, int32_t E, int32_t S,
                        const int32_t* old_expert_of_slot, const int32_t* new_expert_of_slot, void* slots,
                        int32_t* slot_of, void* stream) {
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "E must be >= 1");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E must be <= 1024");
  if (S < 0 || S > E) return fail(MOE_ERR_INVALID_ARG, "S must be in 0..E");
  if (!arena || !slot_of) return fail(MOE_ERR_INVALID_ARG, "arena and slot_of are required");
  if (S > 0 && (!slots || !old_expert_of_slot || !new_expert_of_slot))
    return fail(MOE_ERR_INVALID_ARG, "slots, old_expert_of_slot and new_expert_of_slot are required");
  if (expert_stride < 256 || expert_stride % 256)
    return fail(MOE_ERR_INVALID_ARG, "expert_stride must be a positive multiple of 256");
  if (!aligned(arena, 256) || !aligned(slots, 256) || !aligned(slot_of, 4))
    return fail(MOE_ERR_INVALID_ARG, "arena and slots must be 256-byte aligned, slot_of 4-byte aligned");
  std::vector<int32_t> old_slot, new_slot;
  int st = check_occupants(old_expert_of_slot, E, S, old_slot, "old_expert_of_slot");
  if (st || (st = check_occupants(new_expert_of_slot, E, S, new_slot, "new_expert_of_slot"))) return st;
  for (int32_t e = 0; e < E; ++e)
    if (old_slot[e] >= 0 && new_slot[e] >= 0 && old_slot[e] != new_slot[e])
      return fail(MOE_ERR_INVALID_ARG, "expert %d moves from slot %d to slot %d", e, old_slot[e], new_slot[e]);
  // map changes: experts that leave (-> -1) and that enter (-> slot); the
  // two sets are disjoint, so their order does not matter
  std::vector<uint32_t> recs;
  for (int32_t e = 0; e < E; ++e)
    if (old_slot[e] != new_slot[e]) recs.push_back(static_cast<uint32_t>(e) | (static_cast<uint32_t>(new_slot[e] + 1) << 16));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* dst = static_cast<uint8_t*>(slots);
  const uint8_t* src = static_cast<const uint8_t*>(arena);
  for (int32_t q = 0; q < S; ++q) {
    const int32_t e = new_expert_of_slot[q];
    if (e < 0 || e == old_expert_of_slot[q]) continue;
    const hipError_t he = hipMemcpyAsync(dst + q * expert_stride, src + e * expert_stride,
                                         static_cast<size_t>(expert_stride), hipMemcpyDefault, s);
    if (he != hipSuccess) return hip_fail(he, "slot copy");
  }
  for (size_t i = 0; i < recs.size(); i += kMapRecs) {
    MapRecs m{};
    const int n = static_cast<int>(std::min<size_t>(kMapRecs, recs.size() - i));
    std::copy(recs.begin() + i, recs.begin() + i + n, m.rec);
    const hipError_t he = launch_residency_map(slot_of, m, n, s);
    if (he != hipSuccess) return hip_fail(he, "slot map launch");
  }
  return MOE_OK;
}

namespace {

// A tiered layer checked as an untiered one whose experts are the arena.
moe_q2_layer flat_of(const moe_q2_tiered_layer* t) {
  moe_q2_layer L;
  L.experts = t->arena;
  L.shared = t->shared;
  L.expert_stride = t->expert_stride;
  L.num_experts = t->num_experts;
  L.hidden = t->hidden;
  L.inter = t->inter;
  return L;
}

// Device address of `p`: device memory as it is, pinned host memory through
// its device mapping; other memory (pageable host memory) is refused.
int device_view(const void* p, const uint8_t** dev, int* kind) {
  hipPointerAttribute_t a;
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // not sticky: the next launch checks the error state
    return fail(MOE_ERR_INVALID_ARG, "arena is neither device memory nor pinned host memory");
  }
  *kind = a.type;
  if (a.type == hipMemoryTypeDevice) {
    *dev = static_cast<const uint8_t*>(p);
    return MOE_OK;
  }
  if (a.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return fail(MOE_ERR_INVALID_ARG, "arena is pinned host memory without a device mapping");
    }
    *dev = static_cast<const uint8_t*>(d);
    return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_ARG, "arena is neither device memory nor pinned host memory");
}

// Everything a tiered call adds to the untiered checks, and its LayerArgs.
int tier_args(const moe_q2_tiered_layer* t, LayerArgs& a) {
  if (!t->arena) return fail(MOE_ERR_INVALID_ARG, "layer->arena is NULL");
  if (!t->slot_of || !aligned(t->slot_of, 4))
    return fail(MOE_ERR_INVALID_ARG, "layer->slot_of is required (4-byte aligned)");
  if (t->num_slots < 0 || t->num_slots > t->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "num_slots must be in 0..num_experts");
  if (t->num_slots > 0 && (!t->slots || !aligned(t->slots, 256)))
    return fail(MOE_ERR_INVALID_ARG, "layer->slots is required with num_slots > 0 (256-byte aligned)");
  // the first and the last byte of the arena are memory the device can read
  const uint8_t* dev = nullptr;
  const uint8_t* dev_end = nullptr;
  int kind = 0, kind_end = 0;
  int st = device_view(t->arena, &dev, &kind);
  if (st) return st;
  const uint8_t* last = static_cast<const uint8_t*>(t->arena) + t->num_experts * t->expert_stride - 1;
  if ((st = device_view(last, &dev_end, &kind_end))) return st;
  if (kind_end != kind || dev_end != dev + t->num_experts * t->expert_stride - 1)
    return fail(MOE_ERR_INVALID_ARG, "the arena's E * expert_stride bytes are not one mapped range");
  a.experts = static_cast<const uint8_t*>(t->slots);
  a.slot_of = t->slot_of;
  a.arena = dev;
  a.S = t->num_slots;
  return MOE_OK;
}

}  // namespace

int moe_expert_forward_decode_tiered(const moe_q2_tiered_layer* layer, const void* x, int32_t x_dtype,
                                     int32_t T, const float* logits, int32_t k, int32_t* topk_ids,
                                     float* topk_w, const void* residual, void* out, int32_t out_dtype,
                                     uint32_t flags, uint64_t* usage_counts, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!layer) return fail(MOE_ERR_INVALID_ARG, "layer descriptor is NULL");
  const moe_q2_layer flat = flat_of(layer);
  int st = check_routed_args(&flat, x, x_dtype, T, logits, k, topk_ids, topk_w, residual, out, out_dtype, flags);
  if (st || (st = check_workspace(workspace))) return st;
  if (!aligned(usage_counts, 8)) return fail(MOE_ERR_INVALID_ARG, "usage_counts must be 8-byte aligned");
  const size_t need = decode_workspace_bytes(T, k, layer->hidden, layer->inter);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace too small: need %lld bytes", (long long)need);
  LayerArgs a = layer_args(&flat);
  if ((st = tier_args(layer, a))) return st;
  a.usage = reinterpret_cast<unsigned long long*>(usage_counts);
  const hipError_t e = launch_decode(a, x, x_dtype == MOE_BF16, T, nullptr, nullptr, logits, topk_ids, topk_w, k,
                                     residual, out, out_dtype == MOE_BF16, (flags & MOE_FLAG_PRENORM_RMS) ? 1 : 0,
                                     workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "decode launch");
}

int moe_expert_forward_prefill_tiered(const moe_q2_tiered_layer* layer, const void* x, int32_t x_dtype,
                                      int32_t T, const int32_t* topk_ids, const float* topk_w, int32_t k,
                                      const int32_t* counts, const int32_t* offsets,
                                      const int32_t* sorted_pairs, const int32_t* pair_pos,
                                      const void* residual, void* out, int32_t out_dtype, uint32_t flags,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!layer) return fail(MOE_ERR_INVALID_ARG, "layer descriptor is NULL");
  const moe_q2_layer flat = flat_of(layer);
  int st = check_prefill(&flat, x, x_dtype, T, topk_ids, topk_w, k, counts, offsets, sorted_pairs, pair_pos,
                         residual, out, out_dtype, flags, workspace, workspace_bytes);
  if (st) return st;
  LayerArgs a = layer_args(&flat);
  if ((st = tier_args(layer, a))) return st;
  const hipError_t e = launch_prefill(a, x, x_dtype == MOE_BF16, T, topk_ids, topk_w, k, counts, offsets,
                                      sorted_pairs, pair_pos, residual, out, out_dtype == MOE_BF16,
                                      (flags & MOE_FLAG_PRENORM_RMS) ? 1 : 0, workspace,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "prefill launch");
}

int moe_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return MOE_OK;
}

int moe_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (int i = 0; i < K_NUM_KERNELS; ++i) {
    p.drain(i);
    p.launches[i] = 0;
    p.total_ms[i] = 0.0;
  }
  return MOE_OK;
}

int moe_profile_num_kernels(void) { return K_NUM_KERNELS; }

const char* moe_profile_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= K_NUM_KERNELS) return nullptr;
  return kKernelNames[kernel_id];
}

int moe_profile_query(int kernel_id, int64_t* launches, double* total_ms) {
  if (kernel_id < 0 || kernel_id >= K_NUM_KERNELS || !launches || !total_ms)
    return fail(MOE_ERR_INVALID_ARG, "bad kernel id or NULL output");
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.drain(kernel_id);
  *launches = p.launches[kernel_id];
  *total_ms = p.total_ms[kernel_id];
  return MOE_OK;
}

}  // extern "C"
