/*
 * moe_q2.h -- C ABI of the MI355X (gfx950) routed-MoE expert layer on 2-bit
 * block-quantized weights.
 *
 * The layer is the routed mixture-of-experts block of a 48-layer model with
 * 512 routed experts per layer, 10 of them active per token plus 1 shared
 * expert ("Strata 实测：125B MoE 跑在 62 GB 内存的游戏本上", kefong.net,
 * section 二, model table).  Experts are SwiGLU FFNs whose weights stay in
 * their 2-bit blocks: Q2_0, an affine codebook with bias -1
 * ("32GB Mac mini 跑 1250 亿参数 Qwen3.8 Flash Next 实测", blog.devlabs.cc,
 * section 四, second validation layer), 32 weights per block, one fp16 scale
 * d per block, w = d * (q - 1).
 *
 * Three calls make up one layer:
 *   moe_route_topk             router top-k + weights (+ token->expert
 *                              histogram and stable permutation for prefill)
 *   moe_expert_forward_decode  1..8 tokens (a decode step or a verify window)
 *   moe_expert_forward_prefill any number of tokens (prompt chunks of 1024
 *                              or 32768 tokens), grouped by expert
 * and moe_expert_forward_decode_routed does the first two for decode in one
 * call; moe_route_topk_gemv computes the router logits themselves and their
 * top-k for decode.  The residency tier (moe_expert_usage_update,
 * moe_residency_plan, moe_residency_apply and the *_tiered forward calls)
 * keeps the most used experts in device slots and reads the others from an
 * arena in device or pinned host memory.
 *
 * Conventions for every entry point
 *   - Pointers marked [device] are device addresses (hipMalloc'd memory or
 *     torch tensors); [host] pointers are read during the call only.
 *   - The caller owns all memory, including `workspace`.  The library never
 *     allocates, frees or synchronises, and never reads device data on the
 *     host (the tiered calls only ask the runtime what kind of memory the
 *     arena is).  Each call only enqueues work -- kernels, and for
 *     moe_residency_apply slot copies -- on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream), in stream order.
 *   - Every argument is validated before anything is enqueued: a non-zero
 *     status means nothing was enqueued (except MOE_ERR_HIP, which reports a
 *     failed launch; moe_last_error() gives the detail).
 *   - Calls are re-entrant; calls that may run concurrently need separate
 *     workspaces.  Inputs must be finite (NaN/Inf give unspecified results).
 *   - Results are deterministic: no floating-point atomics, fixed summation
 *     order; repeated calls on the same inputs give the same bytes.
 *
 * Weight layout (one expert = [gate | up | down], gate/up are I x H, down is
 * H x I; rows are output features, columns the reduction dimension).  A matrix
 * of R rows x K columns (R % 16 == 0, K % 256 == 0) is a row-tile-major array
 * of 1280-byte tile records, tile (rt, kt) covering rows 16rt..16rt+15 and
 * columns 256kt..256kt+255 at record index rt*(K/256) + kt.  Record bytes
 * 0..1023 hold the 2-bit codes as 64 lanes of 16 bytes: lane L covers tile row
 * n = L % 16 and column slice g = L / 16; its four little-endian 32-bit words
 * w_i (i = 0..3) hold blocks 2i and 2i+1 of the tile; nibble m (bits
 * 4m..4m+3) of w_i holds the code of column 32*(2i) + 8g + m in its low two
 * bits and that of column 32*(2i+1) + 8g + m in its high two bits.  Bytes
 * 1024..1279 hold the fp16 scale of (row n, block j) at 1024 + 2*(8n + j).
 * A matrix takes R*K*5/16 bytes (2.5 bits per weight); gate starts at byte 0
 * of the expert, up at I*H*5/16, down at 2*I*H*5/16.
 */
#ifndef MOE_Q2_H
#define MOE_Q2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad alignment      */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside the library's limits    */
  MOE_ERR_WORKSPACE = -3,    /* workspace smaller than moe_workspace_bytes */
  MOE_ERR_HIP = -4           /* a kernel launch failed                     */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* x_hat = x * (mean(x^2) + 1e-6)^(-1/2) per token (no weight) before the
 * experts; the pre-norm of a residual block x + MoE(rmsnorm(x)). */
#define MOE_FLAG_PRENORM_RMS 1u

enum { MOE_OP_ROUTE = 0, MOE_OP_DECODE = 1, MOE_OP_PREFILL = 2, MOE_OP_ROUTE_GEMV = 3 };

/* Limits of the library (validated): */
#define MOE_MAX_EXPERTS 1024     /* E                                        */
#define MOE_MAX_TOPK 16          /* k                                        */
#define MOE_MAX_DECODE_TOKENS 8  /* T of moe_expert_forward_decode           */
#define MOE_MAX_GEMV_TOKENS 4    /* T of moe_route_topk_gemv                  */
#define MOE_MAX_DIM 8192         /* H and I (each a multiple of 256)         */
#define MOE_MAX_TOKENS (1 << 17) /* T of routing and prefill (131072)        */

typedef struct {
  const void* experts;    /* [device] E experts; expert e at experts + e*expert_stride;
                             256-byte aligned                                  */
  const void* shared;     /* [device] the shared expert (same layout), or NULL */
  int64_t expert_stride;  /* bytes, >= 3*I*H*5/16, multiple of 256             */
  int32_t num_experts;    /* E, 1..1024                                        */
  int32_t hidden;         /* H, multiple of 256, <= 8192                       */
  int32_t inter;          /* I (expert intermediate size), multiple of 256     */
} moe_q2_layer;

/* Bytes of workspace the given call needs (0 if none).  op is MOE_OP_*; for
 * MOE_OP_ROUTE the size assumes the histogram outputs are requested. */
size_t moe_workspace_bytes(int32_t op, int32_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/*
 * Router (the per-token list of selected experts that the GPU hands to the
 * expert compute: "RTX PRO 4500 单卡跑 125B MoE", lcz.me/topic/2169, section
 * 最重要机制, item 1).
 *   logits   [device] float32 [T, E] row-major router logits.
 *   topk_ids [device] int32 [T, k]: the k experts with the largest logits,
 *            compared as exact float32 values (-0.0 == +0.0); equal logits go
 *            to the lower expert id; slots in descending logit order.
 *   topk_w   [device] float32 [T, k]: exp(l_j - l_max) / sum over the k
 *            selected (the softmax over E renormalised over the selection).
 *   counts, offsets, sorted_pairs, pair_pos: [device] int32 [E], [E+1],
 *            [T*k], [T*k], all four or none (NULL).  counts[e] = pairs routed
 *            to e; offsets = exclusive prefix sum; sorted_pairs = pair ids
 *            p = t*k + j ordered by (expert, p); pair_pos = its inverse.
 *   workspace [device] >= moe_workspace_bytes(MOE_OP_ROUTE, ...) when the
 *            histogram is requested (else may be NULL), 256-byte aligned.
 * Errors: INVALID_ARG for null required pointers, T < 1, k < 1, k > E, a
 * partial set of histogram outputs; UNSUPPORTED for E > 1024, k > 16,
 * T > 2^17; WORKSPACE when too small.
 */
int moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                   int32_t* topk_ids, float* topk_w,
                   int32_t* counts, int32_t* offsets,
                   int32_t* sorted_pairs, int32_t* pair_pos,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Router logits and top-k in one kernel, for T = 1..4 decode tokens: the
 * router is the linear map logits = x W^T with a bf16 weight W [E, H]
 * (the routing step that hands the selected expert ids to the expert
 * compute, "RTX PRO 4500 ...", section 最重要机制, item 1).  Each logit is
 * the dot product of exact fp64 products accumulated in fp64 and rounded
 * once to float32; the selection and weights are then exactly those of
 * moe_route_topk on these logits.
 *   x         [device] [T, H] activations, x_dtype MOE_F32 or MOE_BF16, 16-byte aligned.
 *   router_w  [device] bf16 [E, H] (row e belongs to expert e), 16-byte aligned.
 *   logits    [device] float32 [T, E] output, or NULL (then only in the workspace).
 *   topk_ids, topk_w  [device] [T, k] outputs, or both NULL: then only the
 *             logits are computed (they must then be requested), e.g. to feed
 *             moe_expert_forward_decode_routed, which takes the top-k itself.
 *   workspace [device] >= moe_workspace_bytes(MOE_OP_ROUTE_GEMV, T, E, k, H, 0),
 *             256-byte aligned; may be NULL when topk_ids is NULL.  Its first
 *             4 bytes are a counter that must be zero before the first call
 *             on this workspace; every call leaves it zero.  Concurrent calls
 *             need separate workspaces.
 * Errors: INVALID_ARG (null x or router_w, only one of topk_ids / topk_w,
 * neither logits nor topk_ids, T, E or k < 1, k > E, H not a multiple of 256,
 * unknown dtype, misalignment), UNSUPPORTED (T > 4, E > 1024, k > 16,
 * H > 8192), WORKSPACE.
 */
int moe_route_topk_gemv(const void* x, int32_t x_dtype, int32_t T, const uint16_t* router_w,
                        int32_t E, int32_t H, int32_t k, float* logits, int32_t* topk_ids,
                        float* topk_w, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-time expert layer for T = 1..8 tokens (one decode step or a verify
 * window that checks a few drafted tokens at once: "32GB Mac mini ...",
 * section 一, and "RTX PRO 4500 ...", section 最重要机制, item 3).  Only the
 * selected experts' weights are read.
 *   layer     [host] weights descriptor (above).
 *   x         [device] [T, H] activations, x_dtype MOE_F32 or MOE_BF16;
 *             16-byte aligned (as are out and residual).
 *   topk_ids, topk_w  [device] [T, k] as produced by moe_route_topk.  A
 *             token may list an expert more than once (its weights then add
 *             up); an id outside [0, E) contributes nothing.
 *   residual  [device] [T, H] in out_dtype, or NULL; either `out` itself
 *             (updated in place) or not overlapping it.
 *   out       [device] [T, H] in out_dtype; must not overlap x:
 *             out[t] = sum_j topk_w[t,j] * FFN_{topk_ids[t,j]}(x_hat_t)
 *                      + FFN_shared(x_hat_t) (+ residual[t]),
 *             FFN(x) = W_down (silu(W_gate x) * (W_up x)).
 *   flags     0 or MOE_FLAG_PRENORM_RMS.
 *   workspace [device] >= moe_workspace_bytes(MOE_OP_DECODE, ...), 256-B aligned.
 * Errors: INVALID_ARG (null pointers, T < 1, k < 1 or > E, stride too small or
 * unaligned, H or I not multiples of 256, unknown dtype or flag),
 * UNSUPPORTED (T > 8, E > 1024, k > 16, H or I > 8192), WORKSPACE.
 */
int moe_expert_forward_decode(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                              int32_t T, const int32_t* topk_ids, const float* topk_w,
                              int32_t k, const void* residual, void* out, int32_t out_dtype,
                              uint32_t flags, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Router and decode-time expert layer in one call, for T = 1..8 tokens: the
 * top-k of `logits` is taken inside the expert kernels (every workgroup
 * selects the experts of the T tokens itself), so no separate routing
 * kernel runs before the weights can be fetched.  Same routing as
 * moe_route_topk and same `out` as moe_expert_forward_decode on that routing.
 *   logits    [device] float32 [T, E] router logits (E = layer->num_experts).
 *   topk_ids, topk_w  [device] [T, k] outputs, or both NULL: receive the
 *             routing (identical to moe_route_topk's).
 *   other arguments as for moe_expert_forward_decode; the workspace size is
 *             moe_workspace_bytes(MOE_OP_DECODE, ...).
 * Errors: as for moe_expert_forward_decode, plus INVALID_ARG for a NULL
 * `logits` or only one of topk_ids / topk_w.
 */
int moe_expert_forward_decode_routed(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                                     int32_t T, const float* logits, int32_t k,
                                     int32_t* topk_ids, float* topk_w, const void* residual,
                                     void* out, int32_t out_dtype, uint32_t flags,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_forward_decode_routed without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The workspace is a
 * static device array inside the library, one per GPU, of
 * MOE_DECODE_STATIC_SCRATCH_BYTES (2,306,048 bytes: the largest decode call,
 * T = 8, k = 16, I = 8192), held from the first call on that GPU until the
 * process ends.  Its address is resolved on the first call on each device
 * (hipGetSymbolAddress with that device current); no call allocates or
 * frees anything.  Nothing in it needs to start at zero.
 * Every call on one GPU uses the same array: calls that may overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller, e.g. all on one stream.
 * Arguments, results and errors: as moe_expert_forward_decode_routed, plus
 * UNSUPPORTED if a call would need more scratch than the array holds, and
 * HIP if the array's address cannot be resolved.
 */
#define MOE_DECODE_STATIC_SCRATCH_BYTES 2306048
int moe_expert_forward_decode_routed_noalloc(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                                             int32_t T, const float* logits, int32_t k,
                                             int32_t* topk_ids, float* topk_w, const void* residual,
                                             void* out, int32_t out_dtype, uint32_t flags, void* stream);

/*
 * Prefill-time expert layer for a chunk of T tokens, grouped by expert from
 * the routing histogram (prompts are read in chunks and the experts are
 * processed block by block: strata-mlx README, section 它是什么; chunk sizes
 * 1024 and 32768: "Strata 实测 ...", section 四, change 4).
 * Arguments as for the decode call, plus the four histogram arrays from
 * moe_route_topk for the same topk_ids.  Computes the same `out`.
 * Errors: as for decode, with T limited to 1..2^17 instead of 1..8 (so that
 * every activation offset fits in 32 bits).
 */
int moe_expert_forward_prefill(const moe_q2_layer* layer, const void* x, int32_t x_dtype,
                               int32_t T, const int32_t* topk_ids, const float* topk_w,
                               int32_t k, const int32_t* counts, const int32_t* offsets,
                               const int32_t* sorted_pairs, const int32_t* pair_pos,
                               const void* residual, void* out, int32_t out_dtype,
                               uint32_t flags, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Residency tier: the hottest experts in device memory, the rest read from
 * an arena that holds all of them ("RTX PRO 4500 单卡跑 125B MoE",
 * lcz.me/topic/2169, section 最重要机制: the table of what sits in VRAM,
 * RAM and SSD, and items 1 and 2 -- experts the GPU does not hold are
 * computed where they are, and the resident set is re-chosen every few
 * rounds from the experts the conversation uses most).  On MI355X the GPU
 * itself reads a non-resident expert: from device memory, or from pinned
 * host memory mapped into the device's address space (hipHostMalloc), over
 * PCIe; no CPU pipeline is involved.
 *
 * The layer descriptor of a tiered call:
 */
typedef struct {
  const void* slots;      /* [device] S resident experts: slot s at slots + s*expert_stride;
                             256-byte aligned (may be NULL when S = 0)          */
  const int32_t* slot_of; /* [device] int32 [E]: the slot holding expert e, or -1; a
                             value outside [0, S) reads e from the arena         */
  const void* arena;      /* every expert: e at arena + e*expert_stride; device memory or
                             mapped pinned host memory (validated), 256-B aligned */
  const void* shared;     /* [device] the shared expert, or NULL                 */
  int64_t expert_stride;  /* bytes, >= 3*I*H*5/16, multiple of 256               */
  int32_t num_slots;      /* S, 0..E                                            */
  int32_t num_experts;    /* E, 1..1024                                          */
  int32_t hidden;         /* H, multiple of 256, <= 8192                         */
  int32_t inter;          /* I, multiple of 256, <= 8192                         */
} moe_q2_tiered_layer;

/*
 * Usage histogram: counts[e] += the number of entries of ids[0..n) equal to
 * e (entries outside [0, E) are skipped).  Integer atomics: the result does
 * not depend on order.  The caller clears counts to start a window.
 *   ids    [device] int32 [n] (e.g. topk_ids of a prefill chunk), n >= 0.
 *   counts [device] uint64 [E], 8-byte aligned.
 * Errors: INVALID_ARG (NULL pointers with n > 0, E < 1, n > 2^31 - 1),
 * UNSUPPORTED (E > 1024).
 */
int moe_expert_usage_update(const int32_t* ids, int64_t n, int32_t E, uint64_t* counts, void* stream);

/*
 * Residency plan (host only; no device memory, nothing enqueued): the S
 * experts to hold are those with the S largest counts, equal counts going
 * to the lower expert id.  A chosen expert already in a slot keeps it; the
 * other chosen experts fill the remaining slots, lowest slot first, in
 * ascending expert id.
 *   counts             [host] uint64 [E] usage counts.
 *   expert_of_slot     [host] int32 [S] current occupant of each slot, -1 =
 *                      empty; distinct experts in [0, E).
 *   new_expert_of_slot [host] int32 [S] out: the plan (may alias
 *                      expert_of_slot only if it is not needed afterwards).
 *   slot_of            [host] int32 [E] out, or NULL: slot of each expert
 *                      under the plan, -1 if not held.
 *   n_changed          [host] out, or NULL: slots whose occupant changes.
 * Errors: INVALID_ARG (NULL counts or outputs with S > 0, E < 1, S outside
 * 0..E, an occupant out of range or held twice), UNSUPPORTED (E > 1024).
 */
int moe_residency_plan(const uint64_t* counts, int32_t E, int32_t S, const int32_t* expert_of_slot,
                       int32_t* new_expert_of_slot, int32_t* slot_of, int32_t* n_changed);

/*
 * Move the tier from one plan to the next on `stream`: for each slot whose
 * occupant changes to an expert, its expert_stride bytes are copied from the
 * arena (hipMemcpyAsync), then the device map slot_of is updated for the
 * experts that leave and enter (a small kernel whose changes travel as
 * kernel arguments, so the host arrays are read during the call only).
 *   arena, expert_stride, E, S   as in moe_q2_tiered_layer.
 *   old_expert_of_slot [host] int32 [S]: the occupants slot_of describes now
 *                      (all -1, with slot_of all -1, before the first plan).
 *   new_expert_of_slot [host] int32 [S]: the occupants to move to; an expert
 *                      held in both keeps its slot (as moe_residency_plan
 *                      guarantees).
 *   slots   [device] the S slots (written).  slot_of [device] int32 [E].
 * Calls that read the tier must be ordered after this one (the same stream,
 * or an event); calls ordered before it read the old state.
 * Errors: INVALID_ARG (NULL pointers, bad alignment or stride, S outside
 * 0..E, occupants out of range or repeated, an expert that changes slot),
 * UNSUPPORTED (E > 1024), HIP (a copy or launch failed).
 */
int moe_residency_apply(const void* arena, int64_t expert_stride, int32_t E, int32_t S,
                        const int32_t* old_expert_of_slot, const int32_t* new_expert_of_slot,
                        void* slots, int32_t* slot_of, void* stream);

/*
 * moe_expert_forward_decode_routed and moe_expert_forward_prefill on a
 * tiered layer: each selected expert is read from its slot, or from the
 * arena when slot_of gives none.  The outputs are those of the untiered
 * calls on the arena's experts, bit for bit, whatever the plan.
 *   usage_counts [device] uint64 [E] or NULL (decode only): += the pairs
 *                routed to each expert, as moe_expert_usage_update on
 *                topk_ids, inside the expert kernels (no extra launch).
 * Errors: as for the untiered calls, plus INVALID_ARG for a NULL arena or
 * slot_of, S outside 0..E, NULL slots with S > 0, an arena that is neither
 * device memory nor pinned host memory, or misaligned pointers.
 */
int moe_expert_forward_decode_tiered(const moe_q2_tiered_layer* layer, const void* x, int32_t x_dtype,
                                     int32_t T, const float* logits, int32_t k, int32_t* topk_ids,
                                     float* topk_w, const void* residual, void* out, int32_t out_dtype,
                                     uint32_t flags, uint64_t* usage_counts, void* workspace,
                                     size_t workspace_bytes, void* stream);
int moe_expert_forward_prefill_tiered(const moe_q2_tiered_layer* layer, const void* x, int32_t x_dtype,
                                      int32_t T, const int32_t* topk_ids, const float* topk_w, int32_t k,
                                      const int32_t* counts, const int32_t* offsets,
                                      const int32_t* sorted_pairs, const int32_t* pair_pos,
                                      const void* residual, void* out, int32_t out_dtype,
                                      uint32_t flags, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Text of a status code; detail of the last error on this thread. */
const char* moe_status_string(int status);
const char* moe_last_error(void);

/*
 * Measurement hooks (host-side only; no device memory).  When enabled, every
 * kernel is launched with a pair of hipEvents that the runtime stamps with the
 * begin and end of that dispatch (hipExtLaunchKernel), so the pair measures
 * the kernel's execution alone; moe_profile_query returns, per kernel id, the
 * number of launches and the summed time (it waits for the events).  Ids run
 * 0..moe_profile_num_kernels()-1; moe_profile_kernel_name names them.  Leave
 * the hooks off while a stream is being captured into a graph.
 */
int moe_profile_enable(int on);
int moe_profile_reset(void);
int moe_profile_num_kernels(void);
const char* moe_profile_kernel_name(int kernel_id);
int moe_profile_query(int kernel_id, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q2_H */
