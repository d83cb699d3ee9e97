"""fp64 CPU oracle: routed-MoE expert layer (top-k router, token->expert
permutation, SwiGLU experts on 2-bit block-quantized weights, weighted combine
with one shared expert).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Every function here is
the plain definition of what the hot path computes, in float64, with numpy
primitives (matmul, argsort, bincount) as the only library steps.  No blocking,
fusion or reordering of arithmetic beyond the definitions cited below.

Sources (the pages are cited by title and section):
  * Model structure -- "Strata 实测：125B MoE 跑在 62 GB 内存的游戏本上"
    (kefong.net), section 二, model table: 48 layers, 512 routed experts per
    layer, 10 routed experts active per token plus 1 shared expert.
  * Weight format -- "32GB Mac mini 跑 1250 亿参数 Qwen3.8 Flash Next 实测"
    (blog.devlabs.cc), section 四, second validation layer: Q2_0 is a 2-bit
    code with an affine codebook of bias -1, and its dequantize round trip is
    checked to be bit exact.  The block size (32 weights), the fp16 per-block
    scale d and w = d*(q-1) are fixed by the workload definition that goes with
    this path.
  * Routing on the GPU hands the per-token list of selected expert ids to the
    expert compute -- "RTX PRO 4500 单卡跑 125B MoE" (lcz.me/topic/2169),
    section 最重要机制, item 1.
  * Prompt chunks are processed expert block by expert block -- strata-mlx
    README (bittide.aicompass.dev), section 它是什么; chunk size 1024 tokens --
    "32GB Mac mini ..." section 一.

Readings where the pages are silent:
  R1 tile layout of the 2-bit codes and fp16 scales (our own device format);
  R2 top-k ties go to the lower expert id, output slots in descending logit;
  R3 weights are the softmax over the selected k (== full softmax renormalised);
  R4 shared expert weight 1.0, no gate;  R5 SwiGLU = silu(gate) * up;
  R6 optional unweighted RMS pre-norm, eps 1e-6, for stacked layers;
  R7 stacked layers: x_{l+1} = x_l + MoE_l(rmsnorm(x_l)).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "TILE_ROWS", "TILE_COLS", "TILE_BYTES", "CODE_BYTES", "BLOCK",
    "matrix_nbytes", "expert_layout", "decode_matrix", "encode_matrix",
    "dequantize", "quantize_q2", "ExpertBlob",
    "router_logits", "route_topk", "route_weights", "route_histogram",
    "rms_prenorm", "silu", "expert_ffn", "moe_token", "moe_layer", "moe_stack",
    "RMS_EPS", "usage_counts", "residency_plan",
]

# --------------------------------------------------------------------------
# R1: the tiled Q2 format.  A matrix W with R rows and K columns (K is the
# reduction dimension) is cut into tiles of 16 rows x 256 columns.  Tile
# (rt, kt) is record rt*(K/256)+kt, 1280 bytes: 1024 bytes of codes, then 256
# bytes of fp16 scales.  Codes: 64 "lanes" of 16 bytes; lane L covers tile row
# n = L % 16 and column slice g = L // 16.  The lane's 16 bytes are four
# little-endian 32-bit words; word i carries blocks 2i and 2i+1 of the tile
# (block j = tile columns 32j..32j+31).  Nibble m of word i (bits 4m..4m+3)
# holds, in its low two bits, the code of column 32*(2i) + 8g + m and, in its
# high two bits, the code of column 32*(2i+1) + 8g + m.  Scales: fp16 of
# (row n, block j) at byte 1024 + 2*(8n + j).
# Dequantization (affine codebook, bias -1):  W = d * (q - 1).
# --------------------------------------------------------------------------
TILE_ROWS = 16
TILE_COLS = 256
CODE_BYTES = 1024
TILE_BYTES = 1280
BLOCK = 32
RMS_EPS = 1e-6


def matrix_nbytes(R: int, K: int) -> int:
    """Bytes of one R x K matrix: R*K/4 bytes of codes + R*K/32 fp16 scales."""
    if R % TILE_ROWS or K % TILE_COLS:
        raise ValueError("R must be a multiple of 16 and K of 256")
    return R * K * 5 // 16


def expert_layout(H: int, I: int) -> dict:
    """Byte offsets of gate (I x H), up (I x H) and down (H x I) inside one
    expert blob, and the expert stride (rounded up to 4 KiB)."""
    g = matrix_nbytes(I, H)
    d = matrix_nbytes(H, I)
    nbytes = 2 * g + d
    stride = (nbytes + 4095) // 4096 * 4096
    return {"gate": 0, "up": g, "down": 2 * g, "nbytes": nbytes, "stride": stride}


def decode_matrix(buf: np.ndarray, offset: int, R: int, K: int):
    """Read codes (uint8 0..3, [R, K]) and scales (float16, [R, K/32]) of one
    matrix from raw bytes, following the R1 layout above."""
    nb = matrix_nbytes(R, K)
    raw = np.asarray(buf, dtype=np.uint8)[offset:offset + nb]
    if raw.size != nb:
        raise ValueError("buffer too short for matrix")
    RT, KT = R // TILE_ROWS, K // TILE_COLS
    rec = raw.reshape(RT, KT, TILE_BYTES)
    words = rec[:, :, :CODE_BYTES].copy().view("<u4").reshape(RT, KT, 4, 16, 4)
    # words[rt, kt, g, n, i]  (lane L = 16*g + n, word i)
    codes = np.empty((RT, KT, 16, 8, 4, 8), dtype=np.uint8)  # [rt,kt,n,j,g,m]
    for i in range(4):
        w = words[:, :, :, :, i].transpose(0, 1, 3, 2)  # [rt, kt, n, g]
        for h in range(2):
            j = 2 * i + h
            for m in range(8):
                codes[:, :, :, j, :, m] = (w >> np.uint32(4 * m + 2 * h)) & np.uint32(3)
    # column inside the tile = 32*j + 8*g + m  ->  (j, g, m) nesting
    codes = codes.reshape(RT, KT, 16, TILE_COLS).transpose(0, 2, 1, 3).reshape(R, K)
    sc = rec[:, :, CODE_BYTES:].copy().view("<f2").reshape(RT, KT, 16, 8)
    scales = sc.transpose(0, 2, 1, 3).reshape(R, K // BLOCK)
    return codes, scales


def encode_matrix(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of decode_matrix: pack codes [R, K] (values 0..3) and fp16
    scales [R, K/32] into the R1 byte layout.  Used to build pinned inputs."""
    codes = np.asarray(codes)
    R, K = codes.shape
    if codes.min() < 0 or codes.max() > 3:
        raise ValueError("codes must be in 0..3")
    RT, KT = R // TILE_ROWS, K // TILE_COLS
    c = codes.astype(np.uint32).reshape(RT, 16, KT, 8, 4, 8)  # [rt,n,kt,j,g,m]
    c = c.transpose(0, 2, 1, 3, 4, 5)                          # [rt,kt,n,j,g,m]
    words = np.zeros((RT, KT, 4, 16, 4), dtype=np.uint32)     # [rt,kt,g,n,i]
    for i in range(4):
        acc = np.zeros((RT, KT, 16, 4), dtype=np.uint32)       # [rt,kt,n,g]
        for h in range(2):
            for m in range(8):
                acc |= c[:, :, :, 2 * i + h, :, m] << np.uint32(4 * m + 2 * h)
        words[:, :, :, :, i] = acc.transpose(0, 1, 3, 2)
    out = np.empty((RT, KT, TILE_BYTES), dtype=np.uint8)
    out[:, :, :CODE_BYTES] = words.astype("<u4").view(np.uint8).reshape(RT, KT, CODE_BYTES)
    s = np.asarray(scales, dtype="<f2").reshape(RT, 16, KT, 8).transpose(0, 2, 1, 3)
    out[:, :, CODE_BYTES:] = np.ascontiguousarray(s).view(np.uint8).reshape(RT, KT, 256)
    return out.reshape(-1)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[r, c] = float64(d[r, c // 32]) * (q[r, c] - 1)  (affine codebook,
    bias -1; "32GB Mac mini ..." section 四, second layer)."""
    d = np.repeat(np.asarray(scales, dtype=np.float64), BLOCK, axis=1)
    return d * (np.asarray(codes, dtype=np.float64) - 1.0)


def quantize_q2(W: np.ndarray):
    """The oracle's quantizer for the round-trip check: per 32-weight block
    d = max(max(w)/2, -min(w)) (so the codebook {-d, 0, d, 2d} covers the
    block), rounded to fp16, and q = clip(rint(w/d) + 1, 0, 3); an all-zero
    block gets d = 0, q = 1."""
    W = np.asarray(W, dtype=np.float64)
    R, K = W.shape
    blk = W.reshape(R, K // BLOCK, BLOCK)
    # "+ 0.0" turns a -0.0 (all-zero block) into +0.0 so the round trip is
    # bit exact, signed zeros included
    d = np.maximum(blk.max(axis=2) / 2.0, -blk.min(axis=2)) + 0.0
    d16 = d.astype(np.float16)
    d64 = d16.astype(np.float64)
    safe = np.where(d64 > 0, d64, 1.0)
    q = np.clip(np.rint(blk / safe[:, :, None]) + 1.0, 0, 3)
    q = np.where(d64[:, :, None] > 0, q, 1.0)
    return q.reshape(R, K).astype(np.uint8), d16


class ExpertBlob:
    """Read-only view of E experts (plus an optional shared expert) stored as
    raw bytes in the R1 layout: expert e at byte e*stride, each expert
    [gate | up | down].  Decoding is lazy and cached per expert."""

    def __init__(self, experts: np.ndarray, E: int, H: int, I: int,
                 shared: np.ndarray | None = None, stride: int | None = None,
                 cache: int = 64):
        self.lay = expert_layout(H, I)
        self.E, self.H, self.I = E, H, I
        self.stride = self.lay["stride"] if stride is None else stride
        self.experts = np.asarray(experts, dtype=np.uint8).reshape(-1)
        self.shared = None if shared is None else np.asarray(shared, dtype=np.uint8).reshape(-1)
        self._cache: dict = {}
        self._order: list = []
        self._cap = cache

    def _decode(self, buf, base):
        H, I, lay = self.H, self.I, self.lay
        Wg = dequantize(*decode_matrix(buf, base + lay["gate"], I, H))
        Wu = dequantize(*decode_matrix(buf, base + lay["up"], I, H))
        Wd = dequantize(*decode_matrix(buf, base + lay["down"], H, I))
        return Wg, Wu, Wd

    def weights(self, e):
        """(W_gate [I,H], W_up [I,H], W_down [H,I]) in float64; e == 'shared'
        selects the shared expert."""
        if e in self._cache:
            return self._cache[e]
        if e == "shared":
            if self.shared is None:
                raise KeyError("no shared expert")
            w = self._decode(self.shared, 0)
        else:
            if not 0 <= e < self.E:
                raise IndexError(e)
            w = self._decode(self.experts, int(e) * self.stride)
        self._cache[e] = w
        self._order.append(e)
        if len(self._order) > self._cap:
            self._cache.pop(self._order.pop(0), None)
        return w


# --------------------------------------------------------------------------
# Router (a1) and permutation (a2)
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Router logits for the GPU-side router (reading R7): the token
    activations times the router weight, W [E, H] with row e belonging to
    expert e, accumulated in float64 and rounded once to float32.  The
    routing step is the one that hands the per-token expert ids to the
    expert compute ("RTX PRO 4500 单卡跑 125B MoE", section 最重要机制,
    item 1)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return (x @ W.T).astype(np.float32)


def route_topk(logits: np.ndarray, k: int):
    """Per token, the k experts with the largest logit, compared as exact
    float32 values; equal logits go to the lower expert id (R2).  Returns
    ids [T, k] int32 in descending-logit order and weights [T, k] float64
    (route_weights).  Softmax is strictly increasing, so this is the top-k of
    the router probabilities."""
    lg = np.asarray(logits)
    if lg.dtype != np.float32 or lg.ndim != 2:
        raise TypeError("logits must be a float32 [T, E] array")
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("logits must be finite")
    # stable sort of the negated values: ties keep ascending expert id
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    return ids, route_weights(lg, ids)


def route_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = exp(l_j - m) / sum_{i in S_t} exp(l_i - m), m = max selected
    logit, in float64: the softmax over E renormalised over the selected set
    (R3)."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), ids, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route_histogram(ids: np.ndarray, E: int):
    """counts[e] = number of (token, slot) pairs routed to e; offsets =
    exclusive prefix sum (length E+1); sorted_pairs = pair ids p = t*k + j
    ordered by (expert, p) (a stable sort of the flattened ids); pair_pos =
    its inverse permutation."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    pair_pos = np.empty_like(sorted_pairs)
    pair_pos[sorted_pairs] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_pairs, pair_pos


# --------------------------------------------------------------------------
# Experts (a3..a7)
# --------------------------------------------------------------------------
def rms_prenorm(x: np.ndarray) -> np.ndarray:
    """R6: x_hat = x * (mean(x^2) + 1e-6)^(-1/2) per token, no weight."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + RMS_EPS)


def silu(a: np.ndarray) -> np.ndarray:
    # for a below about -709, exp(-a) is inf in float64 and a / inf = -0.0,
    # the correctly rounded value; the overflow is expected, not reported
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(xh: np.ndarray, Wg, Wu, Wd) -> np.ndarray:
    """R5: y = W_d (silu(W_g x) * (W_u x)) for each row of xh [n, H]."""
    xh = np.asarray(xh, dtype=np.float64)
    g = xh @ Wg.T
    u = xh @ Wu.T
    return (silu(g) * u) @ Wd.T


def moe_token(x_t, ids_t, w_t, blob: ExpertBlob, prenorm=False, residual_t=None):
    """Definition for one token: sum_j w_j * FFN_{ids_j}(x_hat) +
    FFN_shared(x_hat) (+ residual).  Used as the brute-force reference for
    moe_layer on small cases."""
    xh = rms_prenorm(x_t) if prenorm else np.asarray(x_t, dtype=np.float64)
    out = np.zeros(blob.H, dtype=np.float64)
    for e, w in zip(ids_t, w_t):
        out += w * expert_ffn(xh[None, :], *blob.weights(int(e)))[0]
    if blob.shared is not None:
        out += expert_ffn(xh[None, :], *blob.weights("shared"))[0]
    if residual_t is not None:
        out += np.asarray(residual_t, dtype=np.float64)
    return out


def moe_layer(x, ids, w, blob: ExpertBlob, prenorm=False, residual=None,
              tokens=None):
    """out[t] = sum_j w[t,j] * FFN_{ids[t,j]}(x_hat_t) + FFN_shared(x_hat_t)
    (+ residual[t]) for every token t (or only the listed `tokens`, returned
    in that order).  Tokens routed to the same expert are evaluated together
    so each expert is decoded once; the arithmetic per token is unchanged."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    sel = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    xh = rms_prenorm(x[sel]) if prenorm else x[sel]
    ids_s, w_s = ids[sel], w[sel]
    out = np.zeros((sel.size, blob.H), dtype=np.float64)
    for e in np.unique(ids_s):
        rows, slots = np.nonzero(ids_s == e)
        y = expert_ffn(xh[rows], *blob.weights(int(e)))
        # np.add.at: a token listing expert e twice adds both of its pairs
        np.add.at(out, rows, w_s[rows, slots][:, None] * y)
    if blob.shared is not None:
        out += expert_ffn(xh, *blob.weights("shared"))
    if residual is not None:
        out += np.asarray(residual, dtype=np.float64)[sel]
    return out


def moe_stack(x, layers, k, prenorm=True):
    """R7: x_{l+1} = x_l + MoE_l(rmsnorm(x_l)); `layers` yields
    (logits_fn, blob) per layer where logits_fn(x_l) gives float32 logits."""
    x = np.asarray(x, dtype=np.float64)
    for logits_fn, blob in layers:
        ids, w = route_topk(logits_fn(x), k)
        x = moe_layer(x, ids, w, blob, prenorm=prenorm, residual=x)
    return x


# --------------------------------------------------------------------------
# Expert residency (NEXT row f4): a fixed number of expert slots in fast
# memory hold the experts the recent routing used most; the refresh replaces
# the rest ("RTX PRO 4500 单卡跑 125B MoE", section 最重要机制, item 2: the
# resident expert set is refreshed every few rounds with the experts the
# conversation uses most).
# --------------------------------------------------------------------------
def usage_counts(ids: np.ndarray, E: int, counts=None) -> np.ndarray:
    """counts[e] (+=) the number of (token, slot) pairs routed to expert e;
    ids outside [0, E) are not counted."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    flat = flat[(flat >= 0) & (flat < E)]
    add = np.bincount(flat, minlength=E).astype(np.uint64)
    base = np.zeros(E, dtype=np.uint64) if counts is None else np.asarray(counts, dtype=np.uint64)
    return base + add


def residency_plan(counts: np.ndarray, S: int, expert_of_slot) -> tuple:
    """The S experts to hold: the S largest counts, equal counts going to the
    lower expert id.  An expert already in a slot and still chosen keeps its
    slot; the other chosen experts fill the remaining slots, lowest slot
    first, in ascending expert id.  expert_of_slot: the current occupant of
    each of the S slots (-1 = empty).  Returns (new_expert_of_slot [S],
    slot_of [E] with -1 for experts not held, changed slots [sorted])."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    if not 0 <= S <= E:
        raise ValueError("need 0 <= S <= E")
    cur = np.asarray(expert_of_slot, dtype=np.int64).reshape(-1)
    if cur.size != S:
        raise ValueError("expert_of_slot must have S entries")
    order = np.lexsort((np.arange(E), -counts))      # count descending, then id ascending
    chosen = set(int(e) for e in order[:S])
    new = np.full(S, -1, dtype=np.int64)
    kept = set()
    for s in range(S):
        e = int(cur[s])
        if e in chosen and e not in kept:
            new[s] = e
            kept.add(e)
    incoming = sorted(chosen - kept)
    free = [s for s in range(S) if new[s] < 0]
    for s, e in zip(free, incoming):
        new[s] = e
    slot_of = np.full(E, -1, dtype=np.int64)
    for s in range(S):
        slot_of[new[s]] = s
    changed = [s for s in range(S) if new[s] != cur[s]]
    return new.astype(np.int32), slot_of.astype(np.int32), np.array(changed, dtype=np.int32)
