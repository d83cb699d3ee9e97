"""Pins for the oracle's expert layer: brute force with explicit per-element
loops (reading the test's own code/scale arrays, not the oracle's decoder),
closed forms, and the pre-norm / stack definitions.

Structure pinned: 10-of-512 routed experts plus 1 shared expert per token
("Strata 实测 ..." (kefong.net), section 二, model table); shared expert weight
1 and SwiGLU silu(gate)*up are readings R4/R5.
"""
import math

import numpy as np
import pytest

import oracle as O


def make_blob(rng, E, H, I, code_fn=None, scale_fn=None):
    """Build E experts + a shared expert from explicit codes and scales;
    returns the blob and the per-expert (codes, scales) the test keeps."""
    lay = O.expert_layout(H, I)
    kept = []
    bufs = []
    for e in range(E + 1):
        mats = []
        parts = []
        for (R, K) in ((I, H), (I, H), (H, I)):
            q = code_fn(e, R, K) if code_fn else rng.integers(0, 4, size=(R, K), dtype=np.uint8)
            d = scale_fn(e, R, K) if scale_fn else rng.uniform(0.01, 0.05, size=(R, K // 32)).astype(np.float16)
            mats.append((q, d))
            parts.append(O.encode_matrix(q, d))
        b = np.zeros(lay["stride"], dtype=np.uint8)
        cat = np.concatenate(parts)
        b[:cat.size] = cat
        bufs.append(b)
        kept.append(mats)
    experts = np.concatenate(bufs[:E])
    blob = O.ExpertBlob(experts, E, H, I, shared=bufs[E])
    return blob, kept


def brute_ffn(x, mats):
    """y = Wd (silu(Wg x) * (Wu x)) with every weight formed as d*(q-1) from
    the stored arrays, element by element."""
    (qg, dg), (qu, du), (qd, dd) = mats
    I, H = qg.shape
    h = []
    for r in range(I):
        g = 0.0
        u = 0.0
        for c in range(H):
            g += float(dg[r, c // 32]) * (int(qg[r, c]) - 1) * x[c]
            u += float(du[r, c // 32]) * (int(qu[r, c]) - 1) * x[c]
        h.append(g / (1.0 + math.exp(-g)) * u)
    y = []
    for r in range(H):
        s = 0.0
        for c in range(I):
            s += float(dd[r, c // 32]) * (int(qd[r, c]) - 1) * h[c]
        y.append(s)
    return np.array(y)


def test_brute_force_tiny_layer():
    rng = np.random.default_rng(11)
    E, H, I, k, T = 5, 512, 256, 2, 2     # H != I catches a transposed operand
    blob, kept = make_blob(rng, E, H, I)
    x = rng.standard_normal((T, H))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    res = rng.standard_normal((T, H))
    out = O.moe_layer(x, ids, w, blob, residual=res)
    for t in range(T):
        ref = res[t].copy()
        for j in range(k):
            ref += w[t, j] * brute_ffn(x[t], kept[ids[t, j]])
        ref += brute_ffn(x[t], kept[E])
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-11)


def test_layer_matches_per_token_definition():
    rng = np.random.default_rng(12)
    E, H, I, k, T = 8, 256, 256, 3, 9
    blob, _ = make_blob(rng, E, H, I)
    x = rng.standard_normal((T, H))
    ids, w = O.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    out = O.moe_layer(x, ids, w, blob, prenorm=True)
    for t in range(T):
        assert np.allclose(out[t], O.moe_token(x[t], ids[t], w[t], blob, prenorm=True),
                           rtol=1e-12, atol=1e-12)
    sub = O.moe_layer(x, ids, w, blob, prenorm=True, tokens=[7, 2])
    assert np.allclose(sub, out[[7, 2]], rtol=1e-12, atol=1e-12)


def test_closed_form_codes_one_gives_shared_only():
    """Code 1 dequantizes to 0, so routed experts with only code 1 add nothing;
    the output is the shared expert alone (a dropped shared term fails here)."""
    rng = np.random.default_rng(13)
    E, H, I = 4, 256, 256
    ones = lambda e, R, K: np.ones((R, K), dtype=np.uint8) if e < E else rng.integers(0, 4, (R, K), dtype=np.uint8)
    blob, kept = make_blob(rng, E, H, I, code_fn=ones)
    x = rng.standard_normal((3, H))
    ids, w = O.route_topk(rng.standard_normal((3, E)).astype(np.float32), 2)
    out = O.moe_layer(x, ids, w, blob)
    assert np.any(out != 0)
    for t in range(3):
        assert np.allclose(out[t], brute_ffn(x[t], kept[E]), rtol=1e-11, atol=1e-11)
    # shared expert with code 1 as well -> zero output (+ residual)
    blob0, _ = make_blob(rng, E, H, I, code_fn=lambda e, R, K: np.ones((R, K), dtype=np.uint8))
    res = rng.standard_normal((3, H))
    assert np.array_equal(O.moe_layer(x, ids, w, blob0, residual=res), res)


def test_closed_form_all_code_two():
    """All codes 2, one scale d everywhere: g = u = d*sum(x), h = silu(g)*g,
    y_r = d*I*h for every output r; with k routed experts of weight summing
    to 1 plus the shared expert the output is 2*y."""
    rng = np.random.default_rng(14)
    E, H, I, d = 4, 256, 512, 0.03125
    blob, _ = make_blob(rng, E, H, I,
                        code_fn=lambda e, R, K: np.full((R, K), 2, dtype=np.uint8),
                        scale_fn=lambda e, R, K: np.full((R, K // 32), d, dtype=np.float16))
    x = rng.standard_normal((2, H)) * 0.1
    ids, w = O.route_topk(rng.standard_normal((2, E)).astype(np.float32), 3)
    out = O.moe_layer(x, ids, w, blob)
    for t in range(2):
        g = d * x[t].sum()
        h = g / (1 + math.exp(-g)) * g
        y = d * I * h
        assert np.allclose(out[t], 2 * y, rtol=1e-12, atol=0)


def test_zero_input_zero_output():
    rng = np.random.default_rng(15)
    blob, _ = make_blob(rng, 3, 256, 256)
    ids, w = O.route_topk(rng.standard_normal((2, 3)).astype(np.float32), 2)
    assert np.array_equal(O.moe_layer(np.zeros((2, 256)), ids, w, blob), np.zeros((2, 256)))


def test_prenorm_closed_form():
    x = np.full((2, 64), 3.0)
    xh = O.rms_prenorm(x)
    assert np.allclose(xh, 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    z = O.rms_prenorm(np.zeros((1, 8)))
    assert np.array_equal(z, np.zeros((1, 8)))
    # scale invariance up to eps: at 1000x the eps term is negligible
    y = np.random.default_rng(0).standard_normal((3, 128))
    ms = np.mean(y * y, axis=1, keepdims=True)
    assert np.allclose(O.rms_prenorm(1000 * y), y / np.sqrt(ms + 1e-12), rtol=1e-12)
    assert np.allclose(O.rms_prenorm(y), y / np.sqrt(ms + 1e-6), rtol=1e-14)


def test_silu_values():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-15
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15


def test_stack_is_residual_prenorm():
    rng = np.random.default_rng(16)
    E, H, I, k = 4, 256, 256, 2
    blobs = [make_blob(rng, E, H, I)[0] for _ in range(2)]
    W = [rng.standard_normal((H, E)) for _ in range(2)]
    x0 = rng.standard_normal((3, H))
    fns = [lambda x, Wl=Wl: (x @ Wl).astype(np.float32) for Wl in W]
    out = O.moe_stack(x0, zip(fns, blobs), k)
    x = x0
    for fn, b in zip(fns, blobs):
        ids, w = O.route_topk(fn(x), k)
        x = x + np.stack([O.moe_token(x[t], ids[t], w[t], b, prenorm=True) for t in range(3)])
    assert np.allclose(out, x, rtol=1e-12, atol=1e-12)


def test_every_token_same_experts_reduces_to_dense_gemms():
    """All tokens pick the same k experts: the layer is k dense SwiGLU
    GEMMs evaluated with numpy matmuls on the dequantized weights."""
    rng = np.random.default_rng(17)
    E, H, I, k, T = 6, 256, 256, 3, 5
    blob, kept = make_blob(rng, E, H, I)
    lg = np.tile(np.array([0.0, 3.0, 1.0, 2.0, -1.0, 0.5], dtype=np.float32), (T, 1))
    ids, w = O.route_topk(lg, k)
    assert np.all(ids == [1, 3, 2])
    x = rng.standard_normal((T, H))
    out = O.moe_layer(x, ids, w, blob)
    ref = np.zeros((T, H))
    for j, e in enumerate([1, 3, 2]):
        Wg, Wu, Wd = (O.dequantize(q, d) for q, d in kept[e])
        ref += w[0, j] * ((x @ Wg.T) / (1 + np.exp(-(x @ Wg.T))) * (x @ Wu.T)) @ Wd.T
    Wg, Wu, Wd = (O.dequantize(q, d) for q, d in kept[E])
    ref += ((x @ Wg.T) / (1 + np.exp(-(x @ Wg.T))) * (x @ Wu.T)) @ Wd.T
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_repeated_expert_in_a_token_adds_both_pairs():
    """A routing in which a token lists one expert twice: the layer is the sum
    over every listed pair (brute force), so both pairs count."""
    rng = np.random.default_rng(18)
    E, H, I, T = 4, 256, 256, 2
    blob, kept = make_blob(rng, E, H, I)
    x = rng.standard_normal((T, H))
    ids = np.array([[2, 2, 0], [1, 3, 1]], dtype=np.int32)
    w = np.array([[0.5, 0.3, 0.2], [0.1, 0.6, 0.3]])
    out = O.moe_layer(x, ids, w, blob)
    for t in range(T):
        ref = brute_ffn(x[t], kept[E])
        for j in range(3):
            ref = ref + w[t, j] * brute_ffn(x[t], kept[ids[t, j]])
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-11)
        assert np.allclose(out[t], O.moe_token(x[t], ids[t], w[t], blob), rtol=1e-12, atol=1e-12)


def test_stack_against_brute_force():
    """Two stacked layers on a tiny shape against element-by-element loops:
    rms pre-norm written as a loop, every FFN by brute_ffn, residual added."""
    rng = np.random.default_rng(19)
    E, H, I, k, T = 3, 256, 256, 2, 2
    made = [make_blob(rng, E, H, I) for _ in range(2)]
    W = [rng.standard_normal((H, E)) for _ in range(2)]
    x0 = rng.standard_normal((T, H))
    fns = [lambda x, Wl=Wl: (x @ Wl).astype(np.float32) for Wl in W]
    out = O.moe_stack(x0, zip(fns, [m[0] for m in made]), k)
    x = x0.copy()
    for (blob, kept), fn in zip(made, fns):
        ids, w = O.route_topk(fn(x), k)
        nxt = x.copy()
        for t in range(T):
            ss = 0.0
            for c in range(H):
                ss += x[t, c] * x[t, c]
            xh = x[t] / math.sqrt(ss / H + 1e-6)
            acc = brute_ffn(xh, kept[E])
            for j in range(k):
                acc = acc + w[t, j] * brute_ffn(xh, kept[ids[t, j]])
            nxt[t] = x[t] + acc
        x = nxt
    assert np.allclose(out, x, rtol=1e-10, atol=1e-10)
