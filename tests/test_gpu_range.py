"""Range and special cases of the HIP path against the fp64 oracle, through
the C ABI.

* Closed forms: every weight of every expert equal (every 2-bit code c,
  every block scale d = fp16(0.05)), x = +1 or -1 everywhere, with and
  without the pre-norm.  Then g = u = d (c - 1) sum(x) for every row and the
  intermediates reach 1e4..1e7, far beyond fp16's range at H = 3072 and
  8192, while the outputs stay well inside float32.  Where silu(g) u
  underflows float32 (x = -1 against codes 2 and 3, g near -150 or -300) the
  exact output is below float32's smallest normal number, so those cases
  allow float32's own resolution (np.finfo(float32).tiny) on top of the
  usual 2e-2 * rms bar.
* Block scales 400..1600 times the usual ones (outputs near 1e9).
* Tokens whose activations differ by up to 10^14 in scale in one call, each
  checked against its own rms.
* A token listing one expert twice (decode and prefill sum its weights).
* The decode down kernel reading h~ from the workspace (too large for LDS).
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_expert_router_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2
TINY = float(np.finfo(np.float32).tiny)


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_quantized_expert_router_amd import binding
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(gpu, ref, what, slack=0.0):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref).max()
    rms = np.sqrt(np.mean(ref * ref))
    print(f"{what}: max|err| = {err:.3e}  rms(ref) = {rms:.3e}  ratio = {err / max(rms, 1e-300):.2e}",
          flush=True)
    assert np.all(np.isfinite(gpu)), what
    assert err <= TOL * rms + slack, (what, err, rms)


class DevLayer:
    """A layer on the device (dev) and its oracle view (ref)."""
    def __init__(self, B, blob, sh, E, H, I):
        self.E, self.H, self.I = E, H, I
        self.dev = B.Layer(dev(blob), dev(sh), E, H, I, synth.expert_stride(H, I))
        self.ref = O.ExpertBlob(blob, E, H, I, shared=sh)


def random_layer(B, seed, E, H, I, **scales):
    return DevLayer(B, synth.expert_blob(synth.rng_for(seed, 0, 1), E, H, I, **scales),
                     synth.expert_blob(synth.rng_for(seed, 0, 2), 1, H, I, **scales), E, H, I)


_const = {}


def const_layer(B, E, H, I, code):
    key = (E, H, I, code)
    if key not in _const:
        _const.clear()          # keep one layer (and its decoded experts) at a time
        _const[key] = DevLayer(B, synth.constant_expert_blob(E, H, I, code, 0.05),
                                synth.constant_expert_blob(1, H, I, code, 0.05), E, H, I)
    return _const[key]


def run_routed(B, L, x, lg, k, flags=0):
    T = x.shape[0]
    out = torch.empty((T, L.H), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, L.E, k, L.H, L.I)
    B.moe_expert_forward_decode_routed(L.dev, x, lg, k, out, None, None, None, flags, ws)
    torch.cuda.synchronize()
    return out


def run_prefill(B, L, x, r, flags=0):
    T, k = r["topk_ids"].shape
    out = torch.empty((T, L.H), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.MOE_OP_PREFILL, T, L.E, k, L.H, L.I)
    B.moe_expert_forward_prefill(L.dev, x, r["topk_ids"], r["topk_w"], r["counts"], r["offsets"],
                                 r["sorted_pairs"], r["pair_pos"], out, None, flags, ws)
    torch.cuda.synchronize()
    return out


CLOSED = [(H, code, sign, pre) for H in (3072, 8192) for code in (0, 2, 3) for sign in (1.0, -1.0)
          for pre in (False, True)]


@pytest.mark.parametrize("H,code,sign,pre", CLOSED)
def test_decode_closed_forms(B, H, code, sign, pre):
    """Decode (T = 1 and T = 3, top-4 of 6 + shared, I = 768) on equal
    weights: with codes 2 or 3 and x = +1 (codes 0 and x = -1), h = silu(g) g
    is 2.4e4..6.7e5, beyond fp16."""
    E, I, k = 6, 768, 4
    L = const_layer(B, E, H, I, code)
    slack = TINY if (code - 1) * sign < 0 else 0.0
    for T in (1, 3):
        print(f"closed form decode H={H} code={code} x={sign:+.0f} prenorm={pre} T={T}", flush=True)
        rng = synth.rng_for(70, T, H + code)
        xv = np.full((T, H), sign, dtype=np.float32)
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = O.route_topk(lg, k)
        out = run_routed(B, L, dev(xv), dev(lg), k, B.MOE_FLAG_PRENORM_RMS if pre else 0)
        ref = O.moe_layer(xv, ids, w, L.ref, prenorm=pre)
        check(to_np(out), ref, f"decode H={H} code={code} x={sign:+.0f} pre={pre} T={T}", slack)


@pytest.mark.parametrize("code,sign,pre", [(c, s, p) for c in (0, 2, 3) for s in (1.0, -1.0)
                                           for p in (False, True)])
def test_prefill_closed_forms(B, code, sign, pre):
    """Prefill at the 512-expert layer's widths (H 3072, I 768) on equal
    weights: 100 tokens, top-4 of 8 + shared, so each expert has about 50
    rows (four M tiles) and the shared expert 100 (two work items); y
    reaches about 1e6 (codes 2) and 4e6 (codes 3)."""
    E, H, I, k, T = 8, 3072, 768, 4, 100
    L = const_layer(B, E, H, I, code)
    slack = TINY if (code - 1) * sign < 0 else 0.0
    print(f"closed form prefill code={code} x={sign:+.0f} prenorm={pre}", flush=True)
    rng = synth.rng_for(71, code, int(sign > 0))
    xv = np.full((T, H), sign, dtype=np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    r = B.route(dev(lg), k, histogram=True)
    out = run_prefill(B, L, dev(xv), r, B.MOE_FLAG_PRENORM_RMS if pre else 0)
    ref = O.moe_layer(xv, ids, w, L.ref, prenorm=pre)
    check(to_np(out), ref, f"prefill code={code} x={sign:+.0f} pre={pre}", slack)


def test_large_scales(B):
    """Block scales U(20, 80) (400..1600 times the usual): outputs near 1e9,
    decode and prefill, random codes and N(0, 1) activations."""
    E, H, I, k = 16, 3072, 768, 4
    L = random_layer(B, 72, E, H, I, scale_lo=20.0, scale_hi=80.0)
    Ld, ref_blob = L.dev, L.ref
    rng = synth.rng_for(72, 0, 3)
    for T in (2, 40):
        _, xv = synth.activations(rng, T, H, "f32")
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = O.route_topk(lg, k)
        ref = O.moe_layer(xv, ids, w, ref_blob)
        r = B.route(dev(lg), k, histogram=True)
        if T <= 8:
            out = torch.empty((T, H), dtype=torch.float32, device="cuda")
            ws = B.workspace(B.MOE_OP_DECODE, T, E, k, H, I)
            B.moe_expert_forward_decode(Ld, dev(xv), r["topk_ids"], r["topk_w"], out, None, 0, ws)
            torch.cuda.synchronize()
            check(to_np(out), ref, f"decode large scales T={T}")
        outp = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws = B.workspace(B.MOE_OP_PREFILL, T, E, k, H, I)
        B.moe_expert_forward_prefill(Ld, dev(xv), r["topk_ids"], r["topk_w"], r["counts"], r["offsets"],
                                     r["sorted_pairs"], r["pair_pos"], outp, None, 0, ws)
        torch.cuda.synchronize()
        check(to_np(outp), ref, f"prefill large scales T={T}")


def test_token_scales_apart(B):
    """Eight tokens scaled by 10^-7 .. 10^0 (no pre-norm): outputs from about
    1e-12 to 1e2 in one call; every token against its own rms."""
    E, H, I, k, T = 16, 1024, 256, 4, 8
    L = random_layer(B, 73, E, H, I)
    ref_blob = L.ref
    rng = synth.rng_for(73, 0, 3)
    _, xv = synth.activations(rng, T, H, "f32")
    xv = (xv * (10.0 ** (np.arange(T) - 7))[:, None]).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    ref = O.moe_layer(xv, ids, w, ref_blob)
    out_d = to_np(run_routed(B, L, dev(xv), dev(lg), k))
    out_p = to_np(run_prefill(B, L, dev(xv), B.route(dev(lg), k, histogram=True)))
    for t in range(T):
        check(out_d[t], ref[t], f"decode token {t} (x * 1e{t - 7})")
        check(out_p[t], ref[t], f"prefill token {t} (x * 1e{t - 7})")


def test_repeated_expert_in_a_token(B):
    """Routing given by the caller in which tokens list an expert twice (and
    one id outside [0, E), which contributes nothing): decode and prefill
    equal the oracle's sum over the listed pairs."""
    E, H, I, k, T = 16, 1024, 256, 4, 3
    L = random_layer(B, 74, E, H, I)
    Ld, ref_blob = L.dev, L.ref
    rng = synth.rng_for(74, 0, 3)
    _, xv = synth.activations(rng, T, H, "f32")
    ids = np.array([[3, 3, 7, 1], [5, 9, 5, 5], [2, 11, 4, 6]], dtype=np.int32)
    w = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.3, 0.2], [0.1, 0.2, 0.3, 0.4]], dtype=np.float32)
    ref = O.moe_layer(xv, ids, w.astype(np.float64), ref_blob)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, E, k, H, I)
    B.moe_expert_forward_decode(Ld, dev(xv), dev(ids), dev(w), out, None, 0, ws)
    torch.cuda.synchronize()
    check(to_np(out), ref, "decode, repeated ids")
    counts, offsets, sp, pp = O.route_histogram(ids, E)
    r = {"topk_ids": dev(ids), "topk_w": dev(w), "counts": dev(counts), "offsets": dev(offsets),
         "sorted_pairs": dev(sp), "pair_pos": dev(pp)}
    outp = run_prefill(B, L, dev(xv), r)
    check(to_np(outp), ref, "prefill, repeated ids")
    # an id outside [0, E) contributes nothing (decode)
    ids2 = ids.copy()
    ids2[0, 3] = E + 5
    ref2 = ref.copy()
    ref2[0] -= 0.1 * O.expert_ffn(xv[:1].astype(np.float64), *ref_blob.weights(1))[0]
    B.moe_expert_forward_decode(Ld, dev(xv), dev(ids2), dev(w), out, None, 0, ws)
    torch.cuda.synchronize()
    check(to_np(out), ref2, "decode, one id out of range")


def test_decode_down_from_workspace(B):
    """T = 8, k = 16, I = 2048: 136 pairs of h~ (557 KB) do not fit in LDS,
    so the down kernel reads h~ from the workspace and rescales each fragment
    there.  Routed decode against the oracle, and equal to the two-call form."""
    E, H, I, k, T = 32, 1024, 2048, 16, 8
    L = random_layer(B, 75, E, H, I)
    Ld, ref_blob = L.dev, L.ref
    rng = synth.rng_for(75, 0, 3)
    xd, xv = synth.activations(rng, T, H, "bf16")
    x = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).cuda()
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    out = run_routed(B, L, x, dev(lg), k)
    check(to_np(out), O.moe_layer(xv, ids, w, ref_blob), "decode, h~ read from the workspace")
    r = B.route(dev(lg), k)
    two = torch.empty_like(out)
    B.moe_expert_forward_decode(Ld, x, r["topk_ids"], r["topk_w"], two, None, 0,
                                B.workspace(B.MOE_OP_DECODE, T, E, k, H, I))
    torch.cuda.synchronize()
    assert torch.equal(out, two)
