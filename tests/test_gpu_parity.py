"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Bars: routing ids, counts, offsets, sorted_pairs and pair_pos bit exact;
routing weights |dw| <= 1e-6 and |sum w - 1| <= 1e-6; expert outputs
max|out - ref| <= 2e-2 * rms(ref) over the whole output (relative L2 is
reported too).  Small cases are checked on every output; the full-size
workloads (512 experts, H 3072, I 768; prefill chunks of 1024 and 32768
tokens) on tokens sampled from the same call the benchmark makes.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantized_expert_router_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_quantized_expert_router_amd import binding
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_x(xdev, dtype):
    if dtype == "bf16":
        return torch.from_numpy(xdev.view(np.int16)).view(torch.bfloat16).cuda()
    return dev(xdev)


class Layer:
    def __init__(self, B, cfg, E, H, I, shared=True, layer=0):
        self.E, self.H, self.I = E, H, I
        blob = synth.expert_blob(synth.rng_for(cfg, layer, 1), E, H, I)
        sh = synth.expert_blob(synth.rng_for(cfg, layer, 2), 1, H, I) if shared else None
        self.dev = B.Layer(dev(blob), dev(sh) if shared else None, E, H, I, synth.expert_stride(H, I))
        self.ref = O.ExpertBlob(blob, E, H, I, shared=sh)


def check_out(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref).max()
    rms = np.sqrt(np.mean(ref * ref))
    rel = np.linalg.norm(gpu - ref) / np.linalg.norm(ref)
    print(f"{what}: max|err| = {err:.3e}  rms(ref) = {rms:.3e}  ratio = {err / rms:.2e}  relL2 = {rel:.2e}")
    assert np.all(np.isfinite(gpu))
    assert err <= TOL * rms, (what, err, rms)
    return rel


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def route_both(B, logits, k, hist):
    ids, w = O.route_topk(logits, k)
    r = B.route(dev(logits), k, histogram=hist)
    torch.cuda.synchronize()
    return ids, w, r


def assert_route_exact(ids, w, r, E, hist):
    assert np.array_equal(r["topk_ids"].cpu().numpy(), ids)
    wg = r["topk_w"].cpu().numpy().astype(np.float64)
    assert np.abs(wg - w).max() <= 1e-6
    assert np.abs(wg.sum(axis=1) - 1.0).max() <= 1e-6
    if hist:
        counts, offsets, sp, pp = O.route_histogram(ids, E)
        assert np.array_equal(r["counts"].cpu().numpy(), counts)
        assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
        assert np.array_equal(r["sorted_pairs"].cpu().numpy(), sp)
        assert np.array_equal(r["pair_pos"].cpu().numpy(), pp)


# ------------------------------------------------------------------ routing --
ROUTE_CASES = [
    (1, 64, 4, "router"), (1, 512, 10, "router"), (3, 512, 10, "zipf"), (1024, 512, 10, "biased"),
    (37, 8, 3, "ties"), (300, 1024, 16, "normal"), (5, 16, 16, "ties"), (130, 64, 1, "normal"),
    (65, 512, 10, "const"), (32768, 512, 10, "zipf"),
    # chunk sizes 32 / 64 / 256 tokens, with and without the fused scan + scatter
    (4096, 512, 10, "biased"), (5000, 64, 4, "normal"), (70000, 64, 4, "normal"),
    # the single-launch histogram at its limit (one chunk, 256 pairs) and just past it
    (16, 64, 16, "ties"), (17, 64, 15, "ties"),
    # one token on 8 waves: ties across slices, two logits per lane, E not a
    # multiple of 64, k = E, slices left empty
    (1, 512, 10, "ties"), (1, 1024, 16, "ties"), (1, 300, 7, "normal"), (1, 16, 16, "ties"),
    (1, 8, 3, "const"), (1, 512, 10, "const"),
]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_bit_exact(B, T, E, k, kind):
    print(f"route T={T} E={E} k={k} {kind}", flush=True)
    rng = synth.rng_for(90, T, E)
    if kind == "router":
        _, xv = synth.activations(rng, T, 1024 if E == 64 else 3072, "f32")
        lg = synth.router_logits(rng, xv, E)
    elif kind == "zipf":
        lg = synth.zipf_logits(rng, T, E)
    elif kind == "biased":
        lg = synth.biased_logits(rng, rng.standard_normal((T, E)).astype(np.float32))
    elif kind == "ties":
        lg = synth.tie_logits(rng, T, E)
    elif kind == "const":
        lg = np.full((T, E), -0.0, dtype=np.float32)
        lg[::2, :] = 0.0
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    for hist in (False, True):
        ids, w, r = route_both(B, lg, k, hist)
        assert_route_exact(ids, w, r, E, hist)


# -------------------------------------------------------- router GEMV + top-k --
GEMV_CASES = [  # T, E, H, k, x dtype
    (1, 64, 1024, 4, "f32"), (1, 512, 3072, 10, "bf16"), (2, 512, 3072, 10, "bf16"),
    (3, 512, 3072, 10, "bf16"), (4, 512, 3072, 10, "f32"), (4, 1024, 512, 16, "bf16"),
    (2, 300, 768, 7, "f32"),
]


@pytest.mark.parametrize("T,E,H,k,xdt", GEMV_CASES)
def test_route_gemv_topk(B, T, E, H, k, xdt):
    """Logits bit-exact with the oracle's fp64 dot products rounded to
    float32, ids bit-exact, weights within 1e-6; two calls in a row on one
    workspace (its counter must come back to zero)."""
    print(f"router gemv T={T} E={E} H={H} k={k} {xdt}", flush=True)
    rng = synth.rng_for(60, T, E)
    xd, xv = synth.activations(rng, T, H, xdt)
    Wb = synth.router_weight(rng, E, H)
    ref_lg = O.router_logits(xv, synth.bf16_to_f32(Wb))
    ids, w = O.route_topk(ref_lg, k)
    Wt = torch.from_numpy(Wb.view(np.int16)).cuda()
    ws = B.workspace(B.MOE_OP_ROUTE_GEMV, T, E, k, H, 0)
    for rep in range(2):
        lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
        rid = torch.empty((T, k), dtype=torch.int32, device="cuda")
        rw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        B.moe_route_topk_gemv(dev_x(xd, xdt), Wt, k, rid, rw, lg, ws)
        torch.cuda.synchronize()
        assert np.array_equal(lg.cpu().numpy(), ref_lg), "logits differ"
        assert_route_exact(ids, w, {"topk_ids": rid, "topk_w": rw}, E, False)
    assert int(ws[:4].view(torch.int32)[0]) == 0
    # logits only (no top-k, no workspace)
    lg2 = torch.empty((T, E), dtype=torch.float32, device="cuda")
    B.moe_route_topk_gemv(dev_x(xd, xdt), Wt, k, None, None, lg2, None)
    torch.cuda.synchronize()
    assert np.array_equal(lg2.cpu().numpy(), ref_lg), "logits-only call differs"


def test_route_gemv_then_decode_matches_oracle(B, layer_full):
    """Router GEMV + top-k, then the decode layer: the whole decode path from
    activations and the router weight."""
    L = layer_full
    T = 2
    rng = synth.rng_for(61, 0, 0)
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    Wb = synth.router_weight(rng, 512, 3072)
    ids, w = O.route_topk(O.router_logits(xv, synth.bf16_to_f32(Wb)), 10)
    rid = torch.empty((T, 10), dtype=torch.int32, device="cuda")
    rw = torch.empty((T, 10), dtype=torch.float32, device="cuda")
    B.moe_route_topk_gemv(dev_x(xd, "bf16"), torch.from_numpy(Wb.view(np.int16)).cuda(), 10, rid, rw,
                          None, B.workspace(B.MOE_OP_ROUTE_GEMV, T, 512, 10, 3072, 0))
    out = run_decode(B, L, dev_x(xd, "bf16"), {"topk_ids": rid, "topk_w": rw})
    assert np.array_equal(rid.cpu().numpy(), ids)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), "router gemv + decode")
    # logits only, then the one-call decode that takes the top-k itself
    lg = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    B.moe_route_topk_gemv(dev_x(xd, "bf16"), torch.from_numpy(Wb.view(np.int16)).cuda(), 10, None, None,
                          lg, None)
    out2 = torch.empty((T, 3072), dtype=torch.float32, device="cuda")
    rid2 = torch.empty_like(rid)
    rw2 = torch.empty_like(rw)
    B.moe_expert_forward_decode_routed(L.dev, dev_x(xd, "bf16"), lg, 10, out2, rid2, rw2, None, 0,
                                       B.workspace(B.MOE_OP_DECODE, T, 512, 10, 3072, 768))
    torch.cuda.synchronize()
    assert np.array_equal(rid2.cpu().numpy(), ids)
    assert torch.equal(out2, out)


# ------------------------------------------------------------------- decode --
@pytest.fixture(scope="module")
def layer_small(B):
    return Layer(B, 0, 64, 1024, 256)


@pytest.fixture(scope="module")
def layer_full(B):
    return Layer(B, 1, 512, 3072, 768)


def run_decode(B, L, xt, r, out_dtype=torch.float32, residual=None, flags=0):
    T, k = r["topk_ids"].shape
    out = torch.empty((T, L.H), dtype=out_dtype, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, L.E, k, L.H, L.I)
    B.moe_expert_forward_decode(L.dev, xt, r["topk_ids"], r["topk_w"], out, residual, flags, ws)
    torch.cuda.synchronize()
    return out


def test_decode_small_config(B, layer_small):
    """One token, 64 experts top-4 + shared, H 1024, I 256, fp32 activations,
    router logits from a seeded bf16 router weight, seed 0."""
    L = layer_small
    rng = synth.rng_for(0, 0, 0)
    xd, xv = synth.activations(rng, 1, 1024, "f32")
    lg = synth.router_logits(rng, xv, 64)
    ids, w, r = route_both(B, lg, 4, False)
    assert_route_exact(ids, w, r, 64, False)
    out = run_decode(B, L, dev_x(xd, "f32"), r)
    ref = O.moe_layer(xv, ids, w, L.ref)
    check_out(to_np(out), ref, "decode cfg0")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_full_size(B, layer_full, T):
    L = layer_full
    rng = synth.rng_for(1, 0, 10 + T)
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    lg = synth.router_logits(rng, xv, 512) if T == 1 else synth.zipf_logits(rng, T, 512)
    ids, w, r = route_both(B, lg, 10, False)
    assert_route_exact(ids, w, r, 512, False)
    out = run_decode(B, L, dev_x(xd, "bf16"), r)
    ref = O.moe_layer(xv, ids, w, L.ref)
    check_out(to_np(out), ref, f"decode full T={T}")


def test_decode_prenorm_residual_bf16(B, layer_full):
    L = layer_full
    rng = synth.rng_for(1, 1, 20)
    T = 3
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    xv5 = xv * 5.0
    xd5 = synth.bf16_bits(xv5)
    lg = synth.zipf_logits(rng, T, 512)
    ids, w, r = route_both(B, lg, 10, False)
    res = (rng.standard_normal((T, 3072)) * 0.5).astype(np.float32)
    out = run_decode(B, L, dev_x(xd5, "bf16"), r, torch.float32, dev(res), B.MOE_FLAG_PRENORM_RMS)
    ref = O.moe_layer(xv5, ids, w, L.ref, prenorm=True, residual=res)
    check_out(to_np(out) - res, ref - res, "decode prenorm+residual")
    outb = run_decode(B, L, dev_x(xd5, "bf16"), r, torch.bfloat16,
                      dev(res).to(torch.bfloat16), B.MOE_FLAG_PRENORM_RMS)
    resb = synth.bf16_to_f32(synth.bf16_bits(res)).astype(np.float64)
    refb = O.moe_layer(xv5, ids, w, L.ref, prenorm=True, residual=resb)
    check_out(to_np(outb), refb, "decode bf16 out")


@pytest.mark.parametrize("T", [4, 8])
def test_decode_duplicates_and_no_shared(B, T):
    """Tokens sharing experts (slot dedup) and a layer without shared expert;
    at T = 8 the 128 pairs are deduplicated in two groups of 64."""
    L = Layer(B, 5, 16, 512, 256, shared=False)
    k = 16
    rng = synth.rng_for(5, 0, T - 1)
    xd, xv = synth.activations(rng, T, 512, "f32")
    lg = synth.tie_logits(rng, T, 16)
    ids, w, r = route_both(B, lg, k, False)
    out = run_decode(B, L, dev_x(xd, "f32"), r)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), "decode dup/no-shared")


def test_decode_deterministic(B, layer_full):
    L = layer_full
    rng = synth.rng_for(1, 2, 30)
    xd, xv = synth.activations(rng, 2, 3072, "bf16")
    _, _, r = route_both(B, synth.zipf_logits(rng, 2, 512), 10, False)
    a = run_decode(B, L, dev_x(xd, "bf16"), r)
    b = run_decode(B, L, dev_x(xd, "bf16"), r)
    assert torch.equal(a, b)


# ------------------------------------------------------- routed decode call --
ROUTED_CASES = [
    # (layer: seed, E, H, I), T, k, logits kind, x dtype
    ((0, 64, 1024, 256), 1, 4, "router", "f32"),
    ((1, 512, 3072, 768), 1, 10, "router", "bf16"),
    ((1, 512, 3072, 768), 1, 10, "ties", "bf16"),      # block-wide top-k, ties across slices
    ((7, 1024, 512, 256), 1, 16, "ties", "f32"),
    ((8, 300, 512, 512), 1, 7, "normal", "f32"),       # slices not a multiple of 64
    ((9, 16, 512, 256), 1, 16, "ties", "f32"),         # k = E: one wave holds every expert
    ((1, 512, 3072, 768), 2, 10, "zipf", "bf16"),
    ((1, 512, 3072, 768), 3, 10, "zipf", "bf16"),
    ((1, 512, 3072, 768), 4, 10, "ties", "bf16"),
    ((1, 512, 3072, 768), 6, 10, "zipf", "f32"),
    ((1, 512, 3072, 768), 8, 10, "zipf", "bf16"),      # 8 routing waves, 80 pairs
    ((7, 1024, 512, 256), 4, 16, "normal", "f32"),     # top-k with 16 experts per lane
    ((7, 1024, 512, 256), 8, 16, "normal", "bf16"),    # 128 pairs, up to 129 slots
    ((8, 300, 512, 512), 2, 7, "normal", "bf16"),      # E not a multiple of 64
]


@pytest.fixture(scope="module")
def routed_layers(B, layer_small, layer_full):
    cache = {(0, 64, 1024, 256): layer_small, (1, 512, 3072, 768): layer_full}

    def get(key):
        if key not in cache:
            cache[key] = Layer(B, *key)
        return cache[key]
    return get


@pytest.mark.parametrize("lkey,T,k,kind,xdt", ROUTED_CASES)
def test_decode_routed(B, routed_layers, lkey, T, k, kind, xdt):
    """moe_expert_forward_decode_routed: routing bit-exact against the oracle
    and identical to moe_route_topk's; output within tolerance of the oracle
    and bitwise equal to the two-call path on the same routing."""
    L = routed_layers(lkey)
    E, H = L.E, L.H
    print(f"routed decode E={E} H={H} T={T} k={k} {kind}", flush=True)
    rng = synth.rng_for(40, T, E)
    xd, xv = synth.activations(rng, T, H, xdt)
    if kind == "router":
        lg = synth.router_logits(rng, xv, E)
    elif kind == "zipf":
        lg = synth.zipf_logits(rng, T, E)
    elif kind == "ties":
        lg = synth.tie_logits(rng, T, E)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    xt = dev_x(xd, xdt)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rid = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, E, k, H, L.I)
    B.moe_expert_forward_decode_routed(L.dev, xt, dev(lg), k, out, rid, rw, None, 0, ws)
    torch.cuda.synchronize()
    assert_route_exact(ids, w, {"topk_ids": rid, "topk_w": rw}, E, False)
    r = B.route(dev(lg), k)
    assert torch.equal(r["topk_ids"], rid) and torch.equal(r["topk_w"], rw)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), f"routed decode T={T} E={E}")
    two = run_decode(B, L, xt, r)
    assert torch.equal(out, two)
    # routing outputs are optional
    out2 = torch.empty_like(out)
    B.moe_expert_forward_decode_routed(L.dev, xt, dev(lg), k, out2, None, None, None, 0, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("T,k", [(1, 1), (1, 16), (2, 3), (3, 16)])
def test_no_shared_expert_and_extreme_k(B, T, k):
    """A layer without a shared expert, with one selected expert per token and
    with every expert selected (k = E): routed decode, the two-call decode and
    prefill against the oracle; the two decode forms bitwise equal."""
    L = Layer(B, 9, 16, 512, 256, shared=False)
    print(f"no shared expert T={T} k={k}", flush=True)
    rng = synth.rng_for(42, T, k)
    xd, xv = synth.activations(rng, T, 512, "f32")
    lg = rng.standard_normal((T, 16)).astype(np.float32)
    ids, w = O.route_topk(lg, k)
    ref = O.moe_layer(xv, ids, w, L.ref)
    xt = dev_x(xd, "f32")
    out = torch.empty((T, 512), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, 16, k, 512, 256)
    B.moe_expert_forward_decode_routed(L.dev, xt, dev(lg), k, out, None, None, None, 0, ws)
    torch.cuda.synchronize()
    check_out(to_np(out), ref, f"routed decode, no shared, T={T} k={k}")
    _, _, r = route_both(B, lg, k, True)
    assert torch.equal(run_decode(B, L, xt, r), out)
    check_out(to_np(run_prefill(B, L, xt, r)), ref, f"prefill, no shared, T={T} k={k}")


def test_decode_routed_prenorm_residual_bf16(B, layer_full):
    L = layer_full
    rng = synth.rng_for(41, 0, 0)
    T = 2
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    lg = synth.zipf_logits(rng, T, 512)
    ids, w = O.route_topk(lg, 10)
    res = (rng.standard_normal((T, 3072)) * 0.5).astype(np.float32)
    resd = dev(res).to(torch.bfloat16)
    out = torch.empty((T, 3072), dtype=torch.bfloat16, device="cuda")
    ws = B.workspace(B.MOE_OP_DECODE, T, 512, 10, 3072, 768)
    B.moe_expert_forward_decode_routed(L.dev, dev_x(xd, "bf16"), dev(lg), 10, out, None, None, resd,
                                       B.MOE_FLAG_PRENORM_RMS, ws)
    torch.cuda.synchronize()
    resb = synth.bf16_to_f32(synth.bf16_bits(res)).astype(np.float64)
    ref = O.moe_layer(xv, ids, w, L.ref, prenorm=True, residual=resb)
    check_out(to_np(out), ref, "routed decode prenorm+residual bf16")


# ------------------------------------------------------------------ prefill --
def run_prefill(B, L, xt, r, out_dtype=torch.float32, residual=None, flags=0):
    T, k = r["topk_ids"].shape
    out = torch.empty((T, L.H), dtype=out_dtype, device="cuda")
    ws = B.workspace(B.MOE_OP_PREFILL, T, L.E, k, L.H, L.I)
    B.moe_expert_forward_prefill(L.dev, xt, r["topk_ids"], r["topk_w"], r["counts"], r["offsets"],
                                 r["sorted_pairs"], r["pair_pos"], out, residual, flags, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [1, 5, 37, 200])
def test_prefill_small(B, T):
    """8 experts top-3, H 512, I 256: several 64-row items per expert, ragged
    tails, empty experts at small T."""
    L = Layer(B, 6, 8, 512, 256)
    rng = synth.rng_for(6, T, 1)
    xd, xv = synth.activations(rng, T, 512, "bf16")
    lg = rng.standard_normal((T, 8)).astype(np.float32)
    ids, w, r = route_both(B, lg, 3, True)
    assert_route_exact(ids, w, r, 8, True)
    out = run_prefill(B, L, dev_x(xd, "bf16"), r)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), f"prefill small T={T}")


@pytest.mark.parametrize("I", [512, 1024, 2048])
def test_prefill_intermediate_widths(B, I):
    """Every token at I = 512 (h resident in LDS), 1024 and 2048 (h streamed
    through the down GEMM tile by tile): 8 experts top-3, H 512."""
    L = Layer(B, 13, 8, 512, I)
    T = 90
    rng = synth.rng_for(13, T, I)
    xd, xv = synth.activations(rng, T, 512, "bf16")
    lg = rng.standard_normal((T, 8)).astype(np.float32)
    ids, w, r = route_both(B, lg, 3, True)
    out = run_prefill(B, L, dev_x(xd, "bf16"), r)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), f"prefill I={I}")


def test_prefill_small_config_all_tokens(B, layer_small):
    L = layer_small
    rng = synth.rng_for(0, 1, 0)
    T = 96
    xd, xv = synth.activations(rng, T, 1024, "f32")
    lg = synth.router_logits(rng, xv, 64)
    ids, w, r = route_both(B, lg, 4, True)
    res = rng.standard_normal((T, 1024)).astype(np.float32)
    out = run_prefill(B, L, dev_x(xd, "f32"), r, torch.float32, dev(res), B.MOE_FLAG_PRENORM_RMS)
    ref = O.moe_layer(xv, ids, w, L.ref, prenorm=True, residual=res)
    check_out(to_np(out) - res, ref - res, "prefill cfg0 shapes prenorm+residual")


@pytest.mark.parametrize("H,xdt,odt", [(1024, "bf16", torch.bfloat16), (4096, "f32", torch.bfloat16),
                                        (8192, "bf16", torch.float32)])
def test_prefill_widths_dtypes_residual(B, H, xdt, odt):
    """Every x-row staging width (H/512 chunks per lane: <= 2, <= 6, <= 16),
    fp32 and bf16 x, bf16 and fp32 out, pre-norm and a residual in the
    output dtype."""
    L = Layer(B, 8, 8, H, 256)
    T = 45
    rng = synth.rng_for(8, T, H)
    xd, xv = synth.activations(rng, T, H, xdt)
    ids, w, r = route_both(B, rng.standard_normal((T, 8)).astype(np.float32), 3, True)
    res = (rng.standard_normal((T, H)) * 0.5).astype(np.float32)
    if odt == torch.bfloat16:
        resd = dev(res).to(torch.bfloat16)
        res = synth.bf16_to_f32(synth.bf16_bits(res)).astype(np.float64)
    else:
        resd = dev(res)
    out = run_prefill(B, L, dev_x(xd, xdt), r, odt, resd, B.MOE_FLAG_PRENORM_RMS)
    ref = O.moe_layer(xv, ids, w, L.ref, prenorm=True, residual=res)
    if odt == torch.bfloat16:
        check_out(to_np(out), ref, f"prefill H={H} x {xdt} bf16 out + residual")
    else:
        check_out(to_np(out) - res, ref - res, f"prefill H={H} x {xdt} fp32 out + residual")


def test_decode_prefill_agree(B, layer_full):
    L = layer_full
    rng = synth.rng_for(1, 3, 40)
    T = 3
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    ids, w, r = route_both(B, synth.zipf_logits(rng, T, 512), 10, True)
    a = to_np(run_decode(B, L, dev_x(xd, "bf16"), r))
    b = to_np(run_prefill(B, L, dev_x(xd, "bf16"), r))
    ref = O.moe_layer(xv, ids, w, L.ref)
    check_out(a, ref, "decode")
    check_out(b, ref, "prefill")
    rms = np.sqrt(np.mean(ref * ref))
    assert np.abs(a - b).max() <= 1e-2 * rms


def _prefill_check(B, L, T, kind, seed, pick=None, flags=0):
    """One prefill call at the 512-expert layer's widths (the call the
    benchmark makes), run twice (bitwise equal); the tokens `pick(ids,
    hist)` returns -- every token when pick is None -- against the oracle."""
    rng = synth.rng_for(3, seed, T)
    xd, xv = synth.activations(rng, T, 3072, "bf16")
    if kind == "biased":
        lg = synth.biased_logits(rng, synth.router_logits(rng, xv[:, :], 512))
    else:
        lg = synth.zipf_logits(rng, T, 512)
    ids, w, r = route_both(B, lg, 10, True)
    assert_route_exact(ids, w, r, 512, True)
    out = run_prefill(B, L, dev_x(xd, "bf16"), r, flags=flags)
    a = run_prefill(B, L, dev_x(xd, "bf16"), r, flags=flags)
    assert torch.equal(out, a)   # deterministic
    if pick is None:
        ref = O.moe_layer(xv, ids, w, L.ref, prenorm=bool(flags))
        check_out(to_np(out), ref, f"prefill T={T} {kind} every token")
        return
    toks = np.unique(np.concatenate([[0, T - 1], pick(ids, O.route_histogram(ids, 512))]))
    ref = O.moe_layer(xv, ids, w, L.ref, prenorm=bool(flags), tokens=toks)
    check_out(to_np(out[torch.from_numpy(toks).cuda()]), ref, f"prefill T={T} {kind}, {toks.size} tokens")


def expert_order_tokens(ids, hist, T, k, E, row_blocks, rows_per_item=64):
    """Tokens that the chunks longer than 4096 tokens place at the edges of
    their work: every row of the most loaded expert's first and last 64-row
    items, and the first and last row of the first and last item of each
    XCD's contiguous range of (item, row block) units, for each GEMM's count
    of row blocks per item (items in expert order, the shared expert's T
    rows last)."""
    counts, offsets, sp, _ = hist
    items = []                                      # (first sorted row, rows)
    for e in range(E):
        for g in range(0, int(counts[e]), rows_per_item):
            items.append((int(offsets[e]) + g, min(rows_per_item, int(counts[e]) - g)))
    for g in range(0, T, rows_per_item):
        items.append((T * k + g, min(rows_per_item, T - g)))

    def tok(row):
        return int(sp[row]) // k if row < T * k else row - T * k

    picked = set()
    head = int(np.argmax(counts))
    first = int(offsets[head])
    last = first + (int(counts[head]) - 1) // rows_per_item * rows_per_item
    for r0 in (first, last):
        n = min(rows_per_item, first + int(counts[head]) - r0)
        picked.update(tok(r) for r in range(r0, r0 + n))
    for RB in row_blocks:
        units = len(items) * RB
        per = (units + 7) // 8
        for x in range(8):
            for u in (x * per, min((x + 1) * per, units) - 1):
                if 0 <= u < units:
                    r0, n = items[u // RB]
                    picked.update((tok(r0), tok(r0 + n - 1)))
    return np.array(sorted(picked))


@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_residual_in_place(B, layer_small, odt):
    """residual may be the output buffer itself (the residual stream updated
    in place): routed decode and prefill against the oracle with that
    residual.  The expert part (out - residual) is held to the usual bound,
    TOL * rms of the oracle's expert part; a bf16 output may in addition
    differ by its own rounding, at most half a bf16 ulp, 2^-9 |value|."""
    L = layer_small
    for T, what in ((3, "decode"), (100, "prefill")):
        print(f"in-place residual {what} T={T} {odt}", flush=True)
        rng = synth.rng_for(46, T, int(odt == torch.bfloat16))
        xd, xv = synth.activations(rng, T, 1024, "f32")
        lg = rng.standard_normal((T, 64)).astype(np.float32)
        ids, w = O.route_topk(lg, 4)
        res = (rng.standard_normal((T, 1024)) * 0.5).astype(np.float32)
        buf = dev(res).to(odt)
        resv = buf.float().cpu().numpy().astype(np.float64)
        if what == "decode":
            ws = B.workspace(B.MOE_OP_DECODE, T, 64, 4, 1024, 256)
            B.moe_expert_forward_decode_routed(L.dev, dev_x(xd, "f32"), dev(lg), 4, buf, None, None, buf, 0, ws)
        else:
            _, _, r = route_both(B, lg, 4, True)
            ws = B.workspace(B.MOE_OP_PREFILL, T, 64, 4, 1024, 256)
            B.moe_expert_forward_prefill(L.dev, dev_x(xd, "f32"), r["topk_ids"], r["topk_w"], r["counts"],
                                         r["offsets"], r["sorted_pairs"], r["pair_pos"], buf, buf, 0, ws)
        torch.cuda.synchronize()
        ref = O.moe_layer(xv, ids, w, L.ref, residual=resv)
        got = to_np(buf)
        moe_rms = np.sqrt(np.mean((ref - resv) ** 2))
        err = np.abs(got - ref)
        print(f"in-place residual {what} {odt}: max|err| = {err.max():.3e}  rms(expert part) = {moe_rms:.3e}")
        assert np.all(np.isfinite(got))
        rounding = np.abs(ref) * 2.0 ** -9 if odt == torch.bfloat16 else 0.0
        assert np.all(err <= TOL * moe_rms + rounding), (what, odt, float(err.max()), moe_rms)


@pytest.mark.parametrize("E,k,T", [(1024, 16, 300), (300, 7, 129)])
def test_prefill_expert_counts(B, E, k, T):
    """Prefill with the largest expert count (five experts per thread of the
    work-item scan) and with a count that is not a multiple of 64, every
    token against the oracle."""
    L = Layer(B, 12, E, 512, 256)
    print(f"prefill E={E} k={k} T={T}", flush=True)
    rng = synth.rng_for(45, E, T)
    xd, xv = synth.activations(rng, T, 512, "f32")
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, r = route_both(B, lg, k, True)
    assert_route_exact(ids, w, r, E, True)
    out = run_prefill(B, L, dev_x(xd, "f32"), r)
    check_out(to_np(out), O.moe_layer(xv, ids, w, L.ref), f"prefill E={E} k={k} T={T}")


@pytest.mark.parametrize("T,shared", [(4096, True), (4096, False), (4097, False), (5000, True)])
def test_prefill_item_orders(B, T, shared):
    """Both work-item orders of the prefill kernels: lists in size order dealt
    to the XCDs in turn (chunks of up to 4096 tokens) and lists in expert
    order split into contiguous ranges (longer chunks), with and without a
    shared expert; Zipf routing gives one expert many 64-row items.  Every
    token against the oracle."""
    L = Layer(B, 11, 64, 1024, 256, shared=shared)
    print(f"prefill item order T={T} shared={shared}", flush=True)
    rng = synth.rng_for(44, T, int(shared))
    xd, xv = synth.activations(rng, T, 1024, "bf16")
    lg = synth.zipf_logits(rng, T, 64)
    ids, w, r = route_both(B, lg, 4, True)
    assert_route_exact(ids, w, r, 64, True)
    out = run_prefill(B, L, dev_x(xd, "bf16"), r)
    ref = O.moe_layer(xv, ids, w, L.ref)
    check_out(to_np(out), ref, f"prefill T={T} shared={shared} every token")


def test_prefill_1024_biased_every_token(B, layer_full):
    """The 1024-token chunk with the skewed router (bias N(0, 0.5)): every
    token of the whole chunk against the oracle."""
    _prefill_check(B, layer_full, 1024, "biased", 0)


def test_prefill_32768_zipf(B, layer_full):
    """A 32768-token Zipf chunk with the pre-norm: every row of the most
    loaded expert's first and last items, the edges of every XCD's range of
    work for both GEMM kernels (6 and 12 row blocks per item), and 16 more
    random tokens, against the oracle."""
    def pick(ids, hist):
        rng = np.random.default_rng(5)
        edge = expert_order_tokens(ids, hist, 32768, 10, 512, (768 // 128, 3072 // 256))
        return np.concatenate([edge, rng.choice(32768, 16, replace=False)])
    _prefill_check(B, layer_full, 32768, "zipf", 1, pick=pick, flags=1)


def test_graph_replay_matches_eager(B, layer_full):
    """route + decode and route + prefill captured in one HIP graph, replayed
    several times with eager work and synchronisations in between; every
    replay must give the eager bytes."""
    L = layer_full
    rng = synth.rng_for(1, 7, 50)
    xd, xv = synth.activations(rng, 64 + 2, 3072, "bf16")
    x_dec = dev_x(xd[:2], "bf16")
    x_pre = dev_x(xd[2:], "bf16")
    lg_dec = dev(synth.zipf_logits(rng, 2, 512))
    lg_pre = dev(synth.zipf_logits(rng, 64, 512))
    rd = {n: torch.empty(s, dtype=d, device="cuda") for n, s, d in [
        ("ids", (2, 10), torch.int32), ("w", (2, 10), torch.float32)]}
    rp = {n: torch.empty(s, dtype=d, device="cuda") for n, s, d in [
        ("ids", (64, 10), torch.int32), ("w", (64, 10), torch.float32), ("counts", (512,), torch.int32),
        ("offsets", (513,), torch.int32), ("sp", (640,), torch.int32), ("pp", (640,), torch.int32)]}
    out_d = torch.empty((2, 3072), dtype=torch.float32, device="cuda")
    out_p = torch.empty((64, 3072), dtype=torch.float32, device="cuda")
    ws_d = B.workspace(B.MOE_OP_DECODE, 2, 512, 10, 3072, 768)
    ws_r = B.workspace(B.MOE_OP_ROUTE, 64, 512, 10, 3072, 768)
    ws_p = B.workspace(B.MOE_OP_PREFILL, 64, 512, 10, 3072, 768)

    def step():
        B.moe_route_topk(lg_dec, 10, rd["ids"], rd["w"])
        B.moe_expert_forward_decode(L.dev, x_dec, rd["ids"], rd["w"], out_d, None, 0, ws_d)
        B.moe_route_topk(lg_pre, 10, rp["ids"], rp["w"], rp["counts"], rp["offsets"], rp["sp"],
                         rp["pp"], ws_r)
        B.moe_expert_forward_prefill(L.dev, x_pre, rp["ids"], rp["w"], rp["counts"], rp["offsets"],
                                     rp["sp"], rp["pp"], out_p, None, 0, ws_p)

    step()
    torch.cuda.synchronize()
    ref_d, ref_p = out_d.clone(), out_p.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                     # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out_d.zero_()
        out_p.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, ref_d), f"decode replay {r}"
        assert torch.equal(out_p, ref_p), f"prefill replay {r}"
        del junk
