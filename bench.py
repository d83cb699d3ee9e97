#!/usr/bin/env python3
"""Benchmark of the routed-MoE expert layer on 2-bit weights (one MI355X).

A step is one MoE layer for one batch of synthetic input through the HIP
library: router top-k and the expert layer.  The headline workload is the
decode step of one token on a 512-expert layer (top-10 + 1 shared, hidden
3072, intermediate 768, 2,211,840 bytes per expert) through
moe_expert_forward_decode_routed (top-k inside the expert kernels); the same
run also measures that step as two calls (moe_route_topk, then
moe_expert_forward_decode), verify windows of 2 and 3 tokens and a
1024-token prefill chunk (router histogram + grouped expert GEMMs + combine)
and reports them in the same JSON line.  Weights rotate over 16 distinct layers (about 18 GB) so
that no step finds its experts in the 256 MB last-level cache.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits with
an error: the library runs the layer on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA, TFLOP/s

E, H, I, K = 512, 3072, 768, 10
EXPERT_BYTES = 3 * I * H * 5 // 16      # 2,211,840
MAT_BYTES = I * H * 5 // 16             # 737,280


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--prefill-steps", type=int, default=80)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default="",
                    help="decode1|decode1_two_calls|decode1_gemv|decode2|decode3|prefill|prefill32768|"
                         "tiered|tiered_device|tiered_host|windows|stack (profiling runs)")
    ap.add_argument("--stack-layers", type=int, default=48,
                    help="layers of the stacked decode/prefill runs (0 = skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--counters", nargs="?", const="decode1", default=None,
                    choices=["decode1", "prefill1024", "prefill32768"],
                    help="eager steps of one case only, 1-token decode by default (hardware-counter runs)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the device-ceiling microbenchmarks (moe_ceilings)")
    return ap.parse_args()


_T0 = time.time()


def progress(msg: str):
    """One line on stderr per finished case (the JSON line goes to stdout)."""
    print(f"bench: {msg} ({time.time() - _T0:.1f} s)", file=sys.stderr, flush=True)


def case_steps(steps: int) -> dict:
    """Timed steps of the secondary cases for `--steps K` (the headline case
    times exactly K): at least one each."""
    return {"half": max(1, steps // 2), "windows": max(32, steps // 8)}


def step_plan(n_steps: int, warmup: int) -> dict:
    """Rows (per-step inputs and routing outputs) that each phase of a case
    uses: eager warmup, eager timing, the untimed warm graph, the graph-timed
    region (exactly n_steps steps) and the hooked per-kernel pass.  The warm
    and timed graphs cover different rows, so the timed steps run other
    rotating layers than the ones just before them."""
    if n_steps < 1 or warmup < 0:
        raise ValueError("need n_steps >= 1 and warmup >= 0")
    w, k = warmup, n_steps
    return {"warmup": range(0, w), "eager_timed": range(w, w + k), "graph_warm": range(w, w + k),
            "graph_timed": range(w + k, w + 2 * k), "hooked": range(w + 2 * k, w + 3 * k)}


def rows_needed(n_steps: int, warmup: int) -> int:
    """Rows a case must allocate: one past the last index step_plan uses."""
    return max(r.stop for r in step_plan(n_steps, warmup).values())


def device_ceilings():
    """Streaming-read, dispatch, MFMA and dequant ceilings measured by the
    moe_ceilings program (a child process, run before this process touches
    the GPU); None when it is not built or fails."""
    import subprocess
    exe = os.path.join(ROOT, "bit_quantized_expert_router_amd", "moe_ceilings")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    except subprocess.TimeoutExpired:
        return None
    if r.returncode != 0:
        print(f"bench.py: moe_ceilings failed: {r.stderr.strip()[-300:]}", file=sys.stderr)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs the MoE layer on one GPU only; "
              "--gpus must be 1 (no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    if args.counters:
        counters_run(args)
        return

    ceilings = None if (args.no_ceilings or args.only) else device_ceilings()
    progress("ceilings")

    import torch
    from bit_quantized_expert_router_amd import binding as B
    from bit_quantized_expert_router_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---------------------------------------------------------------- weights
    t0 = time.time()
    layers = []
    for l in range(args.layers):
        ex = synth.device_expert_blob(E, H, I, synth.torch_seed(1, l, 1), dev)
        sh = synth.device_expert_blob(1, H, I, synth.torch_seed(1, l, 2), dev)
        layers.append(B.Layer(ex, sh, E, H, I, synth.expert_stride(H, I)))
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    progress(f"{args.layers} layers of weights generated")

    results = {}
    prof_kernels = {}

    def timed(fn, idx):
        """Eager steps fn(i) for i in idx (a range), bracketed by events on
        the stream the library launches on; ms per step."""
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in idx:
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / len(idx)

    spread = {}

    def capture(fn, idx):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in idx:
                fn(i)
        return g

    def graphed(fn, plan, extra_replays=4):
        """The timed region: plan["graph_timed"] (exactly the K timed steps)
        captured into one HIP graph and replayed once between a
        synchronisation on each side, after one untimed replay of a graph
        over plan["graph_warm"] (the K steps before, on other rotating
        layers, so the timed steps do not find their weights in the
        last-level cache).  Returns ms per step; `spread` receives the 10th,
        50th and 90th percentiles of ms per step over the timed replay and
        `extra_replays` more, each preceded by a replay of the warm graph."""
        torch.cuda.synchronize()
        gw = capture(fn, plan["graph_warm"])
        gt = capture(fn, plan["graph_timed"])
        n = len(plan["graph_timed"])
        gw.replay()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        gt.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / n
        per = [ms]
        for _ in range(extra_replays):
            gw.replay()
            ev0.record()
            gt.replay()
            ev1.record()
            torch.cuda.synchronize()
            per.append(ev0.elapsed_time(ev1) / n)
        spread.clear()
        spread.update({"ms_per_layer_p10": float(np.percentile(per, 10)),
                       "ms_per_layer_p50": float(np.percentile(per, 50)),
                       "ms_per_layer_p90": float(np.percentile(per, 90)), "replays": len(per)})
        del gw, gt
        return ms

    def hooked(fn, idx):
        """Same steps again with the library's per-kernel hipEvent hooks on
        (each launch's events stamped with its dispatch's begin and end)."""
        torch.cuda.synchronize()
        B.profile_reset()
        B.profile_enable(True)
        for i in idx:
            fn(i)
        torch.cuda.synchronize()
        B.profile_enable(False)
        return {k: v for k, v in B.profile_results().items() if v[0] > 0}

    def run_phases(step, n_steps, warmup):
        """Eager warmup, eager timing, the graph-timed region and the hooked
        pass of one case, on the rows step_plan assigns to each."""
        plan = step_plan(n_steps, warmup)
        for i in plan["warmup"]:
            step(i)
        ms_eager = timed(step, plan["eager_timed"])
        ms = graphed(step, plan)
        pct = dict(spread)
        kern = hooked(step, plan["hooked"])
        return plan, ms, ms_eager, pct, kern

    # ---------------------------------------------------------------- decode
    def decode_case(T, kind, n_steps, warmup, routed=True, gemv=False):
        total = rows_needed(n_steps, warmup)
        rng = synth.rng_for(1, 100 + T, 0)
        xd, xv = synth.activations(rng, min(total, 64) * T, H, "bf16")
        xs = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev).view(-1, T, H)
        nx = xs.shape[0]
        if kind == "router":
            lg = synth.router_logits(rng, np.tile(xv, (1, 1))[: nx * T], E).reshape(nx, T, E)
            lg = np.concatenate([lg] * ((total + nx - 1) // nx))[:total]
        else:
            lg = synth.zipf_logits(rng, total * T, E).reshape(total, T, E)
        logits = torch.from_numpy(np.ascontiguousarray(lg)).to(dev)
        ids = torch.empty((total, T, K), dtype=torch.int32, device=dev)
        wts = torch.empty((total, T, K), dtype=torch.float32, device=dev)
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = B.workspace(B.MOE_OP_DECODE, T, E, K, H, I, dev)
        if gemv:         # router weights (bf16 [E, H]) per rotating layer
            wr = [(torch.randn((E, H), device=dev) / np.sqrt(H)).to(torch.bfloat16)
                  for _ in range(len(layers))]
            lgg = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(2)]

        def step(i):
            L = layers[i % len(layers)]
            if gemv:     # router logits GEMV, then the one-call expert layer (top-k inside)
                B.moe_route_topk_gemv(xs[i % nx], wr[i % len(layers)], K, None, None, lgg[i % 2], None)
                B.moe_expert_forward_decode_routed(L, xs[i % nx], lgg[i % 2], K, out, ids[i], wts[i],
                                                   None, 0, ws)
            elif routed:   # one call: top-k inside the expert kernels
                B.moe_expert_forward_decode_routed(L, xs[i % nx], logits[i], K, out, ids[i], wts[i],
                                                   None, 0, ws)
            else:        # moe_route_topk, then the expert layer
                B.moe_route_topk(logits[i], K, ids[i], wts[i])
                B.moe_expert_forward_decode(L, xs[i % nx], ids[i], wts[i], out, None, 0, ws)

        plan, ms, ms_eager, pct, kern = run_phases(step, n_steps, warmup)
        idh = ids.cpu().numpy()
        distinct = np.array([len(np.unique(idh[i])) for i in range(total)])
        # routed experts + the shared one, over the graph-timed steps (the
        # headline) and over the hooked steps (the per-kernel times)
        slots = distinct[list(plan["graph_timed"])].mean() + 1
        slots_hook = distinct[list(plan["hooked"])].mean() + 1
        wbytes = slots * EXPERT_BYTES
        io = T * H * 2 + T * H * 4 + T * E * 4 + T * K * 8
        step_bytes = wbytes + io
        gu = kern.get("decode_gateup_kernel", (1, float("nan")))
        dn = kern.get("decode_down_kernel", (1, float("nan")))
        gu_ms = gu[1] / gu[0]
        kms = {"decode_gateup": gu_ms, "decode_down": dn[1] / dn[0]}
        if "route_topk_kernel" in kern:
            rt = kern["route_topk_kernel"]
            kms = {"route_topk": rt[1] / rt[0], **kms}
        if "route_gemv_topk_kernel" in kern:
            rt = kern["route_gemv_topk_kernel"]
            kms = {"route_gemv_topk": rt[1] / rt[0], **kms}
        gu_bytes = slots_hook * 2 * MAT_BYTES + T * H * 2 + (T * K + T) * I * 2   # weights, x, h
        return {
            "T": T, "routing": kind,
            "calls": ("route_topk_gemv (logits) + decode_routed (router GEMV included)" if gemv else
                      "decode_routed" if routed else "route_topk+decode"),
            "launch": "hip_graph", "ms_per_layer": ms, **pct,
            "ms_per_layer_eager": ms_eager, "tokens_per_s": T * 1000.0 / ms,
            "tokens_per_s_eager": T * 1000.0 / ms_eager,
            "distinct_experts_per_step": float(slots - 1),
            "algorithmic_bytes_per_step": float(step_bytes),
            "GBps": step_bytes / ms / 1e6, "hbm_frac": step_bytes / ms / 1e6 / HBM_PEAK_GBS,
            "kernel_ms": kms,
            "gateup_bytes_per_launch": float(gu_bytes),
            "gateup_GBps": gu_bytes / gu_ms / 1e6,
        }

    # --------------------------------------------------------------- prefill
    def prefill_case(T, n_steps, warmup, routing="biased"):
        rng = synth.rng_for(3, 0, T)
        nvar = 4 if routing == "biased" else 2
        xd, xv = synth.activations(rng, nvar * T, H, "bf16")
        xs = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev).view(nvar, T, H)
        if routing == "biased":
            lgs = [synth.biased_logits(rng, synth.router_logits(rng, xv[v * T:(v + 1) * T], E))
                   for v in range(nvar)]
        else:
            lgs = [synth.zipf_logits(rng, T, E) for v in range(nvar)]
        logits = torch.from_numpy(np.stack(lgs)).to(dev)
        r = {n: torch.empty(s, dtype=dt, device=dev) for n, s, dt in [
            ("ids", (T, K), torch.int32), ("w", (T, K), torch.float32), ("counts", (E,), torch.int32),
            ("offsets", (E + 1,), torch.int32), ("sp", (T * K,), torch.int32),
            ("pp", (T * K,), torch.int32)]}
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        wsr = B.workspace(B.MOE_OP_ROUTE, T, E, K, H, I, dev)
        ws = B.workspace(B.MOE_OP_PREFILL, T, E, K, H, I, dev)

        def step(i):
            L = layers[i % len(layers)]
            v = i % nvar
            B.moe_route_topk(logits[v], K, r["ids"], r["w"], r["counts"], r["offsets"], r["sp"],
                             r["pp"], wsr)
            B.moe_expert_forward_prefill(L, xs[v], r["ids"], r["w"], r["counts"], r["offsets"],
                                         r["sp"], r["pp"], out, None, 0, ws)

        plan, ms, ms_eager, pct, kern = run_phases(step, n_steps, warmup)
        nonempty = []
        for v in range(nvar):
            ids_v = torch.topk(logits[v], K, dim=1).indices.cpu().numpy()
            nonempty.append(len(np.unique(ids_v)))
        ne = float(np.mean(nonempty))
        wbytes = (ne + 1) * EXPERT_BYTES
        step_bytes = wbytes + T * H * 2 + T * H * 4 + T * E * 4
        flops = (T * K + T) * 2 * 3 * H * I
        kms = {k.replace("_kernel", ""): v[1] / v[0] for k, v in kern.items()}
        gemm_ms = kms.get("prefill_gateup", 0) + kms.get("prefill_down", 0)
        gu_ms = kms.get("prefill_gateup", float("nan"))
        gu_flops = (T * K + T) * 2 * 2 * H * I
        gu_bytes = (ne + 1) * 2 * MAT_BYTES + T * H * 2 + (T * K + T) * I * 2   # weights, x, h
        if T > 4096:   # long chunks: the gate/up kernel is bound by the MFMA rate
            roof = {"bound": "mfma", "kernel": "prefill_gateup_kernel",
                    "achieved": round(gu_flops / gu_ms / 1e9, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(gu_flops / gu_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                    "traffic": pmc_traffic("prefill_gateup_T32768_pmc_traffic.txt", "prefill_gateup_kernel"),
                    "algorithmic_flops_per_launch": float(gu_flops),
                    "kernel_us": round(gu_ms * 1e3, 2), "hbm_GBps": round(gu_bytes / gu_ms / 1e6, 1)}
            return {
                "T": T, "routing": "zipf(1.1)", "launch": "hip_graph", "ms_per_layer": ms, **pct,
                "ms_per_layer_eager": ms_eager, "tokens_per_s": T * 1000.0 / ms,
                "nonempty_experts": ne, "flops_per_step": float(flops),
                "TFLOPs": flops / ms / 1e9, "mfma_frac": flops / ms / 1e9 / MFMA_F16_PEAK_TFLOPS,
                "kernel_ms": kms, "grouped_gemm_ms": gemm_ms, "roofline": roof}
        return {
            "T": T, "routing": "router+bias N(0,0.5)", "launch": "hip_graph", "ms_per_layer": ms, **pct,
            "ms_per_layer_eager": ms_eager, "tokens_per_s": T * 1000.0 / ms,
            "tokens_per_s_eager": T * 1000.0 / ms_eager, "nonempty_experts": ne,
            "algorithmic_bytes_per_step": float(step_bytes), "flops_per_step": float(flops),
            "GBps": step_bytes / ms / 1e6, "hbm_frac": step_bytes / ms / 1e6 / HBM_PEAK_GBS,
            "TFLOPs": flops / ms / 1e9, "mfma_frac": flops / ms / 1e9 / MFMA_F16_PEAK_TFLOPS,
            "kernel_ms": kms, "grouped_gemm_ms": gemm_ms,
            "gateup_TFLOPs": gu_flops / gu_ms / 1e9, "gateup_GBps": gu_bytes / gu_ms / 1e6,
            "roofline": {
                "bound": "hbm", "kernel": "prefill_gateup_kernel",
                "achieved": round(gu_bytes / gu_ms / 1e6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_bytes / gu_ms / 1e6 / HBM_PEAK_GBS, 4),
                "traffic": pmc_traffic("prefill_gateup_T1024_pmc_traffic.txt", "prefill_gateup_kernel"),
                "algorithmic_bytes_per_launch": float(gu_bytes), "kernel_us": round(gu_ms * 1e3, 2),
                "mfma_TFLOPs": round(gu_flops / gu_ms / 1e9, 1),
                "mfma_frac": round(gu_flops / gu_ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
            },
        }

    # ------------------------------------------------ verify windows T = 4..8
    # The same Zipf-routed windows through the decode path (one call, top-k
    # inside) and through the grouped prefill path (routing histogram +
    # grouped GEMMs), to find where decode should hand over.
    def grouped_window(T, n_steps, warmup):
        total = rows_needed(n_steps, warmup)
        rng = synth.rng_for(1, 100 + T, 0)
        xd, _ = synth.activations(rng, min(total, 64) * T, H, "bf16")
        xs = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev).view(-1, T, H)
        nx = xs.shape[0]
        lg = synth.zipf_logits(rng, total * T, E).reshape(total, T, E)
        logits = torch.from_numpy(np.ascontiguousarray(lg)).to(dev)
        r = {n: torch.empty(s_, dtype=dt, device=dev) for n, s_, dt in [
            ("ids", (T, K), torch.int32), ("w", (T, K), torch.float32), ("counts", (E,), torch.int32),
            ("offsets", (E + 1,), torch.int32), ("sp", (T * K,), torch.int32),
            ("pp", (T * K,), torch.int32)]}
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        wsr = B.workspace(B.MOE_OP_ROUTE, T, E, K, H, I, dev)
        ws = B.workspace(B.MOE_OP_PREFILL, T, E, K, H, I, dev)

        def step(i):
            L = layers[i % len(layers)]
            B.moe_route_topk(logits[i], K, r["ids"], r["w"], r["counts"], r["offsets"], r["sp"],
                             r["pp"], wsr)
            B.moe_expert_forward_prefill(L, xs[i % nx], r["ids"], r["w"], r["counts"], r["offsets"],
                                         r["sp"], r["pp"], out, None, 0, ws)

        return run_phases(step, n_steps, warmup)[1]

    def verify_windows(Ts, n_steps, warmup):
        rows = {}
        handover = None
        for T in Ts:
            d = decode_case(T, "zipf", n_steps, warmup)
            d2 = decode_case(T, "zipf", n_steps, warmup, routed=False)
            g_ms = grouped_window(T, n_steps, warmup)
            dec_ms = min(d["ms_per_layer"], d2["ms_per_layer"])
            faster = "decode" if dec_ms <= g_ms else "grouped"
            if faster == "grouped" and handover is None:
                handover = T
            rows[f"T{T}"] = {"decode_ms_per_layer": d["ms_per_layer"],
                             "decode_two_calls_ms_per_layer": d2["ms_per_layer"],
                             "grouped_ms_per_layer": g_ms,
                             "decode_tokens_per_s": T * 1000.0 / dec_ms,
                             "grouped_tokens_per_s": T * 1000.0 / g_ms,
                             "distinct_experts": d["distinct_experts_per_step"],
                             "decode_hbm_frac": d["hbm_frac"], "faster": faster}
        return {"routing": "zipf(1.1)", "launch": "hip_graph", "windows": rows,
                "grouped_first_faster_at_T": handover}

    # ------------------------------------------------------- residency tier
    def tiered_case(n_steps, warmup, arena_kind, n_layers, frac=18119 / 24576, learn=256):
        """One token per step, Zipf(1.1) routing with one popularity order
        per run.  Each layer's tier holds the round(frac * E) experts its
        usage histogram over `learn` earlier tokens ranks highest (the
        resident share of the pages' configuration); the arena holds all
        512 (device memory, or pinned host memory read over PCIe).  The
        same rows run untiered on the same layers for comparison; every
        tiered step also adds to the usage histogram."""
        S = int(round(frac * E))
        tl = layers[:n_layers]
        total = rows_needed(n_steps, warmup)
        rng = synth.rng_for(4, 0, 1)
        xd, _ = synth.activations(rng, 64, H, "bf16")
        xs = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(synth.zipf_logits(rng, learn + total, E)).to(dev)
        out = torch.empty((1, H), dtype=torch.float32, device=dev)
        ws = B.workspace(B.MOE_OP_DECODE, 1, E, K, H, I, dev)
        ids = torch.empty((learn + total, K), dtype=torch.int32, device=dev)
        tiers, usage = [], []
        for L in tl:
            if arena_kind == "host":
                arena = torch.empty(L.experts.numel(), dtype=torch.uint8, pin_memory=True)
                arena.copy_(L.experts)
            else:
                arena = L.experts
            tiers.append(B.TieredLayer(torch.empty(S * L.expert_stride, dtype=torch.uint8, device=dev),
                                       torch.full((E,), -1, dtype=torch.int32, device=dev), arena, L.shared,
                                       S, E, H, I, L.expert_stride))
            usage.append(torch.zeros(E, dtype=torch.int64, device=dev))
        # learning window: usage only (every expert still read from the arena)
        wl = torch.empty((1, K), dtype=torch.float32, device=dev)
        for i in range(learn):
            l = i % n_layers
            B.moe_expert_forward_decode_tiered(tiers[l], xs[i % 64].view(1, H), lg[i].view(1, E), K, out,
                                               ids[i].view(1, K), wl, None, 0, usage[l], ws)
        torch.cuda.synchronize()
        t0 = time.time()
        for l in range(n_layers):
            occ = np.full(S, -1, dtype=np.int32)
            new, _, _ = B.moe_residency_plan(usage[l].cpu().numpy().astype(np.uint64), S, occ)
            B.moe_residency_apply(tiers[l], occ, new)
        torch.cuda.synchronize()
        apply_s = (time.time() - t0) / n_layers
        slot_of = np.stack([t.slot_of.cpu().numpy() for t in tiers])
        wts = torch.empty((total, K), dtype=torch.float32, device=dev)

        def step_t(i):
            l = i % n_layers
            B.moe_expert_forward_decode_tiered(tiers[l], xs[i % 64].view(1, H), lg[learn + i].view(1, E), K,
                                               out, ids[learn + i].view(1, K), wts[i].view(1, K), None, 0,
                                               usage[l], ws)

        def step_u(i):
            B.moe_expert_forward_decode_routed(tl[i % n_layers], xs[i % 64].view(1, H), lg[learn + i].view(1, E),
                                               K, out, None, None, None, 0, ws)

        plan, ms, ms_eager, pct, kern = run_phases(step_t, n_steps, warmup)
        plan_u, ms_u, ms_eager_u, pct_u, _ = run_phases(step_u, n_steps, warmup)
        idh = ids[learn:].cpu().numpy()
        rows = list(plan["graph_timed"])
        hit = np.array([(slot_of[i % n_layers][idh[i]] >= 0).mean() for i in rows])
        miss_bytes = (1.0 - hit.mean()) * K * EXPERT_BYTES
        gu = kern.get("decode_gateup_kernel", (1, float("nan")))
        dn = kern.get("decode_down_kernel", (1, float("nan")))
        del tiers
        return {
            "T": 1, "routing": "zipf(1.1), one popularity order", "arena": arena_kind,
            "resident_slots": S, "experts": E, "layers": n_layers, "learn_tokens": learn,
            "calls": "decode_tiered (+ usage histogram) vs decode_routed", "launch": "hip_graph",
            "ms_per_layer": ms, **pct, "ms_per_layer_eager": ms_eager,
            "ms_per_layer_untiered": ms_u, "ms_per_layer_untiered_eager": ms_eager_u,
            "tokens_per_s": 1000.0 / ms, "tokens_per_s_untiered": 1000.0 / ms_u,
            "hit_rate": float(hit.mean()), "miss_bytes_per_step": float(miss_bytes),
            # host arena: the misses' cost over the untiered call on the same
            # rows, as a PCIe rate (a device arena reads them from HBM)
            "miss_GBps_over_untiered": (float(miss_bytes / ((ms - ms_u) * 1e6))
                                        if arena_kind == "host" and ms > ms_u else None),
            "apply_s_per_layer": apply_s,
            "kernel_ms": {"decode_gateup": gu[1] / gu[0], "decode_down": dn[1] / dn[0]},
        }

    only = args.only
    half = case_steps(args.steps)["half"]
    if only in ("", "decode1"):
        results["decode_T1"] = decode_case(1, "router", args.steps, args.warmup)
        progress("decode_T1")
    if only in ("", "decode1_two_calls"):
        results["decode_T1_two_calls"] = decode_case(1, "router", half, args.warmup,
                                                     routed=False)
        progress("decode_T1_two_calls")
    if only in ("", "decode1_gemv"):
        results["decode_T1_router_gemv"] = decode_case(1, "router", half, args.warmup,
                                                       routed=False, gemv=True)
        progress("decode_T1_router_gemv")
    if only in ("", "decode2"):
        results["decode_T2"] = decode_case(2, "zipf", half, args.warmup)
        progress("decode_T2")
    if only in ("", "decode3"):
        results["decode_T3"] = decode_case(3, "zipf", half, args.warmup)
        progress("decode_T3")
    if only in ("", "prefill"):
        results["prefill_T1024"] = prefill_case(1024, args.prefill_steps, max(4, args.warmup // 4))
        progress("prefill_T1024")
    if only == "prefill32768":   # profiling runs only: one 32768-token chunk, Zipf routing
        results["prefill_T32768"] = prefill_case(32768, max(4, args.prefill_steps // 10), 2, "zipf")
        progress("prefill_T32768")
    if only in ("", "tiered", "tiered_device"):
        results["decode_T1_tiered_device_arena"] = tiered_case(half, args.warmup, "device", len(layers))
        progress("decode_T1_tiered_device_arena")
    if only in ("", "tiered", "tiered_host"):
        results["decode_T1_tiered_host_arena"] = tiered_case(half, args.warmup, "host", min(4, len(layers)))
        progress("decode_T1_tiered_host_arena")
    if only in ("", "windows"):
        results["verify_windows"] = verify_windows([4, 5, 6, 7, 8], case_steps(args.steps)["windows"],
                                                   max(4, args.warmup // 2))
        progress("verify_windows")

    # ------------------------------------------------- 48 stacked layers
    # 48 distinct layers (54.5 GB), x_{l+1} = x_l + MoE_l(rmsnorm(x_l)) in a
    # float32 residual stream, Zipf(1.1) routing with a fixed seed per layer.
    if only in ("", "stack") and args.stack_layers > 0:
        NL = args.stack_layers
        del layers[:]                      # free the rotating set first
        torch.cuda.empty_cache()
        stack = []
        for l in range(NL):
            ex = synth.device_expert_blob(E, H, I, synth.torch_seed(2, l, 1), dev)
            sh = synth.device_expert_blob(1, H, I, synth.torch_seed(2, l, 2), dev)
            stack.append(B.Layer(ex, sh, E, H, I, synth.expert_stride(H, I)))
        torch.cuda.synchronize()

        def stack_decode(T, steps):
            lg = [synth.device_zipf_logits(T, E, synth.torch_seed(2, l, 3), dev) for l in range(NL)]
            x0 = torch.randn((T, H), device=dev).to(torch.bfloat16).float()
            bufs = [torch.empty_like(x0) for _ in range(2)]
            ws = B.workspace(B.MOE_OP_DECODE, T, E, K, H, I, dev)

            def step(_i):
                x = x0
                for l in range(NL):
                    o = bufs[l & 1]
                    B.moe_expert_forward_decode_routed(stack[l], x, lg[l], K, o, None, None, x,
                                                       B.MOE_FLAG_PRENORM_RMS, ws)
                    x = o
            g = capture(step, range(1))      # one step = all NL layers
            g.replay()
            torch.cuda.synchronize()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            for _ in range(steps):
                g.replay()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / steps
            del g
            return {"T": T, "layers": NL, "launch": "hip_graph", "ms_per_step": ms,
                    "us_per_layer": ms * 1e3 / NL, "tokens_per_s": T * 1000.0 / ms}

        def stack_prefill(T, steps):
            x0 = torch.randn((T, H), device=dev).to(torch.bfloat16).float()
            bufs = [torch.empty_like(x0) for _ in range(2)]
            ws = B.workspace(B.MOE_OP_PREFILL, T, E, K, H, I, dev)
            wsr = B.workspace(B.MOE_OP_ROUTE, T, E, K, H, I, dev)
            r = {n: torch.empty(sz, dtype=dt, device=dev) for n, sz, dt in [
                ("ids", (T, K), torch.int32), ("w", (T, K), torch.float32), ("counts", (E,), torch.int32),
                ("offsets", (E + 1,), torch.int32), ("sp", (T * K,), torch.int32),
                ("pp", (T * K,), torch.int32)]}
            lg = torch.empty((T, E), dtype=torch.float32, device=dev)

            def run(prof):
                x = x0
                for l in range(NL):
                    lg.copy_(synth.device_zipf_logits(T, E, synth.torch_seed(2, l, 3), dev))
                    B.moe_route_topk(lg, K, r["ids"], r["w"], r["counts"], r["offsets"], r["sp"],
                                     r["pp"], wsr)
                    o = bufs[l & 1]
                    B.moe_expert_forward_prefill(stack[l], x, r["ids"], r["w"], r["counts"],
                                                 r["offsets"], r["sp"], r["pp"], o, x,
                                                 B.MOE_FLAG_PRENORM_RMS, ws)
                    x = o
            run(False)
            torch.cuda.synchronize()
            B.profile_reset()
            B.profile_enable(True)
            run(True)
            torch.cuda.synchronize()
            B.profile_enable(False)
            kern = {k.replace("_kernel", ""): v[1] for k, v in B.profile_results().items() if v[0]}
            moe_ms = sum(kern.values())
            gemm_ms = kern.get("prefill_gateup", 0.0) + kern.get("prefill_down", 0.0)
            return {"T": T, "layers": NL, "launch": "eager, dispatch-stamped kernel times",
                    "moe_ms_per_step": moe_ms, "us_per_layer": moe_ms * 1e3 / NL,
                    "grouped_gemm_us_per_layer": gemm_ms * 1e3 / NL,
                    "tokens_per_s": T * 1000.0 / moe_ms,
                    "kernel_ms_per_layer": {k: v / NL for k, v in kern.items()}}

        for T in (1, 2, 3):
            results[f"stack{NL}_decode_T{T}"] = stack_decode(T, 20)
            progress(f"stack{NL}_decode_T{T}")
        for T in (1024, 32768):
            results[f"stack{NL}_prefill_T{T}"] = stack_prefill(T, 1)
            progress(f"stack{NL}_prefill_T{T}")
        del stack
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ cpu baseline
    cpu = None
    if not args.no_cpu_baseline and only == "":
        cpu = cpu_baseline(args.cpu_seconds)
        progress("cpu_baseline")

    head = results.get("decode_T1") or next(
        (v for v in results.values() if "tokens_per_s" in v and "ms_per_layer" in v),
        {"tokens_per_s": float("nan"), "ms_per_layer": float("nan")})
    line = {
        "metric": "MoE-layer tokens/s (decode B=1..3, prefill 1024 chunk); HBM GB/s % peak",
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_layer"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "moe_layer_decode_T1: router top-k + expert layer (moe_expert_forward_decode_routed), "
                        "1 token, 512 experts top-10 + 1 shared, "
                        "hidden 3072, inter 768, Q2 2-bit weights (2,211,840 B/expert), "
                        f"{args.layers} rotating layers",
            "tokens_per_step": 1, "experts": E, "top_k": K, "hidden": H, "inter": I,
            "parallelism": "single_gpu", "launch": "hip_graph (the timed steps in one graph)",
        },
    }
    if "decode_T1" in results:
        d = results["decode_T1"]
        line["roofline"] = {
            "bound": "hbm", "kernel": "decode_gateup_kernel",
            "achieved": round(d["gateup_GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(d["gateup_GBps"] / HBM_PEAK_GBS, 4),
            "traffic": pmc_traffic("decode_gateup_T1_pmc_traffic.txt", "decode_gateup_kernel"),
            "algorithmic_bytes_per_launch": d["gateup_bytes_per_launch"],
            "kernel_us": round(d["kernel_ms"]["decode_gateup"] * 1e3, 3),
            "layer_GBps": round(d["GBps"], 1), "layer_frac": round(d["hbm_frac"], 4),
        }
    if ceilings:
        line["ceilings"] = ceilings
        if "roofline" in line:
            line["roofline"]["measured_stream_GBps"] = ceilings["stream_read_GBps"]
    line["results"] = results
    if cpu:
        line["cpu_baseline"] = cpu
    line["weights_generated_s"] = round(gen_s, 1)
    print(json.dumps(line))


def pmc_traffic(name: str, kernel: str):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, each scaled
    by its copy-kernel calibration) from the committed counter summary
    profiles/<name>; None when the file is absent or when the kernel's
    sources (comments aside) no longer hash to what they were when the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in lines if ": " in l and not l.startswith("#"))
    srcs = kv.get("sources", "").split()
    if kv.get("kernel") != kernel or not srcs:
        return None
    from bit_quantized_expert_router_amd.profsum import code_sha256
    try:
        sha = code_sha256([os.path.join(ROOT, f) for f in srcs])
    except OSError:
        return None
    if sha != kv.get("source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(seconds: float, prefill_tokens: int = 1024):
    """The fp64 oracle on the host cores, on the same workload shape (512
    experts top-10 + shared, H 3072, I 768): decode of one token for a
    bounded number of steps (about `seconds` of oracle time), then one full
    prefill chunk of `prefill_tokens` tokens with the skewed router (logits
    from a bf16 router weight plus a per-expert N(0, 0.5) bias): routing,
    histogram and the expert layer, every used expert decoded from its 2-bit
    bytes once."""
    import platform
    import oracle as O
    from bit_quantized_expert_router_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    rng = synth.rng_for(1, 500, 0)
    blob = synth.expert_blob(rng, E, H, I)
    sh = synth.expert_blob(rng, 1, H, I)
    steps = 0
    spent = 0.0
    while spent < seconds and steps < 64:
        ob = O.ExpertBlob(blob, E, H, I, shared=sh, cache=0)   # decodes from bytes every step
        _, xv = synth.activations(rng, 1, H, "bf16")
        lg = synth.router_logits(rng, xv, E)
        t1 = time.perf_counter()
        ids, w = O.route_topk(lg, K)
        O.moe_layer(xv, ids, w, ob)
        spent += time.perf_counter() - t1
        steps += 1
    res = {"value": round(steps / spent, 4), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle", "cpu": cpu_model,
           "sample": f"{steps} decode steps of 1 token (route + 11 experts decoded from the 2-bit "
                     f"bytes and evaluated in float64), {spent:.1f} s of oracle time; input "
                     f"generation excluded; cores = BLAS threads"}
    if prefill_tokens:
        T = prefill_tokens
        rngp = synth.rng_for(3, 500, T)
        _, xv = synth.activations(rngp, T, H, "bf16")
        lg = synth.biased_logits(rngp, synth.router_logits(rngp, xv, E))
        ob = O.ExpertBlob(blob, E, H, I, shared=sh, cache=0)
        t1 = time.perf_counter()
        ids, w = O.route_topk(lg, K)
        O.route_histogram(ids, E)
        O.moe_layer(xv, ids, w, ob)
        sp = time.perf_counter() - t1
        res["prefill_T1024"] = {
            "value": round(T / sp, 3), "unit": "tokens/s", "seconds": round(sp, 2),
            "cores": int(threads), "kind": "oracle",
            "sample": f"one full {T}-token prefill layer (router N(0,0.5) bias; "
                      f"{len(np.unique(ids))} non-empty experts + shared, each decoded once from its "
                      f"2-bit bytes, float64)"}
    return res


def counters_run(args):
    """Eager steps of one case only (no graph capture, no measurement hooks,
    no ceilings, no oracle), for hardware-counter collection: every dispatch
    is an ordinary stream launch.  decode1: 1-token routed decode; prefill1024
    / prefill32768: routing + prefill of one chunk (biased router logits,
    resp. Zipf(1.1) ids) per step."""
    import torch
    from bit_quantized_expert_router_amd import binding as B
    from bit_quantized_expert_router_amd import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    layers = []
    for l in range(args.layers):
        ex = synth.device_expert_blob(E, H, I, synth.torch_seed(1, l, 1), dev)
        sh = synth.device_expert_blob(1, H, I, synth.torch_seed(1, l, 2), dev)
        layers.append(B.Layer(ex, sh, E, H, I, synth.expert_stride(H, I)))
    if args.counters != "decode1":
        T = 1024 if args.counters == "prefill1024" else 32768
        rng = synth.rng_for(3, 0, T)
        xd, xv = synth.activations(rng, T, H, "bf16")
        x = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev)
        lg = (synth.biased_logits(rng, synth.router_logits(rng, xv, E)) if T == 1024 else
              synth.zipf_logits(rng, T, E))
        r = B.route(torch.from_numpy(lg).to(dev), K, histogram=True)
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = B.workspace(B.MOE_OP_PREFILL, T, E, K, H, I, dev)
        torch.cuda.synchronize()
        t0 = time.time()
        for i in range(args.steps):
            B.moe_expert_forward_prefill(layers[i % len(layers)], x, r["topk_ids"], r["topk_w"], r["counts"],
                                         r["offsets"], r["sorted_pairs"], r["pair_pos"], out, None, 0, ws)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": f"prefill_T{T} eager", "steps": args.steps,
                          "wall_s": round(time.time() - t0, 4), "out_finite": bool(torch.isfinite(out).all().item())}))
        return
    rng = synth.rng_for(1, 101, 0)
    n = args.steps
    xd, xv = synth.activations(rng, n, H, "bf16")
    xs = torch.from_numpy(xd.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(synth.router_logits(rng, xv, E)).to(dev)
    out = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = B.workspace(B.MOE_OP_DECODE, 1, E, K, H, I, dev)
    torch.cuda.synchronize()
    t0 = time.time()
    for i in range(n):
        B.moe_expert_forward_decode_routed(layers[i % len(layers)], xs[i:i + 1], logits[i:i + 1], K, out,
                                           None, None, None, 0, ws)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": "decode_T1 eager", "steps": n, "wall_s": round(time.time() - t0, 4),
                      "out_finite": bool(torch.isfinite(out).all().item())}))


if __name__ == "__main__":
    main()
