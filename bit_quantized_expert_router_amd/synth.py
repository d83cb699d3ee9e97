"""Seeded synthetic inputs for the MoE expert layer.

This module holds input generation only -- random bytes, random scales,
random activations and router logits -- and none of the layer's own
arithmetic.  Both the fp64 oracle (in the tests) and the HIP path take their
inputs from here.

Recipe (one seed stream per (config, layer, tensor)):
  * codes: uniform random bytes, i.e. four i.i.d. U{0..3} 2-bit codes per byte;
  * scales: U(0.01, 0.05) rounded to fp16, written at the scale positions of
    every 1280-byte tile record (bytes 1024..1279 of the record);
  * activations: N(0, 1) as float32, or rounded to bfloat16 (RNE);
  * router logits: float32(float64(x) @ float64(W_r)), W_r = bf16(N(0, 1/H));
    optional per-expert bias N(0, sigma) for skewed loads;
  * Zipf routing: logits = float32(log p(rank(e)) + Gumbel(0, 1)) with
    p(r) ~ r^-s over ranks 1..E and a per-layer random rank->expert map, so
    the top-k is a Plackett-Luce (without replacement) Zipf draw.
"""
from __future__ import annotations

import numpy as np

TILE_BYTES = 1280     # one tile record: 1024 code bytes + 128 fp16 scales
SCALE_OFFSET = 1024


def rng_for(config: int, layer: int, tensor: int, base: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([base, config, layer, tensor])))


def torch_seed(config: int, layer: int, tensor: int, base: int = 0) -> int:
    ss = np.random.SeedSequence([base, config, layer, tensor])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def expert_nbytes(H: int, I: int) -> int:
    return 3 * I * H * 5 // 16


def expert_stride(H: int, I: int) -> int:
    return (expert_nbytes(H, I) + 4095) // 4096 * 4096


# ---------------------------------------------------------------- bfloat16 --
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ weights --
def expert_blob(rng: np.random.Generator, E: int, H: int, I: int,
                scale_lo: float = 0.01, scale_hi: float = 0.05) -> np.ndarray:
    """E experts back to back at stride expert_stride(H, I); returns uint8."""
    stride = expert_stride(H, I)
    nb = expert_nbytes(H, I)
    buf = np.zeros(E * stride, dtype=np.uint8)
    nrec = nb // TILE_BYTES
    for e in range(E):
        rec = buf[e * stride:e * stride + nb].reshape(nrec, TILE_BYTES)
        rec[:, :SCALE_OFFSET] = rng.integers(0, 256, size=(nrec, SCALE_OFFSET), dtype=np.uint8)
        sc = rng.uniform(scale_lo, scale_hi, size=(nrec, 128)).astype("<f2")
        rec[:, SCALE_OFFSET:] = sc.view(np.uint8).reshape(nrec, 256)
    return buf


def constant_expert_blob(E: int, H: int, I: int, code: int, scale: float) -> np.ndarray:
    """E experts whose every 2-bit code is `code` (0..3) and every block scale
    fp16(`scale`), in the same byte layout as expert_blob: each code byte
    repeats the code four times and every record's scale bytes hold the fp16
    value.  Inputs for closed-form cases (all weights equal)."""
    if not 0 <= code <= 3:
        raise ValueError("code must be in 0..3")
    stride = expert_stride(H, I)
    nb = expert_nbytes(H, I)
    buf = np.zeros(E * stride, dtype=np.uint8)
    nrec = nb // TILE_BYTES
    byte = code | (code << 2) | (code << 4) | (code << 6)
    sc = np.full(128, scale, dtype="<f2").view(np.uint8)
    for e in range(E):
        rec = buf[e * stride:e * stride + nb].reshape(nrec, TILE_BYTES)
        rec[:, :SCALE_OFFSET] = byte
        rec[:, SCALE_OFFSET:] = sc[None, :]
    return buf


def device_expert_blob(E: int, H: int, I: int, seed: int, device="cuda",
                       scale_lo: float = 0.01, scale_hi: float = 0.05):
    """Same recipe, generated with torch's RNG straight into device memory
    (used for the multi-GB stacked workloads), every expert's codes in one
    draw and every scale in another.  Returns a uint8 tensor."""
    import torch
    stride = expert_stride(H, I)
    nb = expert_nbytes(H, I)
    nrec = nb // TILE_BYTES
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    buf = torch.empty(E * stride, dtype=torch.uint8, device=device)
    view = buf.view(E, stride)[:, :nb].view(E, nrec, TILE_BYTES)
    view[:, :, :SCALE_OFFSET] = torch.randint(0, 256, (E, nrec, SCALE_OFFSET), dtype=torch.uint8,
                                              device=device, generator=g)
    sc = (torch.rand((E, nrec, 128), device=device, generator=g, dtype=torch.float32)
          * (scale_hi - scale_lo) + scale_lo).to(torch.float16)
    view[:, :, SCALE_OFFSET:] = sc.view(torch.uint8)
    del sc
    if stride > nb:
        buf.view(E, stride)[:, nb:].zero_()
    return buf


# --------------------------------------------------------------- activations --
def activations(rng: np.random.Generator, T: int, H: int, dtype: str = "bf16"):
    """N(0,1) activations.  Returns (device_array, float32 values): for bf16
    the device array is uint16 bits and the values are their exact float32."""
    a = rng.standard_normal((T, H)).astype(np.float32)
    if dtype == "bf16":
        b = bf16_bits(a)
        return b, bf16_to_f32(b)
    if dtype == "f32":
        return a, a
    raise ValueError(dtype)


# -------------------------------------------------------------------- logits --
def router_weight(rng: np.random.Generator, E: int, H: int) -> np.ndarray:
    """bf16 router weight [E, H] (row e for expert e), N(0, 1/H), as raw
    bf16 bits (uint16)."""
    return bf16_bits((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))


def router_logits(rng: np.random.Generator, x_f32: np.ndarray, E: int) -> np.ndarray:
    """float32(float64(x) @ float64(W_r)), W_r = bf16(N(0, 1/H)) [H, E]."""
    H = x_f32.shape[1]
    W = bf16_to_f32(bf16_bits((rng.standard_normal((H, E)) / np.sqrt(H)).astype(np.float32)))
    return (np.asarray(x_f32, dtype=np.float64) @ W.astype(np.float64)).astype(np.float32)


def biased_logits(rng: np.random.Generator, logits: np.ndarray, sigma: float = 0.5) -> np.ndarray:
    """Adds a per-expert bias N(0, sigma) in float32 (skewed expert loads)."""
    bias = rng.normal(0.0, sigma, size=logits.shape[1]).astype(np.float32)
    return (logits + bias[None, :]).astype(np.float32)


def zipf_logits(rng: np.random.Generator, T: int, E: int, s: float = 1.1) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -s * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    perm = rng.permutation(E)              # rank r -> expert perm[r]
    base = np.empty(E, dtype=np.float64)
    base[perm] = logp
    gumbel = -np.log(-np.log(rng.uniform(np.finfo(np.float64).tiny, 1.0, size=(T, E))))
    return (base[None, :] + gumbel).astype(np.float32)


def device_zipf_logits(T: int, E: int, seed: int, device="cuda", s: float = 1.1):
    """zipf_logits' recipe with torch's generator on the device (for the
    large stacked workloads whose logits would take long to make on the
    host).  Returns a float32 [T, E] tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    ranks = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    logp = -s * torch.log(ranks)
    logp -= torch.log(torch.exp(logp).sum())
    perm = torch.randperm(E, device=device, generator=g)
    base = torch.empty(E, dtype=torch.float64, device=device)
    base[perm] = logp
    u = torch.rand((T, E), dtype=torch.float64, device=device, generator=g).clamp_min_(1e-300)
    return (base[None, :] - torch.log(-torch.log(u))).to(torch.float32)


def tie_logits(rng: np.random.Generator, T: int, E: int, levels: int = 4) -> np.ndarray:
    """Logits drawn from a few values only, so equal logits are common."""
    return rng.integers(0, levels, size=(T, E)).astype(np.float32) * np.float32(0.5)
