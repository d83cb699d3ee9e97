"""ctypes binding of libmoe_q2.so (C ABI: include/moe_q2.h).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and a non-zero status becomes a
MoeError.  Every step of the layer runs in the library's HIP kernels; there
is no fallback.  Importing this module loads the library and raises if it
is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_Q2_LIB", os.path.join(_HERE, "libmoe_q2.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_FLAG_PRENORM_RMS = 1
MOE_OP_ROUTE, MOE_OP_DECODE, MOE_OP_PREFILL, MOE_OP_ROUTE_GEMV = 0, 1, 2, 3

EXPORTS = ["moe_workspace_bytes", "moe_route_topk", "moe_route_topk_gemv", "moe_expert_forward_decode",
           "moe_expert_forward_decode_routed", "moe_expert_forward_decode_routed_noalloc",
           "moe_expert_forward_prefill", "moe_expert_usage_update", "moe_residency_plan",
           "moe_residency_apply", "moe_expert_forward_decode_tiered", "moe_expert_forward_prefill_tiered",
           "moe_status_string", "moe_last_error",
           "moe_profile_enable", "moe_profile_reset", "moe_profile_num_kernels",
           "moe_profile_kernel_name", "moe_profile_query"]


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_string(status)}: {detail}")
        self.status = status


class _Layer(C.Structure):
    _fields_ = [("experts", C.c_void_p), ("shared", C.c_void_p), ("expert_stride", C.c_int64),
                ("num_experts", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32)]


class _TieredLayer(C.Structure):
    _fields_ = [("slots", C.c_void_p), ("slot_of", C.c_void_p), ("arena", C.c_void_p), ("shared", C.c_void_p),
                ("expert_stride", C.c_int64), ("num_slots", C.c_int32), ("num_experts", C.c_int32),
                ("hidden", C.c_int32), ("inter", C.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m bit_quantized_expert_router_amd.build_lib`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    lib.moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_topk.restype = C.c_int
    lib.moe_route_topk_gemv.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_route_topk_gemv.restype = C.c_int
    lib.moe_expert_forward_decode.argtypes = [C.POINTER(_Layer), vp, i32, i32, vp, vp, i32, vp, vp,
                                              i32, C.c_uint32, vp, sz, vp]
    lib.moe_expert_forward_decode.restype = C.c_int
    lib.moe_expert_forward_decode_routed.argtypes = [C.POINTER(_Layer), vp, i32, i32, vp, i32, vp, vp,
                                                     vp, vp, i32, C.c_uint32, vp, sz, vp]
    lib.moe_expert_forward_decode_routed.restype = C.c_int
    lib.moe_expert_forward_decode_routed_noalloc.argtypes = [C.POINTER(_Layer), vp, i32, i32, vp, i32, vp, vp,
                                                             vp, vp, i32, C.c_uint32, vp]
    lib.moe_expert_forward_decode_routed_noalloc.restype = C.c_int
    lib.moe_expert_forward_prefill.argtypes = [C.POINTER(_Layer), vp, i32, i32, vp, vp, i32, vp, vp,
                                               vp, vp, vp, vp, i32, C.c_uint32, vp, sz, vp]
    lib.moe_expert_forward_prefill.restype = C.c_int
    lib.moe_expert_usage_update.argtypes = [vp, i64, i32, vp, vp]
    lib.moe_expert_usage_update.restype = C.c_int
    lib.moe_residency_plan.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.moe_residency_plan.restype = C.c_int
    lib.moe_residency_apply.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_residency_apply.restype = C.c_int
    lib.moe_expert_forward_decode_tiered.argtypes = [C.POINTER(_TieredLayer), vp, i32, i32, vp, i32, vp, vp,
                                                     vp, vp, i32, C.c_uint32, vp, vp, sz, vp]
    lib.moe_expert_forward_decode_tiered.restype = C.c_int
    lib.moe_expert_forward_prefill_tiered.argtypes = [C.POINTER(_TieredLayer), vp, i32, i32, vp, vp, i32, vp,
                                                      vp, vp, vp, vp, vp, i32, C.c_uint32, vp, sz, vp]
    lib.moe_expert_forward_prefill_tiered.restype = C.c_int
    lib.moe_status_string.argtypes = [C.c_int]
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = C.c_char_p
    lib.moe_profile_enable.argtypes = [C.c_int]
    lib.moe_profile_reset.argtypes = []
    lib.moe_profile_num_kernels.argtypes = []
    lib.moe_profile_kernel_name.argtypes = [C.c_int]
    lib.moe_profile_kernel_name.restype = C.c_char_p
    lib.moe_profile_query.argtypes = [C.c_int, C.POINTER(C.c_int64), C.POINTER(C.c_double)]
    return lib


lib = _load()


def _status_string(s: int) -> str:
    return lib.moe_status_string(s).decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib.moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


@dataclass
class Layer:
    """Expert weights of one layer on the device (uint8 tensors)."""
    experts: torch.Tensor
    shared: Optional[torch.Tensor]
    num_experts: int
    hidden: int
    inter: int
    expert_stride: int

    def _c(self) -> _Layer:
        return _Layer(self.experts.data_ptr(), None if self.shared is None else self.shared.data_ptr(),
                      self.expert_stride, self.num_experts, self.hidden, self.inter)


def moe_workspace_bytes(op: int, T: int, E: int, k: int, H: int, I: int) -> int:
    return int(lib.moe_workspace_bytes(op, T, E, k, H, I))


def workspace(op: int, T: int, E: int, k: int, H: int, I: int, device="cuda") -> torch.Tensor:
    """Workspace for one call (zeroed for MOE_OP_ROUTE_GEMV, whose counter
    must start at zero)."""
    n = max(moe_workspace_bytes(op, T, E, k, H, I), 256)
    if op == MOE_OP_ROUTE_GEMV:
        return torch.zeros(n, dtype=torch.uint8, device=device)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route_topk(logits, k, topk_ids, topk_w, counts=None, offsets=None, sorted_pairs=None,
                   pair_pos=None, ws=None, stream=None):
    T, E = logits.shape
    _check(lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                              _ptr(offsets), _ptr(sorted_pairs), _ptr(pair_pos), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)))


def moe_route_topk_gemv(x, router_w, k, topk_ids, topk_w, logits=None, ws=None, stream=None):
    """router_w: bf16 tensor [E, H] (or its int16/uint16 bits).  topk_ids and
    topk_w may both be None (logits only; ws may then be None too)."""
    T, H = x.shape
    E = router_w.shape[0]
    _check(lib.moe_route_topk_gemv(_ptr(x), _dtype_code(x), T, _ptr(router_w), E, H, k, _ptr(logits),
                                   _ptr(topk_ids), _ptr(topk_w), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream)))


def moe_expert_forward_decode(layer: Layer, x, topk_ids, topk_w, out, residual=None, flags=0,
                              ws=None, stream=None):
    T, k = topk_ids.shape
    c = layer._c()
    _check(lib.moe_expert_forward_decode(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(topk_ids),
                                         _ptr(topk_w), k, _ptr(residual), _ptr(out), _dtype_code(out),
                                         flags, _ptr(ws), 0 if ws is None else ws.numel(),
                                         _stream(stream)))


def moe_expert_forward_decode_routed(layer: Layer, x, logits, k, out, topk_ids=None, topk_w=None,
                                     residual=None, flags=0, ws=None, stream=None):
    T = logits.shape[0]
    c = layer._c()
    _check(lib.moe_expert_forward_decode_routed(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(logits), k,
                                                _ptr(topk_ids), _ptr(topk_w), _ptr(residual), _ptr(out),
                                                _dtype_code(out), flags, _ptr(ws),
                                                0 if ws is None else ws.numel(), _stream(stream)))


def moe_expert_forward_decode_routed_noalloc(layer: Layer, x, logits, k, out, topk_ids=None, topk_w=None,
                                             residual=None, flags=0, stream=None):
    """The routed decode call on the library's static per-GPU scratch (no
    workspace argument, nothing allocated)."""
    T = logits.shape[0]
    c = layer._c()
    _check(lib.moe_expert_forward_decode_routed_noalloc(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(logits), k,
                                                        _ptr(topk_ids), _ptr(topk_w), _ptr(residual),
                                                        _ptr(out), _dtype_code(out), flags, _stream(stream)))


def moe_expert_forward_prefill(layer: Layer, x, topk_ids, topk_w, counts, offsets, sorted_pairs,
                               pair_pos, out, residual=None, flags=0, ws=None, stream=None):
    T, k = topk_ids.shape
    c = layer._c()
    _check(lib.moe_expert_forward_prefill(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(topk_ids),
                                          _ptr(topk_w), k, _ptr(counts), _ptr(offsets),
                                          _ptr(sorted_pairs), _ptr(pair_pos), _ptr(residual),
                                          _ptr(out), _dtype_code(out), flags, _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(stream)))


# --------------------------------------------------------- residency tier --
def _arena_ptr(t: torch.Tensor):
    """The arena may be device memory or pinned host memory (a CPU tensor
    made with pin_memory=True); the library maps the latter itself."""
    if not t.is_contiguous():
        raise ValueError("the arena must be contiguous")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("the arena must be on the GPU or in pinned host memory")
    return C.c_void_p(t.data_ptr())


def _host_i32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(C.c_void_p)


@dataclass
class TieredLayer:
    """A layer whose experts live in `arena` (all E, device or pinned host
    memory), S of them copied into `slots` (device); slot_of (device int32
    [E]) maps expert -> slot or -1."""
    slots: Optional[torch.Tensor]
    slot_of: torch.Tensor
    arena: torch.Tensor
    shared: Optional[torch.Tensor]
    num_slots: int
    num_experts: int
    hidden: int
    inter: int
    expert_stride: int

    def _c(self) -> _TieredLayer:
        return _TieredLayer(None if self.slots is None else _ptr(self.slots).value, _ptr(self.slot_of).value,
                            _arena_ptr(self.arena).value,
                            None if self.shared is None else _ptr(self.shared).value, self.expert_stride,
                            self.num_slots, self.num_experts, self.hidden, self.inter)


def moe_expert_usage_update(ids, E: int, counts, stream=None):
    """counts (device uint64/int64 [E]) += occurrences of each expert in ids."""
    _check(lib.moe_expert_usage_update(_ptr(ids), ids.numel(), E, _ptr(counts), _stream(stream)))


def moe_residency_plan(counts, S: int, expert_of_slot):
    """Host plan: (new_expert_of_slot [S], slot_of [E], n_changed)."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    E = c.size
    cur, cur_p = _host_i32(np.asarray(expert_of_slot).reshape(-1))
    new = np.empty(S, dtype=np.int32)
    slot_of = np.empty(E, dtype=np.int32)
    n = C.c_int32(0)
    _check(lib.moe_residency_plan(c.ctypes.data_as(C.c_void_p), E, S, cur_p, new.ctypes.data_as(C.c_void_p),
                                  slot_of.ctypes.data_as(C.c_void_p), C.byref(n)))
    return new, slot_of, n.value


def moe_residency_apply(layer: TieredLayer, old_expert_of_slot, new_expert_of_slot, stream=None):
    """Copies the changed slots from the arena and updates layer.slot_of."""
    old, old_p = _host_i32(old_expert_of_slot)
    new, new_p = _host_i32(new_expert_of_slot)
    _check(lib.moe_residency_apply(_arena_ptr(layer.arena), layer.expert_stride, layer.num_experts,
                                   layer.num_slots, old_p, new_p, _ptr(layer.slots), _ptr(layer.slot_of),
                                   _stream(stream)))


def moe_expert_forward_decode_tiered(layer: TieredLayer, x, logits, k, out, topk_ids=None, topk_w=None,
                                     residual=None, flags=0, usage_counts=None, ws=None, stream=None):
    T = logits.shape[0]
    c = layer._c()
    _check(lib.moe_expert_forward_decode_tiered(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(logits), k,
                                                _ptr(topk_ids), _ptr(topk_w), _ptr(residual), _ptr(out),
                                                _dtype_code(out), flags, _ptr(usage_counts), _ptr(ws),
                                                0 if ws is None else ws.numel(), _stream(stream)))


def moe_expert_forward_prefill_tiered(layer: TieredLayer, x, topk_ids, topk_w, counts, offsets, sorted_pairs,
                                      pair_pos, out, residual=None, flags=0, ws=None, stream=None):
    T, k = topk_ids.shape
    c = layer._c()
    _check(lib.moe_expert_forward_prefill_tiered(C.byref(c), _ptr(x), _dtype_code(x), T, _ptr(topk_ids),
                                                 _ptr(topk_w), k, _ptr(counts), _ptr(offsets),
                                                 _ptr(sorted_pairs), _ptr(pair_pos), _ptr(residual),
                                                 _ptr(out), _dtype_code(out), flags, _ptr(ws),
                                                 0 if ws is None else ws.numel(), _stream(stream)))


# ---------------------------------------------------------------- helpers --
def route(logits: torch.Tensor, k: int, histogram: bool = False, ws=None, stream=None) -> dict:
    """Allocates the outputs and calls moe_route_topk."""
    T, E = logits.shape
    dev = logits.device
    r = {"topk_ids": torch.empty((T, k), dtype=torch.int32, device=dev),
         "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev)}
    if histogram:
        r["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
        r["offsets"] = torch.empty(E + 1, dtype=torch.int32, device=dev)
        r["sorted_pairs"] = torch.empty(T * k, dtype=torch.int32, device=dev)
        r["pair_pos"] = torch.empty(T * k, dtype=torch.int32, device=dev)
        if ws is None:
            ws = workspace(MOE_OP_ROUTE, T, E, k, 256, 256, dev)
    moe_route_topk(logits, k, r["topk_ids"], r["topk_w"], r.get("counts"), r.get("offsets"),
                   r.get("sorted_pairs"), r.get("pair_pos"), ws if histogram else None, stream)
    return r


def profile_enable(on: bool = True):
    lib.moe_profile_enable(1 if on else 0)


def profile_reset():
    lib.moe_profile_reset()


def profile_results() -> dict:
    """{kernel name: (launches, total ms)} from the hipEvent hooks."""
    res = {}
    for i in range(lib.moe_profile_num_kernels()):
        n, ms = C.c_int64(0), C.c_double(0.0)
        _check(lib.moe_profile_query(i, C.byref(n), C.byref(ms)))
        res[lib.moe_profile_kernel_name(i).decode()] = (n.value, ms.value)
    return res
