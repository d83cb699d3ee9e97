"""The C-ABI library without a GPU: it loads, exports every function that
include/moe_q2.h declares, and rejects bad arguments before any HIP call
(validation runs first, so these calls never reach the device)."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q2.h")
LIB = os.path.join(ROOT, "bit_quantized_expert_router_amd", "libmoe_q2.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_expert_router_amd import binding
    return binding.lib


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), n


def test_binding_lists_all_exports():
    from bit_quantized_expert_router_amd import binding
    assert sorted(binding.EXPORTS) == declared_functions()


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(-3) == b"MOE_ERR_WORKSPACE"


def test_workspace_sizes(lib):
    from bit_quantized_expert_router_amd import binding as B
    assert B.moe_workspace_bytes(B.MOE_OP_DECODE, 1, 512, 10, 3072, 768) > 0
    # header + h~ rows of T*k + T pairs
    assert B.moe_workspace_bytes(B.MOE_OP_DECODE, 8, 512, 10, 3072, 768) >= 88 * 768 * 2
    assert B.moe_workspace_bytes(B.MOE_OP_DECODE, 9, 512, 10, 3072, 768) == 0
    assert B.moe_workspace_bytes(B.MOE_OP_ROUTE_GEMV, 5, 512, 10, 3072, 0) == 0
    p = B.moe_workspace_bytes(B.MOE_OP_PREFILL, 1024, 512, 10, 3072, 768)
    # x16 + h + y at least
    assert p >= 1024 * 3072 * 2 + 11264 * 768 * 2 + 11264 * 3072 * 2
    assert B.moe_workspace_bytes(B.MOE_OP_ROUTE, 1024, 512, 10, 3072, 768) >= 1024 * 10 * 4


FAKE = 0x100000  # aligned, never dereferenced: validation fails first


def route(lib, **kw):
    a = dict(logits=FAKE, T=4, E=64, k=4, ids=FAKE, w=FAKE, counts=None, offsets=None,
             sp=None, pp=None, ws=None, wsb=0)
    a.update(kw)
    return lib.moe_route_topk(C.c_void_p(a["logits"]), a["T"], a["E"], a["k"], C.c_void_p(a["ids"]),
                              C.c_void_p(a["w"]), C.c_void_p(a["counts"]), C.c_void_p(a["offsets"]),
                              C.c_void_p(a["sp"]), C.c_void_p(a["pp"]), C.c_void_p(a["ws"]),
                              a["wsb"], None)


def gemv(lib, **kw):
    a = dict(x=FAKE, xd=1, T=1, W=FAKE, E=64, H=1024, k=4, lg=None, ids=FAKE, w=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.moe_route_topk_gemv(C.c_void_p(a["x"]), a["xd"], a["T"], C.c_void_p(a["W"]), a["E"], a["H"],
                                   a["k"], C.c_void_p(a["lg"]), C.c_void_p(a["ids"]), C.c_void_p(a["w"]),
                                   C.c_void_p(a["ws"]), a["wsb"], None)


def test_route_gemv_validation(lib):
    assert gemv(lib, x=None) == -1
    assert gemv(lib, W=None) == -1
    assert gemv(lib, T=0) == -1
    assert gemv(lib, T=5) == -2
    assert gemv(lib, E=2048) == -2
    assert gemv(lib, k=17) == -2
    assert gemv(lib, E=3, k=4) == -1
    assert gemv(lib, H=1000) == -1
    assert gemv(lib, H=16384) == -2
    assert gemv(lib, xd=9) == -1
    assert gemv(lib, W=FAKE + 8) == -1
    assert gemv(lib, ws=None) == -3
    assert gemv(lib, wsb=16) == -3
    assert gemv(lib, ids=None) == -1                      # only one routing output
    assert gemv(lib, ids=None, w=None) == -1              # nothing requested
    assert gemv(lib, ids=None, w=None, lg=FAKE + 2) == -1  # unaligned logits
    assert lib.moe_workspace_bytes(3, 4, 512, 10, 3072, 0) >= 256 + 4 * 512 * 4
    assert lib.moe_workspace_bytes(3, 5, 512, 10, 3072, 0) == 0


def test_route_validation(lib):
    assert route(lib, logits=None) == -1
    assert route(lib, T=0) == -1
    assert route(lib, k=0) == -1
    assert route(lib, k=65) == -2      # k > 16 is unsupported
    assert route(lib, E=2048, k=4) == -2
    assert route(lib, E=3, k=4) == -1  # k > E
    assert route(lib, counts=FAKE) == -1   # partial histogram outputs
    assert route(lib, counts=FAKE, offsets=FAKE, sp=FAKE, pp=FAKE) == -3  # no workspace
    assert route(lib, counts=FAKE, offsets=FAKE, sp=FAKE, pp=FAKE, ws=FAKE, wsb=16) == -3
    assert route(lib, counts=FAKE, offsets=FAKE, sp=FAKE, pp=FAKE, ws=FAKE + 4, wsb=1 << 30) == -1
    assert b"workspace" in lib.moe_last_error()


def forward(lib, which, **kw):
    from bit_quantized_expert_router_amd.binding import _Layer
    a = dict(experts=FAKE, shared=FAKE, stride=245760, E=64, H=1024, I=256, x=FAKE, xd=0, T=1,
             ids=FAKE, w=FAKE, k=4, res=None, out=FAKE + (1 << 34), od=0, flags=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    L = _Layer(a["experts"], a["shared"], a["stride"], a["E"], a["H"], a["I"])
    if which.endswith("tiered"):
        from bit_quantized_expert_router_amd.binding import _TieredLayer
        TL = _TieredLayer(a.get("slots", FAKE + (1 << 35)), a.get("slot_of", FAKE), a["experts"], a["shared"],
                          a["stride"], a.get("S", 8), a["E"], a["H"], a["I"])
        if which == "decode_tiered":
            return lib.moe_expert_forward_decode_tiered(C.byref(TL), C.c_void_p(a["x"]), a["xd"], a["T"],
                                                        C.c_void_p(a.get("logits", FAKE)), a["k"],
                                                        C.c_void_p(a["ids"]), C.c_void_p(a["w"]),
                                                        C.c_void_p(a["res"]), C.c_void_p(a["out"]), a["od"],
                                                        a["flags"], C.c_void_p(a.get("usage")),
                                                        C.c_void_p(a["ws"]), a["wsb"], None)
        return lib.moe_expert_forward_prefill_tiered(C.byref(TL), C.c_void_p(a["x"]), a["xd"], a["T"],
                                                     C.c_void_p(a["ids"]), C.c_void_p(a["w"]), a["k"],
                                                     C.c_void_p(a.get("counts", FAKE)),
                                                     C.c_void_p(a.get("offsets", FAKE)),
                                                     C.c_void_p(a.get("sp", FAKE)), C.c_void_p(a.get("pp", FAKE)),
                                                     C.c_void_p(a["res"]), C.c_void_p(a["out"]), a["od"],
                                                     a["flags"], C.c_void_p(a["ws"]), a["wsb"], None)
    if which == "routed":
        return lib.moe_expert_forward_decode_routed(C.byref(L), C.c_void_p(a["x"]), a["xd"], a["T"],
                                                    C.c_void_p(a.get("logits", FAKE)), a["k"],
                                                    C.c_void_p(a["ids"]), C.c_void_p(a["w"]),
                                                    C.c_void_p(a["res"]), C.c_void_p(a["out"]),
                                                    a["od"], a["flags"], C.c_void_p(a["ws"]),
                                                    a["wsb"], None)
    if which == "decode":
        return lib.moe_expert_forward_decode(C.byref(L), C.c_void_p(a["x"]), a["xd"], a["T"],
                                             C.c_void_p(a["ids"]), C.c_void_p(a["w"]), a["k"],
                                             C.c_void_p(a["res"]), C.c_void_p(a["out"]), a["od"],
                                             a["flags"], C.c_void_p(a["ws"]), a["wsb"], None)
    return lib.moe_expert_forward_prefill(C.byref(L), C.c_void_p(a["x"]), a["xd"], a["T"],
                                          C.c_void_p(a["ids"]), C.c_void_p(a["w"]), a["k"],
                                          C.c_void_p(a.get("counts", FAKE)), C.c_void_p(a.get("offsets", FAKE)),
                                          C.c_void_p(a.get("sp", FAKE)), C.c_void_p(a.get("pp", FAKE)),
                                          C.c_void_p(a["res"]), C.c_void_p(a["out"]), a["od"],
                                          a["flags"], C.c_void_p(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("which", ["decode", "routed", "prefill", "decode_tiered", "prefill_tiered"])
def test_forward_validation(lib, which):
    assert forward(lib, which, experts=None) == -1
    assert forward(lib, which, x=None) == -1
    assert forward(lib, which, out=FAKE) == -1          # aliases x
    assert forward(lib, which, H=1000) == -1            # not a multiple of 256
    assert forward(lib, which, H=16384, stride=1 << 30) == -2
    assert forward(lib, which, stride=1000) == -1       # too small
    assert forward(lib, which, stride=245760 + 128) == -1  # not a multiple of 256
    assert forward(lib, which, experts=FAKE + 16) == -1    # unaligned weights
    assert forward(lib, which, k=0) == -1
    assert forward(lib, which, k=17) == -2
    assert forward(lib, which, E=3, k=4) == -1
    assert forward(lib, which, E=2000) == -2
    assert forward(lib, which, xd=7) == -1
    assert forward(lib, which, flags=2) == -1
    assert forward(lib, which, T=0) == -1
    assert forward(lib, which, ws=None) == -3
    assert forward(lib, which, wsb=100) == -3
    assert forward(lib, which, ws=FAKE + 8) == -1
    assert forward(lib, which, res=FAKE + 8) == -1         # unaligned residual
    # out shares bytes with x: fp32 x of T = 1, H = 1024 covers 4096 bytes
    assert forward(lib, which, out=FAKE + 16) == -1
    assert forward(lib, which, out=FAKE - 4096 + 16) == -1
    assert forward(lib, which, out=FAKE + 2048, xd=1, od=1, T=2) == -1   # bf16 x of T = 2 covers 4096
    assert b"overlap" in lib.moe_last_error()
    # residual partly over out (residual == out itself is allowed)
    assert forward(lib, which, res=FAKE + (1 << 34) + 1024) == -1
    assert b"residual" in lib.moe_last_error()
    if which in ("decode", "routed", "decode_tiered"):
        assert forward(lib, which, T=9) == -2
    if which in ("routed", "decode_tiered"):
        assert forward(lib, which, logits=None) == -1
        assert forward(lib, which, ids=None) == -1            # only one routing output
        assert forward(lib, which, logits=FAKE + 2) == -1     # unaligned
        assert forward(lib, which, ids=None, w=None, wsb=100) == -3   # outputs are optional
    elif which in ("prefill", "prefill_tiered"):
        assert forward(lib, which, counts=None) == -1
        assert forward(lib, which, T=(1 << 17) + 1) == -2


@pytest.mark.parametrize("which", ["decode_tiered", "prefill_tiered"])
def test_tier_validation(lib, which):
    """The tier's own arguments are checked after the untiered ones and
    before the arena's memory type is looked up."""
    assert forward(lib, which, experts=None) == -1       # the arena
    assert forward(lib, which, slot_of=None) == -1
    assert b"slot_of" in lib.moe_last_error()
    assert forward(lib, which, slot_of=FAKE + 2) == -1   # unaligned
    assert forward(lib, which, S=-1) == -1
    assert forward(lib, which, S=65) == -1               # more slots than experts
    assert b"num_slots" in lib.moe_last_error()
    assert forward(lib, which, slots=None) == -1
    assert forward(lib, which, slots=FAKE + 128) == -1   # unaligned slots
    if which == "decode_tiered":
        assert forward(lib, which, usage=FAKE + 4) == -1
        assert b"usage_counts" in lib.moe_last_error()


def test_usage_update_validation(lib):
    f = lib.moe_expert_usage_update
    assert f(C.c_void_p(FAKE), 8, 0, C.c_void_p(FAKE), None) == -1
    assert f(C.c_void_p(FAKE), 8, 2000, C.c_void_p(FAKE), None) == -2
    assert f(C.c_void_p(FAKE), -1, 64, C.c_void_p(FAKE), None) == -1
    assert f(C.c_void_p(FAKE), 1 << 31, 64, C.c_void_p(FAKE), None) == -1
    assert f(None, 8, 64, C.c_void_p(FAKE), None) == -1
    assert f(C.c_void_p(FAKE), 8, 64, None, None) == -1
    assert f(C.c_void_p(FAKE + 2), 8, 64, C.c_void_p(FAKE), None) == -1
    assert f(C.c_void_p(FAKE), 8, 64, C.c_void_p(FAKE + 4), None) == -1
    assert f(None, 0, 64, None, None) == 0               # nothing to count: no launch


def apply(lib, **kw):
    import numpy as np
    a = dict(arena=FAKE, stride=245760, E=8, S=3, old=[-1, -1, -1], new=[1, 2, 3], slots=FAKE + (1 << 35),
             slot_of=FAKE + (1 << 36))
    a.update(kw)
    old = None if a["old"] is None else np.asarray(a["old"], dtype=np.int32)
    new = None if a["new"] is None else np.asarray(a["new"], dtype=np.int32)
    return lib.moe_residency_apply(C.c_void_p(a["arena"]), a["stride"], a["E"], a["S"],
                                   old.ctypes.data_as(C.c_void_p) if a["old"] is not None else None,
                                   new.ctypes.data_as(C.c_void_p) if a["new"] is not None else None,
                                   C.c_void_p(a["slots"]), C.c_void_p(a["slot_of"]), None)


def test_residency_apply_validation(lib):
    assert apply(lib, E=0) == -1
    assert apply(lib, E=2000) == -2
    assert apply(lib, S=9) == -1
    assert apply(lib, arena=None) == -1
    assert apply(lib, slot_of=None) == -1
    assert apply(lib, slots=None) == -1
    assert apply(lib, old=None) == -1
    assert apply(lib, stride=1000) == -1
    assert apply(lib, arena=FAKE + 16) == -1
    assert apply(lib, slot_of=FAKE + 2) == -1
    assert apply(lib, new=[1, 1, 3]) == -1               # an expert twice
    assert b"twice" in lib.moe_last_error()
    assert apply(lib, new=[1, 8, 3]) == -1               # not an expert
    assert apply(lib, old=[-2, -1, -1]) == -1
    assert apply(lib, old=[2, -1, -1], new=[1, 2, 3]) == -1   # expert 2 changes slot
    assert b"moves" in lib.moe_last_error()
    # S = 0 with no arrays is valid and enqueues nothing
    assert apply(lib, S=0, old=None, new=None, slots=None) == 0


def test_profile_hooks_host_only(lib):
    from bit_quantized_expert_router_amd import binding as B
    B.profile_enable(False)
    B.profile_reset()
    res = B.profile_results()
    assert "decode_gateup_kernel" in res and "prefill_gateup_kernel" in res
    assert all(v == (0, 0.0) for v in res.values())
