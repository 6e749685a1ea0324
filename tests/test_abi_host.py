"""Host-side checks of the C ABI: exports, capacity, status text, and every
argument error the library must report before enqueueing anything.  None of
these calls reaches the GPU, so they run without one."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5, 6


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert getattr(L, name) is not None


def test_capacity(L):
    assert L.moe_capacity(64, 2, 4, 1.25) == 40
    assert L.moe_capacity(4096, 2, 8, 1.25) == 1280
    assert L.moe_capacity(16384, 2, 8, 1.0) == 4096
    assert L.moe_capacity(8192, 2, 8, 1.25) == 2560
    assert L.moe_capacity(32768, 2, 32, 1.25) == 2560
    assert L.moe_capacity(10, 1, 4, 1.0) == 3
    assert L.moe_capacity(0, 2, 8, 1.25) == 0
    assert L.moe_capacity(-1, 2, 8, 1.0) == -1
    assert L.moe_capacity(10, 0, 8, 1.0) == -1
    assert L.moe_capacity(10, 1, 0, 1.0) == -1
    assert L.moe_capacity(10, 1, 4, 0.0) == -1
    assert L.moe_capacity(10, 1, 4, float("nan")) == -1


def test_status_strings(L):
    for s in range(8):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown status"
    assert L.moe_status_string(0) == b"ok"


def test_noalloc_scratch_covers_every_accepted_shape(L):
    """The dispatch workspace is bounded (at most 64 blocks of 16-byte cells
    per expert), so the no-allocation entry point's static array of
    MOE_NOALLOC_SCRATCH_BYTES = 128 KiB holds it for every shape the other
    checks accept."""
    biggest = 256 + 64 * 64 * 16
    for T, E, k in [((1 << 31) // 8 - 1, 64, 8), ((1 << 31) // 2 - 1, 64, 2), (1 << 20, 64, 2),
                    (65536 * 2, 64, 1), (1, 1, 1)]:
        need = L.moe_workspace_bytes(T, E, k)
        assert 256 < need <= biggest <= (128 << 10), (T, E, k, need)
    assert L.moe_workspace_bytes(1 << 20, 64, 2) == biggest


def test_workspace_bytes(L):
    assert L.moe_workspace_bytes(32768, 32, 2) > 0
    assert L.moe_workspace_bytes(0, 8, 2) > 0
    assert L.moe_workspace_bytes(-1, 8, 2) == 0
    assert L.moe_workspace_bytes(10, 65, 2) == 0
    assert L.moe_workspace_bytes(100000, 8, 2) >= L.moe_workspace_bytes(100, 8, 2)


P = 0x10000          # a fake, 16-byte aligned "device pointer": never dereferenced
MIS = 0x10008        # misaligned


def route(L, dtype=1, x=P, w=P, b=None, T=64, H=256, E=8, k=2, mode=0, seq=0, outs=(P, P, P)):
    return L.moe_route(None, dtype, x, w, b, T, H, E, k, mode, 0, seq, outs[0], outs[1], outs[2],
                       None)


def test_route_argument_errors(L):
    assert route(L, dtype=7) == DTYPE
    assert route(L, mode=3) == DTYPE
    assert route(L, T=-1) == SHAPE
    assert route(L, H=0) == SHAPE
    assert route(L, E=0) == SHAPE
    assert route(L, k=0) == SHAPE
    assert route(L, k=9, E=8) == SHAPE
    assert route(L, E=65, k=2) == UNSUP
    assert route(L, E=16, k=9) == UNSUP
    assert route(L, mode=1, seq=0) == SHAPE
    assert route(L, x=None) == NULL
    assert route(L, outs=(P, None, P)) == NULL
    assert route(L, H=200) == ALIGN
    assert route(L, x=MIS) == ALIGN
    assert route(L, dtype=0, H=6) == ALIGN
    assert route(L, H=(1 << 20) + 256) == UNSUP     # hidden sizes up to 2^20 (any multiple of 256)
    assert route(L, T=0, x=None, w=None, outs=(None, None, None)) == OK


def test_aux_argument_errors(L):
    a = lambda **kw: L.moe_aux_stats(None, kw.get("idx", P), kw.get("probs", P), kw.get("T", 64),  # noqa
                                     kw.get("E", 8), kw.get("k", 2), 0.01, kw.get("c", P), P, P, P,
                                     kw.get("ws", P), kw.get("wsb", 1 << 20))
    assert a(T=-1) == SHAPE
    assert a(E=0) == SHAPE
    assert a(k=3, E=2) == SHAPE
    assert a(E=70) == UNSUP
    assert a(c=None) == NULL
    assert a(idx=None) == NULL
    assert a(ws=None) == WS
    assert a(wsb=8) == WS


def test_dispatch_argument_errors(L):
    def d(**kw):
        return L.moe_dispatch(None, kw.get("dtype", 1), kw.get("x", P), kw.get("idx", P),
                              kw.get("T", 64), kw.get("H", 256), kw.get("E", 8), kw.get("k", 2),
                              kw.get("C", 20), kw.get("xd", P), P, P, kw.get("kept", P), P,
                              kw.get("ws", P), kw.get("wsb", 1 << 20))
    assert d(dtype=5) == DTYPE
    assert d(C=-1) == SHAPE
    assert d(T=-1) == SHAPE
    assert d(k=9, E=8) == SHAPE
    assert d(E=100) == UNSUP
    assert d(H=4) == ALIGN                 # 8 bytes per bf16 row: not a 16-byte multiple
    assert d(kept=None) == NULL
    assert d(x=None) == NULL                 # x needed when x_disp is written
    assert d(xd=None, kept=None) == NULL     # indices-only mode still validates
    assert d(x=MIS) == ALIGN
    assert d(ws=None) == WS
    assert d(wsb=4) == WS


def test_expert_ffn_argument_errors(L):
    def f(**kw):
        return L.moe_expert_ffn(None, kw.get("dtype", 1), kw.get("act", 0), kw.get("xd", P),
                                kw.get("kept", P), kw.get("E", 8), kw.get("C", 64),
                                kw.get("H", 256), kw.get("I", 256), kw.get("w1", P),
                                kw.get("w3", P), kw.get("w2", P), kw.get("b1", None),
                                kw.get("b2", None), kw.get("h", P), kw.get("y", P),
                                kw.get("ws", None), kw.get("wsb", 0))
    assert f(dtype=2) == DTYPE
    assert f(act=5) == DTYPE
    assert f(E=0) == SHAPE
    assert f(C=-1) == SHAPE
    assert f(H=0) == SHAPE
    assert f(E=65) == UNSUP
    assert f(w3=None) == NULL                 # SwiGLU needs the up matrix
    assert f(act=1, w3=None) == NULL          # GELU needs b1
    assert f(kept=None) == NULL
    assert f(h=None) == NULL
    assert f(H=200) == ALIGN
    assert f(I=200) == ALIGN
    assert f(w1=MIS) == ALIGN
    assert f(ws=MIS, wsb=1 << 30) == ALIGN
    assert f(C=0, xd=None, h=None, y=None) == OK
    # 32-bit buffer ranges: one expert's weight matrix below 2^31 bytes, one
    # expert's fp32 output rows below 2^32 bytes
    assert f(H=32768, I=32768) == UNSUP
    assert f(C=1 << 20, H=1024, I=1024) == UNSUP


def test_expert_ffn_gather_argument_errors(L):
    def f(**kw):
        return L.moe_expert_ffn_gather(None, kw.get("dtype", 1), kw.get("act", 0), kw.get("x", P),
                                       kw.get("st", P), kw.get("T", 100), kw.get("kept", P),
                                       kw.get("E", 8), kw.get("C", 64), kw.get("H", 256),
                                       kw.get("I", 256), kw.get("w1", P), kw.get("w3", P),
                                       kw.get("w2", P), None, None, kw.get("h", P), kw.get("y", P),
                                       None, 0)
    assert f(st=None) == NULL
    assert f(x=None) == NULL
    assert f(T=-1) == SHAPE
    assert f(x=MIS) == ALIGN
    assert f(H=200) == ALIGN
    assert f(T=1 << 22, H=1 << 10) == UNSUP   # 2^31 bytes of x: past 32-bit row offsets
    assert f(C=0, x=None, st=None, h=None, y=None) == OK


def test_expert_ffn_gather_combine_argument_errors(L):
    """The fused combine's own checks come first (its workspace is required),
    then moe_expert_ffn_gather's; every case below is refused before anything
    is enqueued."""
    def f(**kw):
        T, H = kw.get("T", 100), kw.get("H", 256)
        need = L.moe_expert_ffn_combine_ws_bytes(T, H)
        return L.moe_expert_ffn_gather_combine(
            None, kw.get("act", 0), kw.get("x", P), kw.get("st", P), kw.get("slot", P),
            kw.get("tw", P), T, kw.get("k", 2), kw.get("kept", P), kw.get("E", 8),
            kw.get("C", 64), H, kw.get("I", 256), kw.get("w1", P), kw.get("w3", P),
            kw.get("w2", P), None, None, kw.get("ysh", None), kw.get("h", P), kw.get("yd", P),
            kw.get("ws", P), kw.get("ws_bytes", need), kw.get("y", P))
    assert f(T=-1) == SHAPE
    assert f(k=0) == SHAPE
    assert f(k=9) == UNSUP
    assert f(k=3, E=2) == UNSUP
    assert f(T=0, x=None, st=None, slot=None, tw=None, y=None, ws=None) == OK
    assert f(slot=None) == NULL
    assert f(tw=None) == NULL
    assert f(y=None) == NULL
    assert f(kept=None) == NULL
    assert f(st=None) == NULL
    assert f(ws=None) == WS
    assert f(ws_bytes=16) == WS
    assert f(y=MIS) == ALIGN
    assert f(ws=MIS) == ALIGN
    assert f(ysh=MIS) == ALIGN
    assert f(E=64, C=1 << 20) == UNSUP      # y_disp past one 32-bit buffer range
    assert f(H=200) == ALIGN                # the products' tile width
    assert f(x=None) == NULL                # moe_expert_ffn_gather's checks follow
    assert f(T=1 << 22, H=1 << 10) == UNSUP


def test_expert_ffn_gather_combine_fp8_argument_errors(L):
    def f(**kw):
        T, H = kw.get("T", 100), kw.get("H", 256)
        need = L.moe_expert_ffn_combine_ws_bytes(T, H)
        return L.moe_expert_ffn_gather_combine_fp8(
            None, 0, P, P, P, P, T, 2, P, 8, 64, H, kw.get("I", 256), P, P, P,
            kw.get("s1", P), kw.get("s3", P), kw.get("s2", P), None, None, None, P, P,
            kw.get("ws", P), kw.get("ws_bytes", need), P)
    assert f(s1=None) == NULL
    assert f(s3=None) == NULL          # SwiGLU needs the up matrix's scales
    assert f(s2=None) == NULL
    assert f(ws_bytes=16) == WS
    assert f(H=200) == ALIGN
    assert f(T=-1) == SHAPE


def test_expert_ffn_combine_workspace_size(L):
    # the split tail's workspace, then one 4-byte counter per token and
    # 128-column output tile, rounded up to 256 bytes
    base = L.moe_expert_ffn_ws_bytes()
    assert L.moe_expert_ffn_combine_ws_bytes(32768, 2048) == base + 32768 * 16 * 4
    assert L.moe_expert_ffn_combine_ws_bytes(3, 256) == base + 256
    assert L.moe_expert_ffn_combine_ws_bytes(-1, 256) == 0


def test_expert_ffn_workspace_size(L):
    # one 256 x 256 fp32 partial tile per compute unit, then a 4-byte tile
    # counter per compute unit, rounded up to 256 bytes
    n = L.moe_expert_ffn_ws_bytes()
    tile = 256 * 256 * 4
    cus = n // tile
    assert cus >= 1 and n - cus * tile == (cus * 4 + 255) // 256 * 256


def test_combine_argument_errors(L):
    def c(**kw):
        return L.moe_combine(None, kw.get("dtype", 1), kw.get("yd", P), kw.get("slot", P), P,
                             kw.get("T", 64), kw.get("H", 256), kw.get("k", 2),
                             kw.get("ys", None), kw.get("y", P))
    assert c(dtype=9) == DTYPE
    assert c(T=-1) == SHAPE
    assert c(k=0) == SHAPE
    assert c(k=9) == UNSUP
    assert c(H=4) == ALIGN
    assert c(slot=None) == NULL
    assert c(yd=None) == NULL                 # the expert rows are always read through slot
    assert c(yd=MIS) == ALIGN
    assert c(y=MIS) == ALIGN
    assert c(ys=MIS) == ALIGN
    assert c(T=0, slot=None, y=None) == OK


def test_fp8_argument_errors(L):
    def qz(**kw):
        return L.moe_quantize_fp8(None, kw.get("w", P), kw.get("E", 2), kw.get("K", 64),
                                  kw.get("N", 64), kw.get("q", P), kw.get("s", P))
    assert qz(E=-1) == SHAPE
    assert qz(K=1 << 22) == UNSUP
    assert qz(K=40) == ALIGN
    assert qz(q=MIS) == ALIGN
    assert qz(w=None) == NULL
    assert qz(E=0, w=None) == OK
    assert L.moe_dequantize_fp8(None, P, None, 2, 64, 64, P) == NULL

    def ffn(**kw):
        return L.moe_expert_ffn_fp8(None, kw.get("act", 0), P, P, kw.get("E", 2), kw.get("C", 64),
                                    kw.get("H", 256), kw.get("I", 256), P, kw.get("w3", P), P,
                                    kw.get("s1", P), kw.get("s3", P), kw.get("s2", P), None, None,
                                    P, P, None, 0)
    assert ffn(s1=None) == NULL
    assert ffn(s2=None) == NULL
    assert ffn(s3=None) == NULL
    assert ffn(H=200) == ALIGN
    assert ffn(s1=MIS) == ALIGN
    assert ffn(C=0) == OK
    assert L.moe_expert_ffn_gather_fp8(None, 0, P, None, 64, P, 2, 64, 256, 256, P, P, P, P, P,
                                       P, None, None, P, P, None, 0) == NULL


def test_dispatch_aux_argument_errors(L):
    ws_ok = L.moe_workspace_bytes(64, 8, 2)

    def d(**kw):
        return L.moe_dispatch_aux(None, kw.get("dtype", 1), kw.get("x", P), kw.get("idx", P),
                                  kw.get("probs", P), kw.get("T", 64), kw.get("H", 256),
                                  kw.get("E", 8), kw.get("k", 2), kw.get("C", 20), 0.01,
                                  kw.get("xd", P), P, P, P, P, kw.get("counts", P), P, P, P,
                                  kw.get("ws", P), kw.get("wsb", ws_ok))
    assert d(dtype=7) == DTYPE
    assert d(k=9) == SHAPE
    assert d(E=65, k=2) == UNSUP
    assert d(H=4) == ALIGN
    assert d(probs=None) == NULL
    assert d(counts=None) == NULL
    assert d(ws=None) == WS
    assert d(wsb=16) == WS
    assert d(ws=MIS) == ALIGN
    assert d(xd=MIS) == ALIGN


def test_dispatch_bwd_argument_errors(L):
    def d(**kw):
        return L.moe_dispatch_bwd(None, kw.get("dxd", P), kw.get("slot", P), kw.get("T", 64),
                                  kw.get("H", 256), kw.get("k", 2), kw.get("add", None),
                                  kw.get("dx", P))
    assert d(T=-1) == SHAPE
    assert d(k=9) == UNSUP
    assert d(H=4) == ALIGN
    assert d(dxd=None) == NULL               # the copies' gradients are read through slot
    assert d(slot=None) == NULL
    assert d(dx=None) == NULL
    assert d(dxd=MIS) == ALIGN
    assert d(add=MIS) == ALIGN
    assert d(T=0, dxd=None, slot=None, dx=None) == OK


def route_bwd(L, dtype=1, mode=0, x=P, w=P, probs=P, idx=P, tw=P, dw=P, f=P, T=64, H=256, E=8,
              k=2, seq=0, dl=P, dx=P, dwr=P, dbr=None, ws=P, wsb=1 << 30):
    return L.moe_route_bwd(None, dtype, mode, x, w, probs, idx, tw, dw, f, 0.01, 0.5, T, H, E, k,
                           seq, dl, dx, dwr, dbr, ws, wsb)


def test_route_bwd_argument_errors(L):
    assert route_bwd(L, dtype=7) == DTYPE
    assert route_bwd(L, mode=3) == DTYPE
    assert route_bwd(L, T=-1) == SHAPE
    assert route_bwd(L, k=9, E=8) == SHAPE
    assert route_bwd(L, E=65, k=2) == UNSUP
    assert route_bwd(L, mode=1, seq=-1) == SHAPE
    assert route_bwd(L, H=12) == ALIGN
    assert route_bwd(L, dwr=None) == NULL
    assert route_bwd(L, probs=None) == NULL
    assert route_bwd(L, dx=MIS) == ALIGN
    assert route_bwd(L, x=MIS) == ALIGN          # 16-byte vector loads of x rows
    assert route_bwd(L, w=MIS) == ALIGN          # and of W_r rows
    assert route_bwd(L, ws=MIS) == ALIGN         # 16-byte partial-sum stores
    assert route_bwd(L, ws=None) == WS
    assert route_bwd(L, wsb=16) == WS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()
