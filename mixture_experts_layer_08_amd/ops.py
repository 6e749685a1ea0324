"""Python binding of the C ABI: one function per entry point, same names.

Each function only marshals arguments: it checks tensor dtypes, devices and
contiguity, allocates missing outputs with torch (device memory is the only
thing torch supplies), passes raw device pointers and the current HIP
stream to the library, and turns a non-zero status into MoEError.  All
arithmetic runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._lib import ACTS, MOE_BF16, MOE_F32, ROUTE_MODES, check, lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _want(t: Optional[torch.Tensor], shape, dtype, dev) -> torch.Tensor:
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"output must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def moe_capacity(T: int, k: int, E: int, cf: float) -> int:
    c = lib().moe_capacity(int(T), int(k), int(E), float(cf))
    if c < 0:
        raise ValueError("moe_capacity: argument out of range")
    return int(c)


def moe_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(lib().moe_workspace_bytes(int(T), int(E), int(k)))


def moe_route(x: torch.Tensor, w_r: torch.Tensor, b_r: Optional[torch.Tensor], k: int, *,
              mode: str = "softmax", seed: int = 0, seq_len: int = 0,
              topk_idx: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
              probs: Optional[torch.Tensor] = None, keys: Optional[torch.Tensor] = None,
              want_keys: bool = False
              ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    T, H = x.shape
    E = w_r.shape[1]
    dev = x.device
    topk_idx = _want(topk_idx, (T, k), torch.int32, dev)
    topk_w = _want(topk_w, (T, k), torch.float32, dev)
    probs = _want(probs, (T, E), torch.float32, dev)
    if want_keys or keys is not None:
        keys = _want(keys, (T, E), torch.float32, dev)
    if w_r.dtype != x.dtype or tuple(w_r.shape) != (H, E):
        raise ValueError("w_r must be [H, E] with x's dtype")
    if b_r is not None and (b_r.dtype != torch.float32 or tuple(b_r.shape) != (E,)):
        raise ValueError("b_r must be fp32 [E]")
    st = lib().moe_route(_stream(dev), _dtype_code(x), _ptr(x), _ptr(w_r), _ptr(b_r), T, H, E, k,
                         ROUTE_MODES[mode], int(seed) & (2 ** 64 - 1), int(seq_len),
                         _ptr(topk_idx), _ptr(topk_w), _ptr(probs), _ptr(keys))
    check("moe_route", st)
    return topk_idx, topk_w, probs, keys


def moe_aux_stats(topk_idx: torch.Tensor, probs: torch.Tensor, E: int, alpha: float, *,
                  ws: Optional[torch.Tensor] = None, counts=None, f=None, p=None, l_aux=None):
    """(counts, f, p, l_aux).  ws as for moe_dispatch (shared with it)."""
    T, k = topk_idx.shape
    dev = probs.device
    counts = _want(counts, (E,), torch.int32, dev)
    f = _want(f, (E,), torch.float32, dev)
    p = _want(p, (E,), torch.float32, dev)
    l_aux = _want(l_aux, (1,), torch.float32, dev)
    if ws is None:
        ws = torch.zeros(max(16, moe_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    st = lib().moe_aux_stats(_stream(dev), _ptr(topk_idx), _ptr(probs), T, E, k, float(alpha),
                             _ptr(counts), _ptr(f), _ptr(p), _ptr(l_aux), _ptr(ws), ws.numel())
    check("moe_aux_stats", st)
    return counts, f, p, l_aux


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, C: int, *,
                 ws: Optional[torch.Tensor] = None, x_disp=None, slot=None, slot_token=None,
                 kept=None, dropped=None, copy: bool = True):
    """copy=False: indices only (slot, slot_token, kept, dropped); x_disp is
    then returned as None (for moe_expert_ffn_gather).  A ws passed in must
    have been zero-filled before its first use (each call leaves it zero);
    without one a zero-filled workspace is allocated."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    x_disp = _want(x_disp, (E, C, H), x.dtype, dev) if copy else None
    slot = _want(slot, (T, k), torch.int32, dev)
    slot_token = _want(slot_token, (E, C), torch.int32, dev)
    kept = _want(kept, (E,), torch.int32, dev)
    dropped = _want(dropped, (1,), torch.int32, dev)
    if ws is None:
        ws = torch.zeros(max(16, moe_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    st = lib().moe_dispatch(_stream(dev), _dtype_code(x), _ptr(x), _ptr(topk_idx), T, H, E, k, C,
                            _ptr(x_disp), _ptr(slot), _ptr(slot_token), _ptr(kept),
                            _ptr(dropped), _ptr(ws), ws.numel())
    check("moe_dispatch", st)
    return x_disp, slot, slot_token, kept, dropped


def moe_dispatch_aux(x: torch.Tensor, topk_idx: torch.Tensor, probs: torch.Tensor, E: int, C: int,
                     alpha: float, *, ws: Optional[torch.Tensor] = None, x_disp=None, slot=None,
                     slot_token=None, kept=None, dropped=None, counts=None, f=None, p=None,
                     l_aux=None, copy: bool = True):
    """moe_dispatch and moe_aux_stats in one pass: (x_disp, slot, slot_token,
    kept, dropped, counts, f, p, l_aux).  ws as for moe_dispatch."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    x_disp = _want(x_disp, (E, C, H), x.dtype, dev) if copy else None
    slot = _want(slot, (T, k), torch.int32, dev)
    slot_token = _want(slot_token, (E, C), torch.int32, dev)
    kept = _want(kept, (E,), torch.int32, dev)
    dropped = _want(dropped, (1,), torch.int32, dev)
    counts = _want(counts, (E,), torch.int32, dev)
    f = _want(f, (E,), torch.float32, dev)
    p = _want(p, (E,), torch.float32, dev)
    l_aux = _want(l_aux, (1,), torch.float32, dev)
    if ws is None:
        ws = torch.zeros(max(16, moe_workspace_bytes(T, E, k)), dtype=torch.uint8, device=dev)
    st = lib().moe_dispatch_aux(_stream(dev), _dtype_code(x), _ptr(x), _ptr(topk_idx), _ptr(probs),
                                T, H, E, k, C, float(alpha), _ptr(x_disp), _ptr(slot),
                                _ptr(slot_token), _ptr(kept), _ptr(dropped), _ptr(counts), _ptr(f),
                                _ptr(p), _ptr(l_aux), _ptr(ws), ws.numel())
    check("moe_dispatch_aux", st)
    return x_disp, slot, slot_token, kept, dropped, counts, f, p, l_aux


def moe_dispatch_aux_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, probs: torch.Tensor, E: int,
                             C: int, alpha: float, *, x_disp=None, slot=None, slot_token=None,
                             kept=None, dropped=None, counts=None, f=None, p=None, l_aux=None,
                             copy: bool = True):
    """moe_dispatch_aux with the library's static device workspace instead of
    a workspace argument (same outputs).  Pass every output to allocate
    nothing here either."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    x_disp = _want(x_disp, (E, C, H), x.dtype, dev) if copy else None
    slot = _want(slot, (T, k), torch.int32, dev)
    slot_token = _want(slot_token, (E, C), torch.int32, dev)
    kept = _want(kept, (E,), torch.int32, dev)
    dropped = _want(dropped, (1,), torch.int32, dev)
    counts = _want(counts, (E,), torch.int32, dev)
    f = _want(f, (E,), torch.float32, dev)
    p = _want(p, (E,), torch.float32, dev)
    l_aux = _want(l_aux, (1,), torch.float32, dev)
    st = lib().moe_dispatch_aux_noalloc(_stream(dev), _dtype_code(x), _ptr(x), _ptr(topk_idx),
                                        _ptr(probs), T, H, E, k, C, float(alpha), _ptr(x_disp),
                                        _ptr(slot), _ptr(slot_token), _ptr(kept), _ptr(dropped),
                                        _ptr(counts), _ptr(f), _ptr(p), _ptr(l_aux))
    check("moe_dispatch_aux_noalloc", st)
    return x_disp, slot, slot_token, kept, dropped, counts, f, p, l_aux


def moe_expert_ffn_ws_bytes() -> int:
    return int(lib().moe_expert_ffn_ws_bytes())


def moe_expert_ffn(x_disp: torch.Tensor, kept: torch.Tensor, w1: torch.Tensor,
                   w3: Optional[torch.Tensor], w2: torch.Tensor, b1: Optional[torch.Tensor] = None,
                   b2: Optional[torch.Tensor] = None, *, act: str = "swiglu",
                   h_ws: Optional[torch.Tensor] = None, y_disp: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None):
    """ws: optional uint8 workspace of moe_expert_ffn_ws_bytes() bytes,
    zero-filled when allocated (its tile counters must start at zero; every
    call leaves them zero); None runs every round of tiles whole."""
    E, C, H = x_disp.shape
    I = w1.shape[2]
    dev = x_disp.device
    if tuple(w1.shape) != (E, H, I) or tuple(w2.shape) != (E, I, H):
        raise ValueError("w1 must be [E, H, I] and w2 [E, I, H]")
    if w3 is not None and tuple(w3.shape) != (E, H, I):
        raise ValueError("w3 must be [E, H, I]")
    for t in (w1, w3, w2, b1, b2):
        if t is not None and t.dtype != x_disp.dtype:
            raise ValueError("weights and biases must have x_disp's dtype")
    h_ws = _want(h_ws, (E, C, I), x_disp.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    st = lib().moe_expert_ffn(_stream(dev), _dtype_code(x_disp), ACTS[act], _ptr(x_disp),
                              _ptr(kept), E, C, H, I, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(b1),
                              _ptr(b2), _ptr(h_ws), _ptr(y_disp), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size())
    check("moe_expert_ffn", st)
    return y_disp, h_ws


def moe_expert_ffn_gather(x: torch.Tensor, slot_token: torch.Tensor, kept: torch.Tensor,
                          w1: torch.Tensor, w3: Optional[torch.Tensor], w2: torch.Tensor,
                          b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None, *,
                          act: str = "swiglu", h_ws: Optional[torch.Tensor] = None,
                          y_disp: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """moe_expert_ffn reading each expert's rows straight from x via slot_token."""
    T, H = x.shape
    E, C = slot_token.shape
    I = w1.shape[2]
    dev = x.device
    if tuple(w1.shape) != (E, H, I) or tuple(w2.shape) != (E, I, H):
        raise ValueError("w1 must be [E, H, I] and w2 [E, I, H]")
    if w3 is not None and tuple(w3.shape) != (E, H, I):
        raise ValueError("w3 must be [E, H, I]")
    for t in (w1, w3, w2, b1, b2):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("weights and biases must have x's dtype")
    if slot_token.dtype != torch.int32:
        raise ValueError("slot_token must be int32")
    h_ws = _want(h_ws, (E, C, I), x.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    st = lib().moe_expert_ffn_gather(_stream(dev), _dtype_code(x), ACTS[act], _ptr(x),
                                     _ptr(slot_token), T, _ptr(kept), E, C, H, I, _ptr(w1),
                                     _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2), _ptr(h_ws),
                                     _ptr(y_disp), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size())
    check("moe_expert_ffn_gather", st)
    return y_disp, h_ws


def moe_expert_ffn_combine_ws_bytes(T: int, H: int) -> int:
    return int(lib().moe_expert_ffn_combine_ws_bytes(T, H))


def moe_expert_ffn_gather_combine(x: torch.Tensor, slot_token: torch.Tensor, slot: torch.Tensor,
                                  topk_w: torch.Tensor, kept: torch.Tensor, w1: torch.Tensor,
                                  w3: Optional[torch.Tensor], w2: torch.Tensor,
                                  b1: Optional[torch.Tensor] = None,
                                  b2: Optional[torch.Tensor] = None, *, act: str = "swiglu",
                                  y_shared: Optional[torch.Tensor] = None,
                                  h_ws: Optional[torch.Tensor] = None,
                                  y_disp: Optional[torch.Tensor] = None,
                                  ws: Optional[torch.Tensor] = None,
                                  y: Optional[torch.Tensor] = None):
    """moe_expert_ffn_gather and moe_combine in one call: the down product's
    tiles write each token's bf16 output row once its last kept copy is in.
    ws: zero-filled once, at least moe_expert_ffn_combine_ws_bytes(T, H)
    bytes (every call leaves it zero).  Returns (y, y_disp, h_ws)."""
    T, H = x.shape
    E, C = slot_token.shape
    k = slot.shape[1]
    I = w1.shape[2]
    dev = x.device
    if x.dtype != torch.bfloat16:
        raise ValueError("the fused combine runs on bf16 activations")
    if tuple(w1.shape) != (E, H, I) or tuple(w2.shape) != (E, I, H):
        raise ValueError("w1 must be [E, H, I] and w2 [E, I, H]")
    if w3 is not None and tuple(w3.shape) != (E, H, I):
        raise ValueError("w3 must be [E, H, I]")
    for t in (w1, w3, w2, b1, b2):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("weights and biases must have x's dtype")
    if slot_token.dtype != torch.int32 or slot.dtype != torch.int32:
        raise ValueError("slot_token and slot must be int32")
    if tuple(slot.shape) != (T, k) or tuple(topk_w.shape) != (T, k) or topk_w.dtype != torch.float32:
        raise ValueError("slot must be int32 [T, k] and topk_w fp32 [T, k]")
    if y_shared is not None and (y_shared.dtype != torch.float32 or y_shared.numel() != T * H
                                 or not y_shared.is_contiguous()):
        raise ValueError("y_shared must be a contiguous fp32 [T, H] tensor")
    h_ws = _want(h_ws, (E, C, I), x.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    y = _want(y, (T, H), torch.bfloat16, dev)
    if ws is None:
        ws = torch.zeros(moe_expert_ffn_combine_ws_bytes(T, H), dtype=torch.uint8, device=dev)
    st = lib().moe_expert_ffn_gather_combine(
        _stream(dev), ACTS[act], _ptr(x), _ptr(slot_token), _ptr(slot), _ptr(topk_w), T, k,
        _ptr(kept), E, C, H, I, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2), _ptr(y_shared),
        _ptr(h_ws), _ptr(y_disp), _ptr(ws), ws.numel() * ws.element_size(), _ptr(y))
    check("moe_expert_ffn_gather_combine", st)
    return y, y_disp, h_ws


def moe_expert_ffn_gather_combine_fp8(x: torch.Tensor, slot_token: torch.Tensor,
                                      slot: torch.Tensor, topk_w: torch.Tensor, kept: torch.Tensor,
                                      w1q: torch.Tensor, w3q: Optional[torch.Tensor],
                                      w2q: torch.Tensor, s1: torch.Tensor,
                                      s3: Optional[torch.Tensor], s2: torch.Tensor,
                                      b1: Optional[torch.Tensor] = None,
                                      b2: Optional[torch.Tensor] = None, *, act: str = "swiglu",
                                      y_shared: Optional[torch.Tensor] = None,
                                      h_ws: Optional[torch.Tensor] = None,
                                      y_disp: Optional[torch.Tensor] = None,
                                      ws: Optional[torch.Tensor] = None,
                                      y: Optional[torch.Tensor] = None):
    """moe_expert_ffn_gather_combine on 8-bit weights (codes [E, N, K] and
    per-column scales as moe_quantize_fp8 returns them).  Returns
    (y, y_disp, h_ws)."""
    T, H = x.shape
    E, C = slot_token.shape
    k = slot.shape[1]
    I = w1q.shape[1]
    dev = x.device
    if x.dtype != torch.bfloat16:
        raise ValueError("the fused combine runs on bf16 activations")
    _check_fp8_weights(E, H, I, w1q, w3q, w2q, s1, s3, s2)
    if slot_token.dtype != torch.int32 or slot.dtype != torch.int32:
        raise ValueError("slot_token and slot must be int32")
    if tuple(slot.shape) != (T, k) or tuple(topk_w.shape) != (T, k) or topk_w.dtype != torch.float32:
        raise ValueError("slot must be int32 [T, k] and topk_w fp32 [T, k]")
    if y_shared is not None and (y_shared.dtype != torch.float32 or y_shared.numel() != T * H
                                 or not y_shared.is_contiguous()):
        raise ValueError("y_shared must be a contiguous fp32 [T, H] tensor")
    h_ws = _want(h_ws, (E, C, I), x.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    y = _want(y, (T, H), torch.bfloat16, dev)
    if ws is None:
        ws = torch.zeros(moe_expert_ffn_combine_ws_bytes(T, H), dtype=torch.uint8, device=dev)
    st = lib().moe_expert_ffn_gather_combine_fp8(
        _stream(dev), ACTS[act], _ptr(x), _ptr(slot_token), _ptr(slot), _ptr(topk_w), T, k,
        _ptr(kept), E, C, H, I, _ptr(w1q), _ptr(w3q), _ptr(w2q), _ptr(s1), _ptr(s3), _ptr(s2),
        _ptr(b1), _ptr(b2), _ptr(y_shared), _ptr(h_ws), _ptr(y_disp), _ptr(ws),
        ws.numel() * ws.element_size(), _ptr(y))
    check("moe_expert_ffn_gather_combine_fp8", st)
    return y, y_disp, h_ws


def moe_quantize_fp8(w: torch.Tensor, *, q: Optional[torch.Tensor] = None,
                     scale: Optional[torch.Tensor] = None):
    """bf16 weights [E, K, N] -> (e4m3 codes [E, N, K] uint8, fp32 scales
    [E, N]), one scale per expert and output column."""
    if w.dtype != torch.bfloat16 or w.dim() != 3:
        raise ValueError("w must be a bf16 [E, K, N] tensor")
    E, K, N = w.shape
    q = _want(q, (E, N, K), torch.uint8, w.device)
    scale = _want(scale, (E, N), torch.float32, w.device)
    st = lib().moe_quantize_fp8(_stream(w.device), _ptr(w), E, K, N, _ptr(q), _ptr(scale))
    check("moe_quantize_fp8", st)
    return q, scale


def moe_dequantize_fp8(q: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """e4m3 codes [E, N, K] and scales [E, N] -> fp32 weights [E, K, N]."""
    E, N, K = q.shape
    if q.dtype != torch.uint8 or scale.dtype != torch.float32 or tuple(scale.shape) != (E, N):
        raise ValueError("q must be uint8 [E, N, K] and scale fp32 [E, N]")
    w = torch.empty((E, K, N), dtype=torch.float32, device=q.device)
    st = lib().moe_dequantize_fp8(_stream(q.device), _ptr(q), _ptr(scale), E, K, N, _ptr(w))
    check("moe_dequantize_fp8", st)
    return w


def _check_fp8_weights(E, H, I, w1q, w3q, w2q, s1, s3, s2):
    if tuple(w1q.shape) != (E, I, H) or tuple(w2q.shape) != (E, H, I):
        raise ValueError("w1q must be [E, I, H] and w2q [E, H, I] (codes, K-contiguous)")
    if w3q is not None and tuple(w3q.shape) != (E, I, H):
        raise ValueError("w3q must be [E, I, H]")
    for t in (w1q, w3q, w2q):
        if t is not None and t.dtype != torch.uint8:
            raise ValueError("codes must be uint8")
    for t, n in ((s1, I), (s3, I), (s2, H)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (E, n)):
            raise ValueError("scales must be fp32 [E, N]")


def moe_expert_ffn_fp8(x_disp: torch.Tensor, kept: torch.Tensor, w1q: torch.Tensor,
                       w3q: Optional[torch.Tensor], w2q: torch.Tensor, s1: torch.Tensor,
                       s3: Optional[torch.Tensor], s2: torch.Tensor,
                       b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None, *,
                       act: str = "swiglu", h_ws: Optional[torch.Tensor] = None,
                       y_disp: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """moe_expert_ffn on 8-bit weights (codes and scales from moe_quantize_fp8)."""
    E, C, H = x_disp.shape
    I = w1q.shape[1]
    dev = x_disp.device
    _check_fp8_weights(E, H, I, w1q, w3q, w2q, s1, s3, s2)
    h_ws = _want(h_ws, (E, C, I), x_disp.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    st = lib().moe_expert_ffn_fp8(_stream(dev), ACTS[act], _ptr(x_disp), _ptr(kept), E, C, H, I,
                                  _ptr(w1q), _ptr(w3q), _ptr(w2q), _ptr(s1), _ptr(s3), _ptr(s2),
                                  _ptr(b1), _ptr(b2), _ptr(h_ws), _ptr(y_disp), _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size())
    check("moe_expert_ffn_fp8", st)
    return y_disp, h_ws


def moe_expert_ffn_gather_fp8(x: torch.Tensor, slot_token: torch.Tensor, kept: torch.Tensor,
                              w1q: torch.Tensor, w3q: Optional[torch.Tensor], w2q: torch.Tensor,
                              s1: torch.Tensor, s3: Optional[torch.Tensor], s2: torch.Tensor,
                              b1: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None,
                              *, act: str = "swiglu", h_ws: Optional[torch.Tensor] = None,
                              y_disp: Optional[torch.Tensor] = None,
                              ws: Optional[torch.Tensor] = None):
    """moe_expert_ffn_gather on 8-bit weights."""
    T, H = x.shape
    E, C = slot_token.shape
    I = w1q.shape[1]
    dev = x.device
    _check_fp8_weights(E, H, I, w1q, w3q, w2q, s1, s3, s2)
    h_ws = _want(h_ws, (E, C, I), x.dtype, dev)
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    st = lib().moe_expert_ffn_gather_fp8(_stream(dev), ACTS[act], _ptr(x), _ptr(slot_token), T,
                                         _ptr(kept), E, C, H, I, _ptr(w1q), _ptr(w3q), _ptr(w2q),
                                         _ptr(s1), _ptr(s3), _ptr(s2), _ptr(b1), _ptr(b2),
                                         _ptr(h_ws), _ptr(y_disp), _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size())
    check("moe_expert_ffn_gather_fp8", st)
    return y_disp, h_ws


def moe_combine(y_disp: torch.Tensor, slot: torch.Tensor, topk_w: torch.Tensor, *,
                y: Optional[torch.Tensor] = None, y_shared: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """y_shared: optional fp32 [T, H] (the shared experts' output) added to
    every token's weighted sum."""
    H = y_disp.shape[-1]
    T, k = slot.shape
    dev = slot.device
    if y_disp.dtype != torch.float32:
        raise ValueError("y_disp must be fp32")
    if y_shared is not None and (y_shared.dtype != torch.float32 or y_shared.numel() != T * H
                                 or not y_shared.is_contiguous()):
        raise ValueError("y_shared must be a contiguous fp32 [T, H] tensor")
    y = _want(y, (T, H), out_dtype if y is None else y.dtype, dev)
    st = lib().moe_combine(_stream(dev), _dtype_code(y), _ptr(y_disp), _ptr(slot),
                           _ptr(topk_w), T, H, k, _ptr(y_shared), _ptr(y))
    check("moe_combine", st)
    return y


# ------------------------------------------------------------- backward ----

def moe_combine_bwd(dy: torch.Tensor, y_disp: torch.Tensor, slot: torch.Tensor,
                    topk_w: torch.Tensor, *, dy_disp: Optional[torch.Tensor] = None,
                    dw: Optional[torch.Tensor] = None):
    """dy_disp [E, C, H] (dy's dtype; rows of kept copies written) and dw [T, k]."""
    T, H = dy.shape
    k = slot.shape[1]
    dev = dy.device
    if y_disp.dtype != torch.float32 or y_disp.shape[-1] != H:
        raise ValueError("y_disp must be fp32 [E, C, H]")
    dy_disp = _want(dy_disp, tuple(y_disp.shape), dy.dtype, dev)
    dw = _want(dw, (T, k), torch.float32, dev)
    st = lib().moe_combine_bwd(_stream(dev), _dtype_code(dy), _ptr(dy), _ptr(y_disp), _ptr(slot),
                               _ptr(topk_w), T, H, k, _ptr(dy_disp), _ptr(dw))
    check("moe_combine_bwd", st)
    return dy_disp, dw


def moe_expert_ffn_bwd(x_disp: torch.Tensor, kept: torch.Tensor, w1: torch.Tensor,
                       w3: Optional[torch.Tensor], w2: torch.Tensor, b1: Optional[torch.Tensor],
                       dy_disp: torch.Tensor, *, act: str = "swiglu", has_b2: bool = True,
                       ws: Optional[torch.Tensor] = None, saved: bool = False):
    """Gradients of the expert FFNs: dict with dx_disp [E, C, H] and the
    weight (and GELU bias) gradients, all fp32.  saved: ws holds the first
    product's planes from moe_expert_ffn_fwd_save (no recompute)."""
    if saved and ws is None:
        raise ValueError("saved=True needs the workspace moe_expert_ffn_fwd_save filled")
    E, C, H = x_disp.shape
    I = w1.shape[2]
    dev = x_disp.device
    f32 = torch.float32
    out = {"dx_disp": torch.empty((E, C, H), dtype=f32, device=dev),
           "dw1": torch.empty((E, H, I), dtype=f32, device=dev),
           "dw2": torch.empty((E, I, H), dtype=f32, device=dev),
           "dw3": torch.empty((E, H, I), dtype=f32, device=dev) if act == "swiglu" else None,
           "db1": torch.empty((E, I), dtype=f32, device=dev) if act == "gelu" else None,
           "db2": torch.empty((E, H), dtype=f32, device=dev) if act == "gelu" and has_b2 else None}
    if ws is None:
        ws = torch.zeros(max(16, int(lib().moe_expert_ffn_bwd_ws_bytes(E, C, I))),
                         dtype=torch.uint8, device=dev)
    st = lib().moe_expert_ffn_bwd(_stream(dev), _dtype_code(x_disp), ACTS[act], _ptr(x_disp),
                                  _ptr(kept), E, C, H, I, _ptr(w1), _ptr(w3), _ptr(w2), _ptr(b1),
                                  _ptr(dy_disp), _ptr(out["dx_disp"]), _ptr(out["dw1"]),
                                  _ptr(out["dw3"]), _ptr(out["dw2"]), _ptr(out["db1"]),
                                  _ptr(out["db2"]), _ptr(ws), ws.numel(), 1 if saved else 0)
    check("moe_expert_ffn_bwd", st)
    return out


def moe_expert_ffn_bwd_ws(x_disp: torch.Tensor, I: int) -> torch.Tensor:
    """A workspace for moe_expert_ffn_fwd_save / moe_expert_ffn_bwd."""
    E, C, _ = x_disp.shape
    # zero-filled: the tile counters at its end must start at zero
    return torch.zeros(max(16, int(lib().moe_expert_ffn_bwd_ws_bytes(E, C, I))),
                       dtype=torch.uint8, device=x_disp.device)


def moe_expert_ffn_fwd_save(x_disp: torch.Tensor, kept: torch.Tensor, w1: torch.Tensor,
                            w3: Optional[torch.Tensor], w2: torch.Tensor,
                            b1: Optional[torch.Tensor], b2: Optional[torch.Tensor],
                            ws: torch.Tensor, *, act: str = "swiglu",
                            y_disp: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Training forward of the expert FFNs: y_disp [E, C, H] fp32, with the
    first product's planes kept in ws for moe_expert_ffn_bwd(saved=True)."""
    E, C, H = x_disp.shape
    I = w1.shape[2]
    dev = x_disp.device
    y_disp = _want(y_disp, (E, C, H), torch.float32, dev)
    st = lib().moe_expert_ffn_fwd_save(_stream(dev), _dtype_code(x_disp), ACTS[act],
                                       _ptr(x_disp), _ptr(kept), E, C, H, I, _ptr(w1), _ptr(w3),
                                       _ptr(w2), _ptr(b1), _ptr(b2), _ptr(y_disp), _ptr(ws),
                                       ws.numel())
    check("moe_expert_ffn_fwd_save", st)
    return y_disp


def moe_dispatch_bwd(dx_disp: torch.Tensor, slot: torch.Tensor, *,
                     dx_add: Optional[torch.Tensor] = None,
                     dx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dx [T, H] fp32 = dx_add (optional fp32 [T, H]) + the sum of each
    token's kept copies of dx_disp."""
    H = dx_disp.shape[-1]
    T, k = slot.shape
    dev = slot.device
    if dx_add is not None and (dx_add.dtype != torch.float32 or dx_add.numel() != T * H
                               or not dx_add.is_contiguous()):
        raise ValueError("dx_add must be a contiguous fp32 [T, H] tensor")
    dx = _want(dx, (T, H), torch.float32, dev)
    st = lib().moe_dispatch_bwd(_stream(dev), _ptr(dx_disp), _ptr(slot), T, H, k, _ptr(dx_add),
                                _ptr(dx))
    check("moe_dispatch_bwd", st)
    return dx


def moe_route_bwd(x: torch.Tensor, w_r: torch.Tensor, probs: torch.Tensor,
                  topk_idx: torch.Tensor, topk_w: torch.Tensor, dw: torch.Tensor,
                  f: torch.Tensor, *, alpha: float, dl_aux: float, mode: str = "softmax",
                  seq_len: int = 0, dx: Optional[torch.Tensor] = None, bias: bool = False,
                  ws: Optional[torch.Tensor] = None):
    """dlogits [T, E], dw_r [H, E], db_r [E] (or None); dx, when given, gets
    dlogits W_r^T added in place."""
    T, H = x.shape
    E = w_r.shape[1]
    k = topk_idx.shape[1]
    dev = x.device
    f32 = torch.float32
    dlogits = torch.empty((T, E), dtype=f32, device=dev)
    dw_r = torch.empty((H, E), dtype=f32, device=dev)
    db_r = torch.empty((E,), dtype=f32, device=dev) if bias else None
    if ws is None:
        ws = torch.empty(int(lib().moe_route_bwd_ws_bytes(T, H, E)), dtype=torch.uint8, device=dev)
    st = lib().moe_route_bwd(_stream(dev), _dtype_code(x), ROUTE_MODES[mode], _ptr(x), _ptr(w_r),
                             _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _ptr(dw), _ptr(f),
                             float(alpha), float(dl_aux), T, H, E, k, int(seq_len), _ptr(dlogits),
                             _ptr(dx), _ptr(dw_r), _ptr(db_r), _ptr(ws), ws.numel())
    check("moe_route_bwd", st)
    return dlogits, dw_r, db_r
