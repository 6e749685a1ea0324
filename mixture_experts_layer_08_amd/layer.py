"""The whole layer forward as library calls on one stream: route,
dispatch with the aux statistics (moe_dispatch_aux), the expert products,
combine.

`MoELayerGPU` owns the device weights and every intermediate buffer of one
layer shape, allocated once, so a forward call enqueues only kernels: no
allocation, no host synchronisation.  With fused_gather (the default) the
dispatch step produces only the row indices and the first expert product
reads each expert's rows straight from x (moe_expert_ffn_gather); without
it, dispatch materialises x_disp and moe_expert_ffn reads that.  With
weights="fp8" the routed experts run on 8-bit e4m3 weights quantised on the
device.  It mirrors the (out, aux_loss) return of the minimal MoELayer of the
MoE basics page (dpshk.com/news/6005940, section 3.1).

A shared expert (the LLaMA4-MoE guide, dpshk.com/news/5809432, section 5.2:
an expert every token passes through) is moe_expert_ffn with one expert
whose C = T rows are x itself, enqueued first on the same stream; the
combine adds its output.  (It does not depend on the routing, but running it
on a second stream measured slower: the persistent product kernels fill
every compute unit's registers, so concurrent kernels only queue behind
them, and two interleaved products lose each other's L2 locality.)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import ops
from .synth import MoEConfig


def _to_dev(a: Optional[np.ndarray], dev, dtype: str) -> Optional[torch.Tensor]:
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev)


@dataclass
class Buffers:
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    probs: torch.Tensor
    keys: torch.Tensor
    counts: torch.Tensor
    f: torch.Tensor
    p: torch.Tensor
    l_aux: torch.Tensor
    x_disp: Optional[torch.Tensor]
    slot: torch.Tensor
    slot_token: torch.Tensor
    kept: torch.Tensor
    dropped: torch.Tensor
    h: torch.Tensor
    y_disp: torch.Tensor
    y: torch.Tensor
    ws: torch.Tensor
    ffn_ws: torch.Tensor
    # shared expert (None without one)
    sh_kept: Optional[torch.Tensor] = None
    sh_h: Optional[torch.Tensor] = None
    sh_y: Optional[torch.Tensor] = None
    sh_ws: Optional[torch.Tensor] = None
    # the fused combine's counters and split workspace (None without it)
    fc_ws: Optional[torch.Tensor] = None


class MoELayerGPU:
    """Device-resident weights + buffers for one configuration."""

    def __init__(self, cfg: MoEConfig, inputs: Dict[str, np.ndarray], device="cuda:0",
                 fused_gather: bool = True, weights: str = "bf16", fused_combine: bool = False):
        """weights="fp8": the routed experts run on 8-bit (e4m3) weights with
        per-expert, per-column scales, quantised here on the device from the
        bf16 weights (moe_quantize_fp8).  fused_combine: forward runs the
        expert products and the combine as one call
        (moe_expert_ffn_gather_combine[_fp8]; fused gather, bf16 activations)."""
        if weights not in ("bf16", "fp8"):
            raise ValueError("weights must be 'bf16' or 'fp8'")
        if fused_combine and (not fused_gather or cfg.dtype != "bf16"):
            raise ValueError("the fused combine needs the fused gather and bf16 activations")
        self.cfg = cfg
        self.fused_gather = fused_gather
        self.fused_combine = fused_combine
        self.weights = weights
        dev = torch.device(device)
        self.dev = dev
        self.tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.w_r = _to_dev(inputs["w_r"], dev, cfg.dtype)
        self.b_r = _to_dev(inputs.get("b_r"), dev, cfg.dtype)
        if cfg.act == "swiglu":
            self.w1 = _to_dev(inputs["w_gate"], dev, cfg.dtype)
            self.w3 = _to_dev(inputs["w_up"], dev, cfg.dtype)
            self.w2 = _to_dev(inputs["w_down"], dev, cfg.dtype)
            self.b1 = self.b2 = None
        else:
            self.w1 = _to_dev(inputs["w1"], dev, cfg.dtype)
            self.w3 = None
            self.w2 = _to_dev(inputs["w2"], dev, cfg.dtype)
            self.b1 = _to_dev(inputs["b1"], dev, cfg.dtype)
            self.b2 = _to_dev(inputs.get("b2"), dev, cfg.dtype)
        self.shared = bool(cfg.shared_I)
        if self.shared:
            if cfg.act == "swiglu":
                self.sw1, self.sw3, self.sw2 = (_to_dev(inputs["shared_" + n], dev, cfg.dtype)
                                                for n in ("w_gate", "w_up", "w_down"))
                self.sb1 = self.sb2 = None
            else:
                self.sw1, self.sb1, self.sw2, self.sb2 = (
                    _to_dev(inputs["shared_" + n], dev, cfg.dtype) for n in ("w1", "b1", "w2", "b2"))
                self.sw3 = None
        self.q = None
        if weights == "fp8":
            if cfg.dtype != "bf16":
                raise ValueError("8-bit weights need bf16 activations")
            self.q = {}
            for name, w in (("w1", self.w1), ("w3", self.w3), ("w2", self.w2)):
                if w is not None:
                    self.q[name + "q"], self.q["s" + name[1]] = ops.moe_quantize_fp8(w)
                else:
                    self.q[name + "q"], self.q["s" + name[1]] = None, None
        self.C = ops.moe_capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
        self.buf = self.alloc(cfg.T)
        # training: backward workspaces holding the first products' planes
        # from forward_train (routed experts, shared expert), and whether
        # they belong to the last forward
        self.bws = None
        self.sh_bws = None
        self._saved = False

    def alloc(self, T: int) -> Buffers:
        cfg, dev, C = self.cfg, self.dev, self.C
        E, k, H, I = cfg.E, cfg.k, cfg.H, cfg.I
        i32, f32, td = torch.int32, torch.float32, self.tdtype
        e = lambda *s, dt=f32: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        # the dispatch workspace and the expert products' workspaces hold
        # counters and flags that start at zero (every call leaves them zero)
        z = lambda n: torch.zeros(n, dtype=torch.uint8, device=dev)  # noqa: E731
        sh = {}
        if self.shared:
            sh = dict(sh_kept=torch.full((1,), T, dtype=i32, device=dev),
                      sh_h=e(1, T, cfg.shared_I, dt=td), sh_y=e(1, T, H),
                      sh_ws=z(ops.moe_expert_ffn_ws_bytes()))
        return Buffers(
            **sh,
            topk_idx=e(T, k, dt=i32), topk_w=e(T, k), probs=e(T, E), keys=e(T, E),
            counts=e(E, dt=i32), f=e(E), p=e(E), l_aux=e(1),
            x_disp=None if self.fused_gather else e(E, C, H, dt=td), slot=e(T, k, dt=i32),
            slot_token=e(E, C, dt=i32),
            kept=e(E, dt=i32), dropped=e(1, dt=i32), h=e(E, C, I, dt=td),
            y_disp=e(E, C, H), y=e(T, H, dt=td),
            ws=z(max(16, ops.moe_workspace_bytes(T, E, k))),
            ffn_ws=z(ops.moe_expert_ffn_ws_bytes()),
            fc_ws=z(ops.moe_expert_ffn_combine_ws_bytes(T, H)) if self.fused_combine else None)

    # the five steps, each one library call ---------------------------------
    def route(self, x: torch.Tensor, keys: bool = False):
        b, cfg = self.buf, self.cfg
        return ops.moe_route(x, self.w_r, self.b_r, cfg.k, mode=cfg.route, seed=cfg.seed,
                             seq_len=cfg.seq_len, topk_idx=b.topk_idx, topk_w=b.topk_w,
                             probs=b.probs, keys=b.keys if keys else None)

    def aux(self):
        b = self.buf
        return ops.moe_aux_stats(b.topk_idx, b.probs, self.cfg.E, self.cfg.alpha, ws=b.ws,
                                 counts=b.counts, f=b.f, p=b.p, l_aux=b.l_aux)

    def dispatch(self, x: torch.Tensor, topk_idx: Optional[torch.Tensor] = None):
        b = self.buf
        return ops.moe_dispatch(x, b.topk_idx if topk_idx is None else topk_idx, self.cfg.E,
                                self.C, ws=b.ws, x_disp=b.x_disp, slot=b.slot,
                                slot_token=b.slot_token, kept=b.kept, dropped=b.dropped,
                                copy=not self.fused_gather)

    def dispatch_aux(self, x: torch.Tensor):
        """dispatch() and aux() in one pass over the routing (the forward's
        path: the statistics come out of the dispatch launches)."""
        b, cfg = self.buf, self.cfg
        return ops.moe_dispatch_aux(x, b.topk_idx, b.probs, cfg.E, self.C, cfg.alpha, ws=b.ws,
                                    x_disp=b.x_disp, slot=b.slot, slot_token=b.slot_token,
                                    kept=b.kept, dropped=b.dropped, counts=b.counts, f=b.f, p=b.p,
                                    l_aux=b.l_aux, copy=not self.fused_gather)

    def experts(self, x: Optional[torch.Tensor] = None):
        """x (the token activations) is needed with fused_gather."""
        b = self.buf
        if self.q is not None:
            q = self.q
            if self.fused_gather:
                if x is None:
                    raise ValueError("experts(x): the fused-gather layer reads the token rows")
                return ops.moe_expert_ffn_gather_fp8(
                    x, b.slot_token, b.kept, q["w1q"], q["w3q"], q["w2q"], q["s1"], q["s3"],
                    q["s2"], self.b1, self.b2, act=self.cfg.act, h_ws=b.h, y_disp=b.y_disp,
                    ws=b.ffn_ws)
            return ops.moe_expert_ffn_fp8(
                b.x_disp, b.kept, q["w1q"], q["w3q"], q["w2q"], q["s1"], q["s3"], q["s2"],
                self.b1, self.b2, act=self.cfg.act, h_ws=b.h, y_disp=b.y_disp, ws=b.ffn_ws)
        if self.fused_gather:
            if x is None:
                raise ValueError("experts(x): the fused-gather layer reads the token rows")
            return ops.moe_expert_ffn_gather(x, b.slot_token, b.kept, self.w1, self.w3, self.w2,
                                             self.b1, self.b2, act=self.cfg.act, h_ws=b.h,
                                             y_disp=b.y_disp, ws=b.ffn_ws)
        return ops.moe_expert_ffn(b.x_disp, b.kept, self.w1, self.w3, self.w2, self.b1, self.b2,
                                  act=self.cfg.act, h_ws=b.h, y_disp=b.y_disp, ws=b.ffn_ws)

    def shared_expert(self, x: torch.Tensor):
        """The shared expert over all T rows of x (one expert, C = T) on the
        current stream; its output is buf.sh_y [1, T, H] fp32."""
        b, T, H = self.buf, self.cfg.T, self.cfg.H
        return ops.moe_expert_ffn(x.view(1, T, H), b.sh_kept, self.sw1, self.sw3, self.sw2,
                                  self.sb1, self.sb2, act=self.cfg.act, h_ws=b.sh_h,
                                  y_disp=b.sh_y, ws=b.sh_ws)

    def experts_combine(self, x: torch.Tensor):
        """experts(x) and combine() as one call: the down product's tiles
        write y (moe_expert_ffn_gather_combine)."""
        b = self.buf
        ysh = b.sh_y.view(self.cfg.T, self.cfg.H) if self.shared else None
        if self.q is not None:
            q = self.q
            return ops.moe_expert_ffn_gather_combine_fp8(
                x, b.slot_token, b.slot, b.topk_w, b.kept, q["w1q"], q["w3q"], q["w2q"], q["s1"],
                q["s3"], q["s2"], self.b1, self.b2, act=self.cfg.act, y_shared=ysh, h_ws=b.h,
                y_disp=b.y_disp, ws=b.fc_ws, y=b.y)
        return ops.moe_expert_ffn_gather_combine(
            x, b.slot_token, b.slot, b.topk_w, b.kept, self.w1, self.w3, self.w2, self.b1,
            self.b2, act=self.cfg.act, y_shared=ysh, h_ws=b.h, y_disp=b.y_disp, ws=b.fc_ws,
            y=b.y)

    def combine(self):
        b = self.buf
        ysh = b.sh_y.view(self.cfg.T, self.cfg.H) if self.shared else None
        return ops.moe_combine(b.y_disp, b.slot, b.topk_w, y=b.y, y_shared=ysh)

    def backward(self, x: torch.Tensor, dy: torch.Tensor, dl_aux: float = 1.0) -> Dict:
        """Gradients of sum(dy * y) + dl_aux * L_aux after forward(x) (the
        forward's buffers are read; the layer must keep x_disp, i.e. be built
        with fused_gather=False, with bf16 weights).  Returns fp32 tensors:
        dx [T, H], dw_r, db_r (or None), and the expert weight gradients under
        the input names (w_gate, w_up, w_down or w1, b1, w2, b2; with a shared
        expert also shared_<name> and its part of dx, dx_shared)."""
        if self.q is not None:
            raise ValueError("backward runs on bf16 expert weights (8-bit weights serve inference)")
        if self.buf.x_disp is None:
            raise ValueError("backward needs the dispatched rows: build the layer with "
                             "fused_gather=False")
        b, cfg = self.buf, self.cfg
        saved = self._saved  # forward_train kept the first products' planes
        dy_disp, dw = ops.moe_combine_bwd(dy, b.y_disp, b.slot, b.topk_w)
        g = ops.moe_expert_ffn_bwd(b.x_disp, b.kept, self.w1, self.w3, self.w2, self.b1, dy_disp,
                                   act=cfg.act, has_b2=self.b2 is not None,
                                   ws=self.bws if saved else None, saved=saved)
        g_sh = None
        if self.shared:  # the shared expert's output gradient is dy itself
            T, H = cfg.T, cfg.H
            g_sh = ops.moe_expert_ffn_bwd(x.view(1, T, H), b.sh_kept, self.sw1, self.sw3, self.sw2,
                                          self.sb1, dy.view(1, T, H), act=cfg.act,
                                          has_b2=self.sb2 is not None,
                                          ws=self.sh_bws if saved else None, saved=saved)
        dx = ops.moe_dispatch_bwd(g["dx_disp"], b.slot,
                                  dx_add=None if g_sh is None else g_sh["dx_disp"].view(cfg.T, cfg.H))
        dlogits, dw_r, db_r = ops.moe_route_bwd(
            x, self.w_r, b.probs, b.topk_idx, b.topk_w, dw, b.f, alpha=cfg.alpha, dl_aux=dl_aux,
            mode=cfg.route, seq_len=cfg.seq_len, dx=dx, bias=self.b_r is not None)
        out = {"dx": dx, "dw_r": dw_r, "db_r": db_r, "dw_topk": dw, "dlogits": dlogits,
               "dy_disp": dy_disp, "dx_disp": g["dx_disp"]}
        names = (("w_gate", "dw1"), ("w_up", "dw3"), ("w_down", "dw2")) if cfg.act == "swiglu" \
            else (("w1", "dw1"), ("b1", "db1"), ("w2", "dw2"), ("b2", "db2"))
        for n, gk in names:
            out[n] = g[gk]
            if g_sh is not None:
                out["shared_" + n] = g_sh[gk]
        if g_sh is not None:
            out["dx_shared"] = g_sh["dx_disp"].view(cfg.T, cfg.H)
        return out

    def forward_train(self, x: torch.Tensor):
        """The forward of a training step: as forward (dispatched-copy path),
        but the expert products keep their first product's planes (h and the
        pre-activations) in the backward workspaces, so the backward that
        follows does not recompute them."""
        b, cfg = self.buf, self.cfg
        if b.x_disp is None:
            raise ValueError("forward_train needs the dispatched rows: build the layer with "
                             "fused_gather=False")
        if self.q is not None:
            raise ValueError("training runs on bf16 expert weights")
        T, H = cfg.T, cfg.H
        if self.bws is None:
            self.bws = ops.moe_expert_ffn_bwd_ws(b.x_disp, cfg.I)
            if self.shared:
                self.sh_bws = ops.moe_expert_ffn_bwd_ws(x.view(1, T, H), cfg.shared_I)
        if self.shared:
            ops.moe_expert_ffn_fwd_save(x.view(1, T, H), b.sh_kept, self.sw1, self.sw3, self.sw2,
                                        self.sb1, self.sb2, self.sh_bws, act=cfg.act,
                                        y_disp=b.sh_y)
        self.route(x)
        self.dispatch_aux(x)
        ops.moe_expert_ffn_fwd_save(b.x_disp, b.kept, self.w1, self.w3, self.w2, self.b1, self.b2,
                                    self.bws, act=cfg.act, y_disp=b.y_disp)
        self.combine()
        self._saved = True
        return b.y, b.l_aux

    def graph(self, x: torch.Tensor) -> "torch.cuda.CUDAGraph":
        """forward(x) captured once into a HIP graph (torch.cuda.CUDAGraph),
        for callers that must capture (a larger captured model, a serving
        loop that replays): replay() reruns every launch of the layer with
        one call.  x is the captured input: copy the next tokens into it,
        replay, read self.buf.y.  The layer's calls only enqueue kernels on
        the current stream (no allocation, no memset, no host
        synchronisation) and every workspace counter is left at zero, so each
        replay equals an eager forward.  (Replay measured slower than eager
        launches on this stack, the decode step included.)"""
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):  # first launches outside the capture
            self.forward(x)
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x)
        torch.cuda.synchronize(self.dev)
        return g

    def forward(self, x: torch.Tensor, keys: bool = False):
        """y [T, H] and L_aux [1]; every intermediate stays in self.buf."""
        self._saved = False
        if self.shared:
            self.shared_expert(x)
        self.route(x, keys=keys)
        self.dispatch_aux(x)
        if self.fused_combine:
            self.experts_combine(x)
        else:
            self.experts(x)
            self.combine()
        return self.buf.y, self.buf.l_aux


def x_to_device(inputs: Dict[str, np.ndarray], cfg: MoEConfig, device="cuda:0") -> torch.Tensor:
    return _to_dev(inputs["x"], torch.device(device), cfg.dtype)
