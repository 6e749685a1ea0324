"""CPU oracle for the backward pass of the sparse-MoE FFN layer, in float64.

TEST INFRASTRUCTURE ONLY, like the forward oracle: only the test suite may
import it; the product path never does, and it shares no code with the HIP
library.

What it differentiates: the scalar  L = sum(dy * y) + dl_aux * L_aux  for a
given output gradient dy [T, H] and aux-loss weight dl_aux, through the same
forward as moe_oracle.forward (its functions are reused, so the two stay one
definition).  The chain rule is taken step by step in the forward's order,
reversed:

  combine   y_t = sum_j w_tj Y[slot_tj]            ([P1] section 2.4)
              -> dY[slot_tj] = w_tj dy_t,  dw_tj = <dy_t, Y[slot_tj]>
  experts   SwiGLU h = silu(X W_gate) * (X W_up), Y = h W_down;
            GELU   h = gelu_erf(X W1 + b1),       Y = h W2 + b2
              -> weight gradients X^T (.), h^T dY; input gradient dX
  dispatch  X rows are copies of x rows -> dx_t += sum of its kept copies' dX
  shared    y_t += S(x_t), the shared expert with weight 1 ([P1] section 5.2)
              -> the expert backward with X = x and dY = dy; dx += its dX
  router    w_j = p_sel_j / sum(p_sel)  ([P5] section 3.1)
              -> dp_sel_j = (dw_j - sum_i dw_i w_i) / sum(p_sel)
            L_aux = alpha E sum_e f_e P_e, P_e = mean_t p_te, f held constant
            (a count of the discrete top-k choices)  ([P2] section 2.3)
              -> dp_te += dl_aux alpha E f_e / T
            p = softmax(l)  (Gumbel mode: q = softmax((l + g) / tau))
              -> dl = p * (dp - sum_e dp_e p_e)  (times 1 / tau for Gumbel)
            l = x W_r + b_r -> dx += dl W_r^T, dW_r = x^T dl, db_r = sum_t dl

The top-k selection and the capacity drop are piecewise constant in the
inputs, so they pass no gradient (the selection's hard forward / soft
backward of [P4] section 2 is exactly this for the Gumbel router).
Pins: central finite differences of moe_oracle.forward (tests), and the
one-expert case against torch autograd of a dense FFN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
from scipy.special import erf as _erf, expit as _expit

from . import moe_oracle as M


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = _expit(z)
    return s * (1.0 + z * (1.0 - s))


def gelu_erf_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [0.5 z (1 + erf(z / sqrt 2))] = Phi(z) + z * phi(z)."""
    cdf = 0.5 * (1.0 + _erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Gradient through p = softmax(z) along rows: p * (dp - <dp, p>)."""
    return p * (dp - np.sum(dp * p, axis=1, keepdims=True))


@dataclasses.dataclass
class Grads:
    dx: np.ndarray                  # [T, H]
    dw_r: np.ndarray                # [H, E]
    db_r: Optional[np.ndarray]      # [E] when the router has a bias
    dweights: Dict[str, np.ndarray]  # same keys and shapes as the inputs
    # intermediates, for stage-wise checks
    dw_topk: np.ndarray             # [T, k] gradient of the combine weights
    dprobs: np.ndarray              # [T, E]
    dlogits: np.ndarray             # [T, E]
    dy_disp: np.ndarray             # [E, C, H] (rows >= kept are zero)
    dx_disp: np.ndarray             # [E, C, H]
    dx_experts: np.ndarray          # [T, H] the experts' part of dx
    dx_router: np.ndarray           # [T, H] the router's part of dx
    dx_shared: Optional[np.ndarray] = None  # [T, H] the shared expert's part of dx


def backward(inputs: Dict[str, np.ndarray], cfg, dy: np.ndarray,
             dl_aux: float = 1.0) -> Grads:
    """All gradients of sum(dy * y) + dl_aux * L_aux (see the module doc)."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dy = np.asarray(dy, dtype=np.float64)
    x = M.widen(inputs["x"])
    r = M.route(inputs, cfg)
    a = M.aux_stats(r.idx, r.probs, E, cfg.alpha)
    C = M.capacity(T, k, E, cfg.cf)
    d = M.dispatch(r.idx, E, C)

    # forward of every expert again, keeping what its backward needs
    y_disp = np.zeros((E, C, H))
    dy_disp = np.zeros((E, C, H))
    dx_disp = np.zeros((E, C, H))
    dweights: Dict[str, np.ndarray] = {}
    if cfg.act == "swiglu":
        for name, shape in (("w_gate", (E, H, I)), ("w_up", (E, H, I)), ("w_down", (E, I, H))):
            dweights[name] = np.zeros(shape)
    else:
        dweights["w1"] = np.zeros((E, H, I))
        dweights["b1"] = np.zeros((E, I))
        dweights["w2"] = np.zeros((E, I, H))
        if inputs.get("b2") is not None:
            dweights["b2"] = np.zeros((E, H))
    cache = {}
    for e in range(E):
        n = int(d.kept[e])
        if n == 0:
            continue
        X = x[d.slot_token[e, :n]]
        if cfg.act == "swiglu":
            w1, w3, w2 = (M.widen(inputs[kk][e]) for kk in ("w_gate", "w_up", "w_down"))
            g, u = X @ w1, X @ w3
            h = M.silu(g) * u
            y_disp[e, :n] = h @ w2
            cache[e] = (X, g, u, h, w1, w3, w2)
        else:
            w1, b1, w2 = M.widen(inputs["w1"][e]), M.widen(inputs["b1"][e]), M.widen(inputs["w2"][e])
            z = X @ w1 + b1[None, :]
            h = M.gelu_erf(z)
            ye = h @ w2
            if inputs.get("b2") is not None:
                ye = ye + M.widen(inputs["b2"][e])[None, :]
            y_disp[e, :n] = ye
            cache[e] = (X, z, h, w1, w2)

    # combine backward
    dw_topk = np.zeros((T, k))
    flat_y = y_disp.reshape(-1, H)
    flat_dy = dy_disp.reshape(-1, H)
    for j in range(k):
        s = d.slot[:, j]
        m = s >= 0
        flat_dy[s[m]] = r.w[m, j][:, None] * dy[m]
        dw_topk[m, j] = np.sum(dy[m] * flat_y[s[m]], axis=1)

    # expert backward, then the gather-add of each token's copies
    dx_experts = np.zeros((T, H))
    for e, c in cache.items():
        n = int(d.kept[e])
        dY = dy_disp[e, :n]
        if cfg.act == "swiglu":
            X, g, u, h, w1, w3, w2 = c
            dweights["w_down"][e] = h.T @ dY
            dh = dY @ w2.T
            dg = dh * u * silu_grad(g)
            du = dh * M.silu(g)
            dweights["w_gate"][e] = X.T @ dg
            dweights["w_up"][e] = X.T @ du
            dX = dg @ w1.T + du @ w3.T
        else:
            X, z, h, w1, w2 = c
            dweights["w2"][e] = h.T @ dY
            if "b2" in dweights:
                dweights["b2"][e] = dY.sum(axis=0)
            dz = (dY @ w2.T) * gelu_erf_grad(z)
            dweights["w1"][e] = X.T @ dz
            dweights["b1"][e] = dz.sum(axis=0)
            dX = dz @ w1.T
        dx_disp[e, :n] = dX
        np.add.at(dx_experts, d.slot_token[e, :n], dX)

    # router backward: renormalisation, aux statistics, softmax, linear
    sel = np.take_along_axis(r.probs, r.idx, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    dsel = (dw_topk - np.sum(dw_topk * r.w, axis=1, keepdims=True)) / S
    dprobs = np.zeros((T, E))
    np.put_along_axis(dprobs, r.idx, dsel, axis=1)
    dprobs += dl_aux * cfg.alpha * E * a.f[None, :] / T
    dz_soft = softmax_backward(r.probs, dprobs)
    if cfg.route == "gumbel":
        dlogits = dz_soft / M.gumbel_temperature(cfg.seq_len)
    else:
        dlogits = dz_soft
    w_r = M.widen(inputs["w_r"])
    dx_router = dlogits @ w_r.T
    dw_r = x.T @ dlogits
    db_r = dlogits.sum(axis=0) if inputs.get("b_r") is not None else None

    # shared expert: every token with weight 1, so its output gradient is dy
    dx_shared = None
    if cfg.act == "swiglu" and inputs.get("shared_w_gate") is not None:
        w1, w3, w2 = (M.widen(inputs["shared_" + kk][0]) for kk in ("w_gate", "w_up", "w_down"))
        g, u = x @ w1, x @ w3
        h = M.silu(g) * u
        dh = dy @ w2.T
        dg = dh * u * silu_grad(g)
        du = dh * M.silu(g)
        dweights["shared_w_down"] = (h.T @ dy)[None]
        dweights["shared_w_gate"] = (x.T @ dg)[None]
        dweights["shared_w_up"] = (x.T @ du)[None]
        dx_shared = dg @ w1.T + du @ w3.T
    elif cfg.act == "gelu" and inputs.get("shared_w1") is not None:
        w1, b1, w2 = (M.widen(inputs["shared_" + kk][0]) for kk in ("w1", "b1", "w2"))
        z = x @ w1 + b1[None, :]
        h = M.gelu_erf(z)
        dweights["shared_w2"] = (h.T @ dy)[None]
        dweights["shared_b2"] = dy.sum(axis=0)[None]
        dz = (dy @ w2.T) * gelu_erf_grad(z)
        dweights["shared_w1"] = (x.T @ dz)[None]
        dweights["shared_b1"] = dz.sum(axis=0)[None]
        dx_shared = dz @ w1.T
    dx = dx_experts + dx_router
    if dx_shared is not None:
        dx = dx + dx_shared
    return Grads(dx, dw_r, db_r, dweights, dw_topk, dprobs, dlogits,
                 dy_disp, dx_disp, dx_experts, dx_router, dx_shared)


def objective(inputs: Dict[str, np.ndarray], cfg, dy: np.ndarray, dl_aux: float) -> float:
    """sum(dy * y) + dl_aux * L_aux from the forward oracle (what backward
    differentiates; used by the finite-difference pins)."""
    res = M.forward(inputs, cfg)
    return float(np.sum(dy * res.y) + dl_aux * res.aux.l_aux)
