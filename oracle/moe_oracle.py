"""CPU oracle for the sparse-MoE FFN layer forward, in float64.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the
HIP path is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP library: it widens its inputs itself and
imports nothing from the package.

Sources (cited by page and section; the pages are the authority):
  [P1] LLaMA4-MoE hand-built guide, dpshk.com/news/5809432
  [P2] MoE basics and minimal PyTorch MoELayer, dpshk.com/news/6005940
  [P3] How to Loop MoE: Flatten the Experts, Untie the Attention,
       discosf.com/news/5228035
  [P4] Long-context MoE training on one A100-80G, 2kiu.com/news/5130654
  [P5] pjlab-sys4nlp/llama-moe architecture essay, coreui.cn/article/2610641

Readings taken where the pages are silent or disagree:
  * f_i = assignments to expert i / (T*k), counted from the router's top-k
    before any capacity drop ([P2] sections 2.3 and 3.1).
  * capacity C = ceil(T*k*cf/E), evaluated in float64 in that order.
  * top-k ties go to the lowest expert index; slot 0 holds the largest key.
  * overflow priority is token-major: assignment (t, j) takes the next free
    row of its expert in row-major (t, then j) order; rows >= C are dropped.
  * a dropped assignment contributes nothing; surviving weights are not
    renormalised; a token with every assignment dropped outputs zeros.
  * SwiGLU expert: (silu(x W_gate) * (x W_up)) W_down, no biases.
    GELU expert: gelu_erf(x W1 + b1) W2 + b2 ([P2] section 3.1).
  * Gumbel mode: key s = l + g with g = -log(-log u) from Philox; selection
    by s (dividing by tau > 0 leaves the order unchanged); the soft path
    q = softmax(s / tau) gives both the combine weights (renormalised over
    the selected experts) and p_i; tau = 1 + 1e-4 * seq_len ([P4] sections
    2 and 5.2).
  * shared expert ([P1] section 5.2 names experts that every token passes
    through, without their form): one always-on FFN of the routed experts'
    form (its own intermediate size), added to every token's output with
    weight 1, outside routing, capacity and L_aux.  Several shared experts
    of one form are the same as one whose intermediate size is their sum.

Parity status: every function here is pinned by a CPU test against what the
pages or the mathematics fix (worked example, closed forms, brute force,
library routines); the readings above are fixed by definition and are
recorded as unpinned readings, not as unpinned functions.
"""
from __future__ import annotations

import dataclasses
import math
import time
from typing import Dict, Optional

import numpy as np
from scipy.special import erf as _erf, expit as _expit

from .philox import gumbel_noise


# ---------------------------------------------------------------- inputs ----

def widen(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Stored input -> float64.  uint16 arrays are bfloat16 bit patterns."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        f32 = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- router ----

def router_logits(x: np.ndarray, w_r: np.ndarray,
                  b_r: Optional[np.ndarray] = None) -> np.ndarray:
    """l = x . W_r (+ b_r).  [P2] section 2.1 (score = x . W_r, no bias);
    [P4] section 5.2 and [P5] section 3.1 use a Linear with a bias."""
    l = x @ w_r
    if b_r is not None:
        l = l + b_r[None, :]
    return l


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax over experts, max-subtracted.  [P2] section 2.1."""
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def topk_lowest_index(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, ordered by (key desc, index asc).

    A stable sort of the negated keys keeps equal keys in ascending index
    order, so ties go to the lowest expert index.  [P2] section 2.1 (top-k)."""
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalise(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']].

    [P5] section 3.1 divides the selected probabilities by their sum; [P2]
    section 3.1 takes a softmax over the selected logits, which is the same
    value in exact arithmetic."""
    sel = np.take_along_axis(p, idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def gumbel_temperature(seq_len: int) -> float:
    """tau = 1 + 1e-4 * seq_len.  [P4] sections 2 and 5.2."""
    return 1.0 + 1e-4 * seq_len


@dataclasses.dataclass
class RouteResult:
    logits: np.ndarray      # [T, E]
    keys: np.ndarray        # [T, E] selection keys (l, or l + g)
    probs: np.ndarray       # [T, E] p (softmax of l) or q (softmax of s/tau)
    idx: np.ndarray         # [T, k] int64, slot 0 = largest key
    w: np.ndarray           # [T, k] renormalised combine weights


def route_softmax(x, w_r, b_r, k: int) -> RouteResult:
    """Softmax router with top-k and renormalised weights.
    [P2] sections 2.1 and 3.1; [P5] section 3.1."""
    l = router_logits(x, w_r, b_r)
    p = softmax_rows(l)
    idx = topk_lowest_index(l, k)
    return RouteResult(l, l, p, idx, renormalise(p, idx))


def route_gumbel(x, w_r, b_r, k: int, seed: int, seq_len: int) -> RouteResult:
    """Gumbel hard top-k router.  [P4] sections 2 and 5.2.

    The hard selection uses s = l + g; the soft path q = softmax(s / tau)
    supplies the combine weights and the mean router probability."""
    l = router_logits(x, w_r, b_r)
    T, E = l.shape
    s = l + gumbel_noise(seed, T, E)
    tau = gumbel_temperature(seq_len)
    q = softmax_rows(s / tau)
    idx = topk_lowest_index(s, k)
    return RouteResult(l, s, q, idx, renormalise(q, idx))


# ----------------------------------------------------------- aux losses ----

@dataclasses.dataclass
class AuxResult:
    counts: np.ndarray      # [E] int64
    f: np.ndarray           # [E]
    P: np.ndarray           # [E]
    l_aux: float


def aux_stats(idx: np.ndarray, probs: np.ndarray, E: int, alpha: float) -> AuxResult:
    """Load-balancing statistics, [P2] section 2.3 and section 3.1; [P1] 3.2.

    f_i: fraction of the T*k router assignments that chose expert i;
    P_i: mean router probability of expert i over the T tokens;
    L_aux = alpha * E * sum_i f_i * P_i."""
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.ravel():
        counts[e] += 1
    f = counts.astype(np.float64) / float(T * k)
    P = probs.sum(axis=0) / float(T)
    l_aux = float(alpha * E * np.sum(f * P))
    return AuxResult(counts, f, P, l_aux)


# ------------------------------------------------------------- dispatch ----

def capacity(T: int, k: int, E: int, cf: float) -> int:
    """C = ceil(T*k*cf/E) in float64.  [P2] section 2.4 gives
    ceil(tokens/experts * cf); with k router assignments per token the
    token count is T*k (the two agree for k = 1)."""
    return int(math.ceil(float(T) * float(k) * float(cf) / float(E)))


@dataclasses.dataclass
class DispatchResult:
    C: int
    slot: np.ndarray        # [T, k] int64: e*C + pos, or -1 if dropped
    slot_token: np.ndarray  # [E, C] int64: token in that row, or -1
    kept: np.ndarray        # [E] int64
    dropped: int


def dispatch(idx: np.ndarray, E: int, C: int) -> DispatchResult:
    """Capacity-bounded grouping of assignments by expert.

    Walk assignments in row-major (t, j) order; each takes the next free row
    of its expert; a row index >= C means the assignment is dropped.
    [P2] section 2.4 (overflow is dropped); [P1] section 2.4 (group tokens by
    expert id, which a stable sort by expert id does in this order)."""
    T, k = idx.shape
    fill = np.zeros(E, dtype=np.int64)
    slot = np.full((T, k), -1, dtype=np.int64)
    slot_token = np.full((E, C), -1, dtype=np.int64)
    dropped = 0
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            pos = int(fill[e])
            fill[e] += 1
            if pos < C:
                slot[t, j] = e * C + pos
                slot_token[e, pos] = t
            else:
                dropped += 1
    kept = np.minimum(fill, C)
    return DispatchResult(C, slot, slot_token, kept, dropped)


# -------------------------------------------------------------- experts ----

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z)."""
    return z * _expit(z)


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """Exact GELU: 0.5 * z * (1 + erf(z / sqrt 2)) (the default nn.GELU the
    minimal MoELayer uses, [P2] section 3.1)."""
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def expert_swiglu(xr, w_gate, w_up, w_down) -> np.ndarray:
    """One SwiGLU expert on rows xr [n, H] -> [n, H]; returns (h, y)."""
    h = silu(xr @ w_gate) * (xr @ w_up)
    return h, h @ w_down


def expert_gelu(xr, w1, b1, w2, b2) -> np.ndarray:
    """One biased two-matrix GELU expert ([P2] section 3.1); returns (h, y)."""
    h = gelu_erf(xr @ w1 + b1[None, :])
    y = h @ w2
    if b2 is not None:
        y = y + b2[None, :]
    return h, y


def expert_forward(inputs: Dict[str, np.ndarray], act: str, e: int,
                   xr: np.ndarray):
    """Run expert e on float64 rows; weights are widened one expert at a
    time so host memory stays bounded."""
    if act == "swiglu":
        return expert_swiglu(xr, widen(inputs["w_gate"][e]),
                             widen(inputs["w_up"][e]), widen(inputs["w_down"][e]))
    if act == "gelu":
        b2 = inputs.get("b2")
        return expert_gelu(xr, widen(inputs["w1"][e]), widen(inputs["b1"][e]),
                           widen(inputs["w2"][e]),
                           None if b2 is None else widen(b2[e]))
    raise ValueError(act)


def shared_expert(inputs: Dict[str, np.ndarray], act: str, xr: np.ndarray):
    """The shared expert on float64 rows ([P1] section 5.2: fixed experts
    that join every token's computation); returns (h, y), or None when the
    layer has none.  Same form as a routed expert."""
    if act == "swiglu":
        if inputs.get("shared_w_gate") is None:
            return None
        return expert_swiglu(xr, widen(inputs["shared_w_gate"][0]),
                             widen(inputs["shared_w_up"][0]), widen(inputs["shared_w_down"][0]))
    if inputs.get("shared_w1") is None:
        return None
    return expert_gelu(xr, widen(inputs["shared_w1"][0]), widen(inputs["shared_b1"][0]),
                       widen(inputs["shared_w2"][0]), widen(inputs["shared_b2"][0]))


# -------------------------------------------------------------- combine ----

def combine(y_disp: np.ndarray, slot: np.ndarray, w: np.ndarray,
            H: int) -> np.ndarray:
    """y[t] = sum over kept j of w[t, j] * Y_disp[slot[t, j]].

    [P1] section 2.4 and [P2] section 3.1 (weighted sum of the selected
    experts' outputs); dropped assignments add nothing."""
    T, k = slot.shape
    y = np.zeros((T, H), dtype=np.float64)
    flat = y_disp.reshape(-1, H)
    for j in range(k):
        s = slot[:, j]
        m = s >= 0
        y[m] += w[m, j][:, None] * flat[s[m]]
    return y


# -------------------------------------------------------------- forward ----

@dataclasses.dataclass
class OracleResult:
    route: RouteResult
    aux: AuxResult
    disp: DispatchResult
    y_disp: Optional[np.ndarray]    # [E, C, H] (rows >= kept are zero)
    h: Optional[np.ndarray]         # [E, C, I] (rows >= kept are zero)
    y: np.ndarray                   # [T, H] or [n_sample, H]
    sample: Optional[np.ndarray]    # token ids of y rows when sampled
    timings: Dict[str, float]
    y_shared: Optional[np.ndarray] = None   # the shared expert's rows of y (None: no shared expert)


def route(inputs: Dict[str, np.ndarray], cfg) -> RouteResult:
    x = widen(inputs["x"])
    w_r = widen(inputs["w_r"])
    b_r = widen(inputs.get("b_r"))
    if cfg.route == "gumbel":
        return route_gumbel(x, w_r, b_r, cfg.k, cfg.seed, cfg.seq_len)
    return route_softmax(x, w_r, b_r, cfg.k)


def forward(inputs: Dict[str, np.ndarray], cfg,
            sample: Optional[np.ndarray] = None,
            keep_h: bool = False) -> OracleResult:
    """The whole layer: route, aux statistics, capacity dispatch, experts,
    combine.  With `sample` (token ids), the experts run only on the kept
    assignments of those tokens and y holds only their rows (routing, aux
    statistics and dispatch are always computed for all tokens)."""
    tm: Dict[str, float] = {}
    t0 = time.perf_counter()
    r = route(inputs, cfg)
    tm["route"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    a = aux_stats(r.idx, r.probs, cfg.E, cfg.alpha)
    tm["aux"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    C = capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
    d = dispatch(r.idx, cfg.E, C)
    tm["dispatch"] = time.perf_counter() - t0
    x = inputs["x"]
    H = cfg.H
    t0 = time.perf_counter()
    if sample is None:
        y_disp = np.zeros((cfg.E, C, H), dtype=np.float64)
        h_all = np.zeros((cfg.E, C, cfg.I), dtype=np.float64) if keep_h else None
        for e in range(cfg.E):
            n = int(d.kept[e])
            if n == 0:
                continue
            rows = widen(x[d.slot_token[e, :n]])
            h, ye = expert_forward(inputs, cfg.act, e, rows)
            y_disp[e, :n] = ye
            if keep_h:
                h_all[e, :n] = h
        tm["experts"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        y = combine(y_disp, d.slot, r.w, H)
        tm["combine"] = time.perf_counter() - t0
        sh = shared_expert(inputs, cfg.act, widen(x))
        if sh is not None:
            y = y + sh[1]
        return OracleResult(r, a, d, y_disp, h_all, y, None, tm,
                            None if sh is None else sh[1])
    sample = np.asarray(sample, dtype=np.int64)
    y = np.zeros((sample.size, H), dtype=np.float64)
    for e in range(cfg.E):
        hit = [(i, j) for i, t in enumerate(sample) for j in range(cfg.k)
               if d.slot[t, j] >= 0 and r.idx[t, j] == e]
        if not hit:
            continue
        rows = widen(x[[sample[i] for i, _ in hit]])
        _, ye = expert_forward(inputs, cfg.act, e, rows)
        for n, (i, j) in enumerate(hit):
            y[i] += r.w[sample[i], j] * ye[n]
    sh = shared_expert(inputs, cfg.act, widen(x[sample]))
    if sh is not None:
        y = y + sh[1]
    tm["experts+combine"] = time.perf_counter() - t0
    return OracleResult(r, a, d, None, None, y, sample, tm, None if sh is None else sh[1])


def near_tie_tokens(keys: np.ndarray, k: int, gap: float = 1e-4) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest keys differ by at most `gap`
    (their selected set is not fixed by float32 arithmetic)."""
    E = keys.shape[1]
    if k >= E:
        return np.zeros(keys.shape[0], dtype=bool)
    srt = -np.sort(-keys, axis=1)
    return (srt[:, k - 1] - srt[:, k]) <= gap
