"""GPU parity of the backward pass: the HIP library (through its C ABI)
against the float64 backward oracle.

The GPU keeps the forward's bf16 storage points in the backward too (dy_disp,
h and its pre-activations, dg / du are bf16: 2^-9 relative each; every sum
is fp32).  Bounds:
  * dx rows: max |err| <= 3e-2 RMS(row);
  * each expert's weight (and bias) gradient, a matrix of sums over the
    expert's rows: RMS(err) <= 1e-2 RMS(block) and max |err| <= 6e-2
    RMS(block) (the maximum over ~10^5 elements sits near 4.5 standard
    deviations of the per-element error);
  * the combine weights' gradient dw, the router logits' gradient and dW_r,
    db_r: element by element, by bounds derived from the arithmetic (see
    _router_bounds): dw = <dy_t, Y[slot]> is computed in fp32 from the
    forward's stored fp32 expert rows Y, so its error is at most the fp32
    summation bound plus sum |dy| |Y_gpu - Y_oracle|; that bound is carried
    through the router backward's linear map (whose derivative is known in
    closed form) to dlogits, and through the fp32 sums over tokens to dW_r
    and db_r;
plus bitwise reproducibility of two backward passes, and the training
forward (forward_train: the first products' planes kept for the backward)
giving bitwise the same expert weight gradients as the recomputing backward.
The routing of the chosen seeds has no near tie, so the GPU and the oracle
differentiate the same top-k choice (asserted).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_backward as B
from oracle import moe_oracle as M
from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
from mixture_experts_layer_08_amd.synth import MoEConfig, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

from parity_util import log, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "swiglu-e8-drops": MoEConfig("b-sw", "bf16", T=600, H=256, I=256, E=8, k=2, cf=1.0, seed=31),
    "gelu-e4-b2": MoEConfig("b-ge", "bf16", T=400, H=256, I=512, E=4, k=2, cf=1.25, act="gelu",
                            seed=32),
    "gumbel-e16": MoEConfig("b-gu", "bf16", T=500, H=512, I=256, E=16, k=2, cf=1.25,
                            route="gumbel", seq=500, seed=33),
    "swiglu-e5-k3-bias": MoEConfig("b-k3", "bf16", T=333, H=256, I=256, E=5, k=3, cf=1.0,
                                   router_bias0=1.0, seed=34),
    "swiglu-e8-shared": MoEConfig("b-sh", "bf16", T=600, H=256, I=256, E=8, k=2, cf=1.0,
                                  shared_I=512, seed=35),
    "gelu-e4-shared": MoEConfig("b-sh-ge", "bf16", T=400, H=256, I=256, E=4, k=2, cf=1.25,
                                act="gelu", shared_I=256, seed=36),
    # about 272 rows per expert: most experts have a thin last row tile (at most
    # 64 rows), which the input-gradient products schedule last and split
    "swiglu-e8-thin": MoEConfig("b-thin", "bf16", T=1090, H=256, I=256, E=8, k=2, cf=1.25,
                                seed=37),
}


def _close(got, want, rel, what, rel_max=None):
    """RMS(err) <= rel * RMS(want) and max |err| <= rel_max * RMS(want)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rel_max = 6 * rel if rel_max is None else rel_max
    rms = float(np.sqrt(np.mean(want * want))) if want.size else 0.0
    d = got - want
    erms = float(np.sqrt(np.mean(d * d))) if want.size else 0.0
    err = float(np.max(np.abs(d))) if want.size else 0.0
    assert erms <= rel * rms + 1e-30, f"{what}: rms err {erms:.3e} vs {rel} * rms {rms:.3e}"
    assert err <= rel_max * rms + 1e-30, f"{what}: max err {err:.3e} vs {rel_max} * rms {rms:.3e}"
    return err / rms if rms else 0.0


def _rows_close(got, want, rel, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = np.sqrt(np.mean(want * want, axis=1))
    err = np.max(np.abs(got - want), axis=1)
    bad = err > rel * rms + 1e-30
    assert not bad.any(), f"{what}: {int(bad.sum())} rows out of tolerance (worst row {int(np.argmax(err / np.maximum(rms, 1e-30)))})"


U32 = 2.0 ** -24   # fp32 unit roundoff


def _gamma(n):
    """Worst-case relative error of an n-term fp32 sum (recursive summation)."""
    return n * U32 / (1.0 - n * U32)


def _router_bounds(cfg, inp, layer, ref, dy64):
    """Per-element error bounds of dw [T, k], dlogits [T, E], dW_r [H, E] and
    db_r [E] (see the module doc).

    dw_tj = <dy_t, Y[s]> in fp32 from the GPU's own fp32 Y[s] (s = slot_tj):
      |err| <= gamma_H sum_h |dy_th Y_gpu[s]_h| + sum_h |dy_th| |Y_gpu - Y_orc|[s]_h.
    dlogits_t is linear in dw_t: with p the (soft-path) probabilities, S the
    sum of the selected ones, w the renormalised weights and tau the
    temperature (1 for softmax), d dl_te / d dw_tj = (p_te / S)
    ([e = e_j] - w_j [e selected]) / tau.  The bound is that map applied to
    |dw err| plus 128 fp32 roundoffs of the magnitudes the router backward
    combines (its own fp32 arithmetic on fp32 probabilities and weights).
    dW_r = x^T dl and db_r = sum_t dl (fp32 sums over T tokens) carry the
    dlogits bound through |x| and add gamma_T of their terms' magnitudes."""
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    fwd = M.forward(inp, cfg)
    slot = fwd.disp.slot
    kept = slot >= 0
    s_idx = np.where(kept, slot, 0)
    y_gpu = to_np(layer.buf.y_disp).reshape(-1, H)
    y_orc = fwd.y_disp.reshape(-1, H)
    b_dw = np.zeros((T, k))
    for j in range(k):
        m = kept[:, j]
        yg = y_gpu[s_idx[m, j]]          # rows of kept copies only (others unwritten)
        yo = y_orc[s_idx[m, j]]
        b_dw[m, j] = _gamma(H) * np.sum(np.abs(dy64[m] * yg), axis=1) + \
            np.sum(np.abs(dy64[m]) * np.abs(yg - yo), axis=1)
    p = fwd.route.probs
    idx = fwd.route.idx
    w = fwd.route.w
    tau = M.gumbel_temperature(cfg.seq_len) if cfg.route == "gumbel" else 1.0
    S = np.take_along_axis(p, idx, axis=1).sum(axis=1)            # [T]
    sel = np.zeros((T, E), dtype=bool)
    np.put_along_axis(sel, idx, True, axis=1)
    b_dl = np.zeros((T, E))
    mag = np.zeros((T, E))
    for j in range(k):
        onehot = np.zeros((T, E))
        np.put_along_axis(onehot, idx[:, j:j + 1], 1.0, axis=1)
        jac = (p / S[:, None]) * np.abs(onehot - w[:, j:j + 1] * sel) / tau
        b_dl += jac * b_dw[:, j:j + 1]
        mag += (p / S[:, None]) * (np.abs(ref.dw_topk[:, j:j + 1]) * (1.0 + w[:, j:j + 1])) / tau
    dp = ref.dprobs
    mag += p * (np.abs(dp) + np.sum(p * np.abs(dp), axis=1, keepdims=True)) / tau
    b_dl += 128 * U32 * mag
    x = M.widen(inp["x"])
    ax = np.abs(x)
    b_dwr = ax.T @ b_dl + _gamma(T) * (ax.T @ np.abs(ref.dlogits))
    b_dbr = b_dl.sum(axis=0) + _gamma(T) * np.abs(ref.dlogits).sum(axis=0)
    return b_dw, b_dl, b_dwr, b_dbr


def _within(got, want, bound, what):
    """|got - want| <= bound, element by element; returns the largest
    err / bound."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = err > bound + 1e-30
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond their bound; first at "
                             f"{tuple(i)} got {got[tuple(i)]} want {want[tuple(i)]} "
                             f"bound {bound[tuple(i)]}")
    return float(np.max(err / np.maximum(bound, 1e-30))) if err.size else 0.0


def _check_router_grads(cfg, inp, layer, ref, dy64, gg, what):
    b_dw, b_dl, b_dwr, b_dbr = _router_bounds(cfg, inp, layer, ref, dy64)
    r1 = _within(to_np(gg["dw_topk"]), ref.dw_topk, b_dw, f"{what}: dw")
    r2 = _within(to_np(gg["dlogits"]), ref.dlogits, b_dl, f"{what}: dlogits")
    r3 = _within(to_np(gg["dw_r"]), ref.dw_r, b_dwr, f"{what}: dW_r")
    r4 = 0.0
    if ref.db_r is not None:
        r4 = _within(to_np(gg["db_r"]), ref.db_r, b_dbr, f"{what}: db_r")
    log(f"[bwd] {what}: largest err/bound dw {r1:.3f} dlogits {r2:.3f} dW_r {r3:.3f} db_r {r4:.3f}")


def _run(cfg, dl_aux=0.5, train=False):
    inp = make_inputs(cfg)
    g = np.random.default_rng(cfg.seed + 7)
    dy_bits = f32_to_bf16_bits(g.standard_normal((cfg.T, cfg.H), dtype=np.float32))
    dy64 = bf16_bits_to_f32(dy_bits).astype(np.float64)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=False)
    x = x_to_device(inp, cfg, DEV)
    if train:
        layer.forward_train(x)
    else:
        layer.forward(x)
    dy = torch.from_numpy(dy_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    grads = layer.backward(x, dy, dl_aux)
    torch.cuda.synchronize()
    return inp, layer, x, dy, dy64, grads


@pytest.mark.parametrize("train", [False, True], ids=["recompute", "saved"])
@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name, train):
    cfg = CASES[name]
    log(f"[bwd] {name} ({'saved' if train else 'recompute'}): T={cfg.T} H={cfg.H} I={cfg.I} "
        f"E={cfg.E} k={cfg.k} {cfg.act} {cfg.route}")
    dl_aux = 0.5
    inp, layer, x, dy, dy64, gg = _run(cfg, dl_aux, train)
    ref = B.backward(inp, cfg, dy64, dl_aux)
    r = M.route(inp, cfg)
    np.testing.assert_array_equal(np.sort(to_np(layer.buf.topk_idx), axis=1),
                                  np.sort(r.idx, axis=1), err_msg="routing differs (near tie)")
    # slot order may differ only where the keys tie; with no ties it is identical
    np.testing.assert_array_equal(to_np(layer.buf.topk_idx), r.idx)
    _check_router_grads(cfg, inp, layer, ref, dy64, gg, name)
    _rows_close(to_np(gg["dx"]), ref.dx, 3e-2, f"{name}: dx")
    worst = 0.0
    for key, want in ref.dweights.items():   # routed experts and the shared one
        got = to_np(gg[key])
        for e in range(want.shape[0]):
            if np.any(want[e] != 0):
                worst = max(worst, _close(got[e], want[e], 1e-2, f"{name}: d{key}[{e}]"))
            else:
                assert np.all(got[e] == 0), f"{name}: d{key}[{e}] should be zero"
    log(f"[bwd] {name}: dropped {ref.dy_disp.size and int(to_np(layer.buf.dropped)[0])}, "
        f"worst weight-grad err/rms {worst:.3e}")


# router-only cases: E a multiple of 8 (the 16-byte W_r row loads), bf16
# and fp32 inputs, token counts that end in a partial chunk
ROUTE_CASES = {
    "route-bf16-e8": MoEConfig("r-e8", "bf16", T=1000, H=512, I=256, E=8, k=2, cf=1.25, seed=37),
    "route-f32-e8": MoEConfig("r-f32", "f32", T=300, H=136, I=64, E=8, k=2, cf=1.25, seed=38),
}


@pytest.mark.parametrize("name", ["swiglu-e5-k3-bias", "gumbel-e16"] + list(ROUTE_CASES))
def test_route_bwd_on_oracle_inputs(name):
    """The router backward fed the oracle's own routing and dw: fp32
    arithmetic against float64, so 1e-4 of the matrix RMS."""
    cfg = CASES.get(name) or ROUTE_CASES[name]
    inp = make_inputs(cfg)
    g = np.random.default_rng(cfg.seed + 7)
    dy64 = bf16_bits_to_f32(f32_to_bf16_bits(g.standard_normal((cfg.T, cfg.H),
                                                             dtype=np.float32))).astype(np.float64)
    ref = B.backward(inp, cfg, dy64, 0.5)
    r = M.route(inp, cfg)
    a = M.aux_stats(r.idx, r.probs, cfg.E, cfg.alpha)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=False)
    x = x_to_device(inp, cfg, DEV)
    f32 = lambda v: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(DEV)  # noqa: E731
    dx = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device=DEV)
    from mixture_experts_layer_08_amd import ops
    dl, dw_r, db_r = ops.moe_route_bwd(
        x, layer.w_r, f32(r.probs), torch.from_numpy(r.idx.astype(np.int32)).to(DEV), f32(r.w),
        f32(ref.dw_topk), f32(a.f), alpha=cfg.alpha, dl_aux=0.5, mode=cfg.route,
        seq_len=cfg.seq_len, dx=dx, bias=layer.b_r is not None)
    torch.cuda.synchronize()
    _close(to_np(dl), ref.dlogits, 1e-5, f"{name}: dlogits", 1e-4)
    _close(to_np(dx), ref.dx_router, 1e-5, f"{name}: dx (router part)", 1e-4)
    _close(to_np(dw_r), ref.dw_r, 1e-5, f"{name}: dW_r", 1e-4)
    if ref.db_r is not None:
        _close(to_np(db_r), ref.db_r, 1e-5, f"{name}: db_r", 1e-4)


def test_backward_deterministic_bitwise():
    cfg = CASES["swiglu-e8-drops"]
    _, layer, x, dy, _, g1 = _run(cfg)
    snap = {k: v.clone() for k, v in g1.items() if v is not None}
    g2 = layer.backward(x, dy, 0.5)
    torch.cuda.synchronize()
    kept = to_np(layer.buf.kept).astype(int)
    for k, v in snap.items():
        if k in ("dy_disp", "dx_disp"):  # rows past kept[e] are not outputs
            for e, n in enumerate(kept):
                assert torch.equal(v[e, :n], g2[k][e, :n]), f"{k}[{e}]"
        else:
            assert torch.equal(v, g2[k]), k


@pytest.mark.parametrize("name", ["swiglu-e8-drops", "gelu-e4-shared"])
def test_saved_planes_equal_recompute(name):
    """forward_train keeps the same first-product planes the backward would
    recompute (the same kernel on the same rows), so every expert weight
    gradient is bitwise the one of the recomputing backward."""
    cfg = CASES[name]
    _, la, x, dy, _, g_re = _run(cfg, 0.5, train=False)
    _, lb, _, _, _, g_sv = _run(cfg, 0.5, train=True)
    np.testing.assert_array_equal(to_np(la.buf.kept), to_np(lb.buf.kept))
    keys = [k for k in g_re if k.startswith(("w_", "w1", "w2", "b1", "b2", "shared_"))
            and g_re[k] is not None]
    assert keys
    for k in keys:
        assert torch.equal(g_re[k], g_sv[k]), k


def test_backward_full_size_config2():
    """The 4096-token layer (H 2048, I 4096, E 8) at full size, every
    gradient against the float64 backward oracle."""
    from mixture_experts_layer_08_amd.synth import CONFIGS
    cfg = CONFIGS[2]
    log("[bwd] config 2 full size (training forward, saved planes)")
    inp, layer, x, dy, dy64, gg = _run(cfg, 0.5, train=True)
    r = M.route(inp, cfg)
    near = M.near_tie_tokens(r.keys, cfg.k)
    same = np.all(to_np(layer.buf.topk_idx) == r.idx, axis=1)
    assert np.all(same | near), "routing differs away from near ties"
    assert same.all(), "a near tie flipped: pick another seed for this check"
    ref = B.backward(inp, cfg, dy64, 0.5)
    log("[bwd] config 2: oracle done")
    _rows_close(to_np(gg["dx"]), ref.dx, 3e-2, "config 2: dx")
    _check_router_grads(cfg, inp, layer, ref, dy64, gg, "config 2")
    worst = 0.0
    for key, want in ref.dweights.items():
        got = to_np(gg[key])
        for e in range(cfg.E):
            worst = max(worst, _close(got[e], want[e], 1e-2, f"config 2: d{key}[{e}]"))
    log(f"[bwd] config 2: worst weight-grad err/rms {worst:.3e}")


@pytest.mark.parametrize("cid", [4, 5])
def test_backward_full_size(cid):
    """Workload 4, the wide GELU layer (T 8192, H 4096, I 16384, E 8, both
    biases: the longest products of the backward, dX with K = I = 16384), and
    workload 5, the 32768-token Gumbel layer (E 32: the router backward
    through the tempered soft path), at full size, every gradient against the
    float64 backward oracle."""
    from mixture_experts_layer_08_amd.synth import CONFIGS
    cfg = CONFIGS[cid]
    log(f"[bwd] config {cid} full size (training forward, saved planes)")
    inp, layer, x, dy, dy64, gg = _run(cfg, 0.5, train=True)
    r = M.route(inp, cfg)
    near = M.near_tie_tokens(r.keys, cfg.k)
    same = np.all(to_np(layer.buf.topk_idx) == r.idx, axis=1)
    assert np.all(same | near), "routing differs away from near ties"
    if not same.all():   # the oracle's backward follows its own routing
        pytest.skip(f"{int((~same).sum())} near-tie token(s) routed differently")
    ref = B.backward(inp, cfg, dy64, 0.5)
    log(f"[bwd] config {cid}: oracle done")
    _rows_close(to_np(gg["dx"]), ref.dx, 3e-2, f"config {cid}: dx")
    _check_router_grads(cfg, inp, layer, ref, dy64, gg, f"config {cid}")
    worst = 0.0
    for key, want in ref.dweights.items():
        got = to_np(gg[key])
        for e in range(cfg.E):
            worst = max(worst, _close(got[e], want[e], 1e-2, f"config {cid}: d{key}[{e}]"))
    log(f"[bwd] config {cid}: worst weight-grad err/rms {worst:.3e}")
