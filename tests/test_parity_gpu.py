"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Tolerances (fixed by the layer's specification):
  * expert indices, per-expert counts, slots, slot_token, kept and dropped are
    bit-exact; a top-k set may differ only at a token whose k-th and
    (k+1)-th oracle keys are within 1e-4 (counted and reported);
  * combine weights, probabilities and L_aux agree within 1e-5 relative;
  * layer outputs: max |err| <= 2e-2 * RMS(row) for bf16, <= 1e-4 for fp32.
    A bf16 layer stores y in bf16, rounded once after the fp32 sum; that
    rounding moves an element by up to 2^-8 of its stored value (1.6% of
    the row RMS for an element at 4 RMS, just above a power of two), so it
    is allowed on top of the bound: |y - y_oracle| <= 2e-2 RMS(row) +
    2^-8 |y|.  The fp32 expert outputs y_disp get the plain bound.
Each stage is also run on the oracle's own upstream outputs, so a near-tie
cannot hide a downstream difference.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_oracle as M
from oracle import near_tie_tokens
from mixture_experts_layer_08_amd import ops
from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
from mixture_experts_layer_08_amd.synth import (CONFIGS, MoEConfig, bf16_bits_to_f32, drop_free,
                                                f32_to_bf16_bits, make_inputs)

from parity_util import assert_rel, assert_rows_close, log, to_dev, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SMALL = {
    "bf16-swiglu-e8": MoEConfig("s-e8", "bf16", T=3001, H=512, I=384, E=8, k=2, cf=1.25,
                                seed=11),
    "bf16-swiglu-e5-k3-drops": MoEConfig("s-e5", "bf16", T=777, H=256, I=256, E=5, k=3,
                                         cf=0.8, router_bias0=1.0, seed=12),
    "bf16-gelu-e4": MoEConfig("s-gelu", "bf16", T=600, H=256, I=512, E=4, k=2, cf=1.25,
                              act="gelu", seed=13),
    "bf16-gumbel-e32": MoEConfig("s-gumbel", "bf16", T=900, H=512, I=256, E=32, k=2, cf=1.25,
                                 route="gumbel", seq=900, seed=14),
    "bf16-e64-k8": MoEConfig("s-e64", "bf16", T=300, H=256, I=128, E=64, k=8, cf=1.0, seed=15),
    "bf16-e1-dense": MoEConfig("s-e1", "bf16", T=257, H=256, I=128, E=1, k=1, cf=1.0, seed=17),
    "f32-config1": CONFIGS[1],
    "f32-gelu-e3": MoEConfig("s-f32-gelu", "f32", T=130, H=64, I=96, E=3, k=2, cf=1.0,
                             act="gelu", seed=16),
    # with a shared expert (every token, weight 1), drops on the routed side
    "bf16-swiglu-e8-shared": MoEConfig("s-sh", "bf16", T=1001, H=256, I=256, E=8, k=2, cf=1.0,
                                       shared_I=512, seed=18),
    "bf16-gelu-e4-shared": MoEConfig("s-sh-gelu", "bf16", T=600, H=256, I=512, E=4, k=2,
                                     cf=1.25, act="gelu", shared_I=256, seed=19),
}


def _tol(cfg):
    return (2e-2, 0.0) if cfg.dtype == "bf16" else (0.0, 1e-4)


def _check_y(cfg, got, want, what, layer_out=False):
    """layer_out: `got` is the layer output y, which a bf16 layer stores in
    bf16 (its final rounding is allowed on top of the bound; see
    assert_rows_close).  Expert outputs y_disp are stored in fp32."""
    rel, ab = _tol(cfg)
    if cfg.dtype == "bf16":
        return assert_rows_close(got, want, rel, what, stored_bf16=layer_out)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= ab, f"{what}: max abs err {err}"
    return err


def _check_h(cfg, got, want, what):
    """The hidden activation is an intermediate stored in the storage type:
    bf16 rounding (nearest-even) is at most 2^-9 of the value, and the fp32
    accumulation and activation add ~1e-6 relative; the bound allows twice
    the rounding plus 2e-3 of the row RMS.  fp32 storage: 1e-4 absolute."""
    if cfg.dtype == "bf16":
        rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
        bad = np.abs(got - want) > 2.0 ** -8 * np.abs(want) + 2e-3 * rms
        assert not bad.any(), f"{what}: {int(bad.sum())} elements out of tolerance"
    else:
        assert float(np.max(np.abs(got - want))) <= 1e-4, what


def _route_compare(cfg, gpu_idx, gpu_w, gpu_probs, gpu_keys, r, what):
    """Integer routing bit-exact outside the near-tie set; floats to 1e-5."""
    k = cfg.k
    near = near_tie_tokens(r.keys, k)
    same = np.all(np.sort(gpu_idx, axis=1) == np.sort(r.idx, axis=1), axis=1)
    flips = np.where(~same)[0]
    log(f"[{what}] near-tie tokens {int(near.sum())}, top-k set differences {flips.size}")
    assert np.all(near[flips]), f"{what}: top-k set differs at non-near-tie tokens {flips[~near[flips]][:10]}"
    # slot order where adjacent selected keys are separated by more than 1e-4
    sk = np.take_along_axis(r.keys, r.idx, axis=1)
    for j in range(k - 1):
        sep = (sk[:, j] - sk[:, j + 1]) > 1e-4
        ok = same & sep
        assert np.all(gpu_idx[ok, j] == r.idx[ok, j]), f"{what}: slot order differs"
    # weights, matched by expert id, on tokens with the same set
    gw = np.zeros_like(r.w)
    for j in range(k):
        m = gpu_idx[:, j:j + 1] == r.idx           # [T, k]
        gw += np.where(m, gpu_w[:, j:j + 1], 0.0)
    assert_rel(gw[same], r.w[same], 1e-5, f"{what}: combine weights")
    assert_rel(gpu_probs, r.probs, 1e-5, f"{what}: probabilities", atol=1e-12)
    if gpu_keys is not None:
        assert_rel(gpu_keys, r.keys, 0.0, f"{what}: selection keys",
                   atol=1e-5 * max(1.0, float(np.max(np.abs(r.keys)))))
    return same


def _dispatch_compare(gpu, d, what):
    slot, slot_token, kept, dropped = gpu
    np.testing.assert_array_equal(slot, d.slot, err_msg=f"{what}: slot")
    np.testing.assert_array_equal(slot_token, d.slot_token, err_msg=f"{what}: slot_token")
    np.testing.assert_array_equal(kept, d.kept, err_msg=f"{what}: kept")
    assert int(dropped[0]) == d.dropped, f"{what}: dropped {int(dropped[0])} vs {d.dropped}"


# ------------------------------------------------------------ end to end ----
@pytest.mark.parametrize("fused", [True, False], ids=["gather", "copy"])
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_end_to_end_small(name, fused):
    cfg = SMALL[name]
    log(f"[e2e] {name} ({'gather' if fused else 'copy'}): T={cfg.T} H={cfg.H} I={cfg.I} "
        f"E={cfg.E} k={cfg.k} cf={cfg.cf} {cfg.dtype} {cfg.act} {cfg.route}")
    inp = make_inputs(cfg)
    ref = M.forward(inp, cfg, keep_h=True)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=fused)
    x = x_to_device(inp, cfg, DEV)
    y, l_aux = layer.forward(x, keys=True)
    torch.cuda.synchronize()
    b = layer.buf
    same = _route_compare(cfg, to_np(b.topk_idx), to_np(b.topk_w), to_np(b.probs),
                          to_np(b.keys), ref.route, name)
    gidx = to_np(b.topk_idx).astype(np.int64)
    # dispatch of the GPU's own routing is exactly the oracle's walk over it
    d_gpu = M.dispatch(gidx, cfg.E, layer.C)
    _dispatch_compare((to_np(b.slot), to_np(b.slot_token), to_np(b.kept), to_np(b.dropped)),
                      d_gpu, name)
    assert_rel(to_np(l_aux), [ref.aux.l_aux], 1e-5, f"{name}: L_aux")
    if same.all():
        np.testing.assert_array_equal(to_np(b.counts), ref.aux.counts)
        assert_rel(to_np(b.f), ref.aux.f, 1e-5, f"{name}: f", atol=1e-12)
    assert_rel(to_np(b.p), ref.aux.P, 1e-5, f"{name}: p", atol=1e-12)
    ok = same.copy()
    ok &= np.all(to_np(b.slot) == ref.disp.slot, axis=1)
    worst = _check_y(cfg, to_np(y)[ok], ref.y[ok], f"{name}: y", layer_out=True)
    log(f"[e2e] {name}: dropped {int(to_np(b.dropped)[0])}, compared {int(ok.sum())}/{cfg.T} "
        f"rows, worst err/rms {worst:.3e}")
    # tokens with every copy dropped are exactly zero (without a shared expert)
    all_drop = np.all(ref.disp.slot < 0, axis=1) & ok
    if not cfg.shared_I:
        assert np.all(to_np(y)[all_drop] == 0.0)


# ------------------------------------------------------------- router ----
ROUTE_ONLY = {
    # hidden sizes past the old 4096 limit, an odd number of 256-wide chunks,
    # expert counts that are not a multiple of 8 (scalar W_r loads) and the
    # largest (64, four 16-expert column blocks); token counts that end in a
    # partial tile and in a partial set of tiles
    "h8192-gumbel-e32": MoEConfig("r8k", "bf16", T=1000, H=8192, I=128, E=32, k=2, cf=1.25,
                                  route="gumbel", seq=1000, seed=61),
    "h4352-e5-k3-bias": MoEConfig("r4k", "bf16", T=777, H=4352, I=128, E=5, k=3, cf=1.0,
                                  router_bias0=1.0, seed=62),
    "h1280-e64-k8": MoEConfig("r64", "bf16", T=333, H=1280, I=128, E=64, k=8, cf=1.0, seed=63),
    "h256-e1": MoEConfig("r1", "bf16", T=17, H=256, I=128, E=1, k=1, cf=1.0, seed=64),
    "h768-e12-k2": MoEConfig("r12", "bf16", T=4099, H=768, I=128, E=12, k=2, cf=1.0, seed=65),
    # at least 8 tiles of 16 tokens per compute unit (on 256 compute units):
    # the kernels that give each wave whole tiles, x and W_r staged through
    # LDS (16 and 24 experts; a second, partial round of tiles ending in a
    # partial tile; H = 4096 with a router bias; H = 768, whose half-row
    # start is an odd chunk pair; H = 256, two chunks for eight noise values
    # per lane), and W_r alone in LDS (40 experts, past the staged kernel's
    # LDS; 12 experts, not a multiple of 8)
    "t40007-e16-gumbel": MoEConfig("s16", "bf16", T=40007, H=2048, I=128, E=16, k=2, cf=1.0,
                                   route="gumbel", seq=40007, seed=66),
    "t33000-h4096-e32-bias": MoEConfig("s32", "bf16", T=33000, H=4096, I=128, E=32, k=2, cf=1.0,
                                       router_bias0=1.5, seed=67),
    "t32768-e24-k3": MoEConfig("s24", "bf16", T=32768, H=2048, I=128, E=24, k=3, cf=1.0, seed=68),
    "t32768-h768-e8-gumbel": MoEConfig("s8", "bf16", T=32768, H=768, I=128, E=8, k=2, cf=1.0,
                                       route="gumbel", seq=32768, seed=71),
    "t32768-h256-e32-gumbel": MoEConfig("s32n", "bf16", T=32768, H=256, I=128, E=32, k=4,
                                        cf=1.0, route="gumbel", seq=32768, seed=72),
    "t32800-e40-gumbel": MoEConfig("s40", "bf16", T=32800, H=1024, I=128, E=40, k=2, cf=1.0,
                                   route="gumbel", seq=32800, seed=69),
    "t32790-e12": MoEConfig("s12", "bf16", T=32790, H=1024, I=128, E=12, k=2, cf=1.0, seed=70),
}


@pytest.mark.parametrize("name", list(ROUTE_ONLY))
def test_route_shapes(name):
    """The router alone against the oracle's on shapes the layer tests do not
    reach: probabilities and weights to 1e-5, top-k sets bit-exact outside
    near ties, keys (logits or Gumbel keys) to 1e-5 of their largest size."""
    cfg = ROUTE_ONLY[name]
    log(f"[route] {name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} {cfg.route}")
    rng = np.random.default_rng(cfg.seed)
    x = f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))
    w_r = f32_to_bf16_bits(rng.standard_normal((cfg.H, cfg.E), dtype=np.float32) * np.float32(0.02))
    b_r = None
    if cfg.router_bias0:
        b_r = np.zeros(cfg.E, dtype=np.float32)
        b_r[0] = cfg.router_bias0
    inp = {"x": x, "w_r": w_r, "b_r": b_r}
    r = M.route(inp, cfg)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    wd = torch.from_numpy(w_r.view(np.int16)).view(torch.bfloat16).to(DEV)
    bd = None if b_r is None else torch.from_numpy(b_r).to(DEV)
    idx, w, probs, keys = ops.moe_route(xd, wd, bd, cfg.k, mode=cfg.route, seed=cfg.seed,
                                        seq_len=cfg.seq_len, want_keys=True)
    torch.cuda.synchronize()
    _route_compare(cfg, to_np(idx), to_np(w), to_np(probs), to_np(keys), r, name)


# ------------------------------------------------------------ stage-wise ----
@pytest.mark.parametrize("name", list(SMALL))
def test_stages_on_oracle_inputs(name):
    cfg = SMALL[name]
    log(f"[stages] {name}")
    inp = make_inputs(cfg)
    ref = M.forward(inp, cfg, keep_h=True)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=False)
    x = x_to_device(inp, cfg, DEV)
    idx = to_dev(ref.route.idx.astype(np.int32), torch.int32)
    probs = to_dev(ref.route.probs.astype(np.float32), torch.float32)
    # aux statistics on the oracle's routing
    counts, f, p, l_aux = ops.moe_aux_stats(idx, probs, cfg.E, cfg.alpha)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(counts), ref.aux.counts)
    assert_rel(to_np(f), ref.aux.f, 1e-6, f"{name}: f", atol=1e-12)
    assert_rel(to_np(p), ref.aux.P, 1e-5, f"{name}: p", atol=1e-12)
    assert_rel(to_np(l_aux), [ref.aux.l_aux], 1e-5, f"{name}: L_aux")
    # dispatch on the oracle's routing: every integer output and the copied rows exact
    x_disp, slot, slot_token, kept, dropped = layer.dispatch(x, idx)
    torch.cuda.synchronize()
    _dispatch_compare((to_np(slot), to_np(slot_token), to_np(kept), to_np(dropped)), ref.disp,
                      name)
    xd = _rows_np(x_disp, ref.disp.kept)
    xs = to_np(x)
    for e in range(cfg.E):
        n = int(ref.disp.kept[e])
        np.testing.assert_array_equal(xd[e], xs[ref.disp.slot_token[e, :n]])
    # expert FFN on the oracle's dispatched rows
    y_disp, h = layer.experts()
    torch.cuda.synchronize()
    yd, hh = _rows_np(y_disp, ref.disp.kept), _rows_np(h, ref.disp.kept)
    for e in range(cfg.E):
        n = int(ref.disp.kept[e])
        if n:
            _check_h(cfg, hh[e], ref.h[e, :n], f"{name}: h[{e}]")
            _check_y(cfg, yd[e], ref.y_disp[e, :n], f"{name}: y_disp[{e}]")
    # the same product reading the rows straight from x through slot_token:
    # identical inputs, tiles and summation order, so bitwise equal outputs
    yg, hg = ops.moe_expert_ffn_gather(
        x, to_dev(ref.disp.slot_token.astype(np.int32), torch.int32), kept, layer.w1, layer.w3,
        layer.w2, layer.b1, layer.b2, act=cfg.act, ws=layer.buf.ffn_ws)
    torch.cuda.synchronize()
    ygn, hgn = _rows_np(yg, ref.disp.kept), _rows_np(hg, ref.disp.kept)
    for e in range(cfg.E):
        np.testing.assert_array_equal(ygn[e], yd[e], err_msg=f"{name}: gathered y_disp[{e}]")
        np.testing.assert_array_equal(hgn[e], hh[e], err_msg=f"{name}: gathered h[{e}]")
    if cfg.dtype == "bf16":
        # without a workspace every tile runs whole (with one, a partly filled
        # last round is cut into K pieces and the last piece of each tile to
        # arrive sums them, which is all these small shapes have)
        yw, hw = ops.moe_expert_ffn(x_disp, kept, layer.w1, layer.w3, layer.w2, layer.b1,
                                    layer.b2, act=cfg.act)
        torch.cuda.synchronize()
        ywn, hwn = _rows_np(yw, ref.disp.kept), _rows_np(hw, ref.disp.kept)
        for e in range(cfg.E):
            n = int(ref.disp.kept[e])
            if n:
                _check_h(cfg, hwn[e], ref.h[e, :n], f"{name}: h[{e}], no workspace")
                _check_y(cfg, ywn[e], ref.y_disp[e, :n], f"{name}: y_disp[{e}], no workspace")
    # combine of the oracle's expert outputs (stored in fp32, as the library keeps them)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ydisp_store = ref.y_disp.astype(np.float32).astype(np.float64)
    w32 = ref.route.w.astype(np.float32).astype(np.float64)
    y = ops.moe_combine(to_dev(ydisp_store, torch.float32),
                        to_dev(ref.disp.slot.astype(np.int32), torch.int32),
                        to_dev(w32.astype(np.float32), torch.float32), out_dtype=tdt)
    torch.cuda.synchronize()
    want = M.combine(ydisp_store, ref.disp.slot, w32, cfg.H)
    got = to_np(y)
    if cfg.dtype == "bf16":
        assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-30 +
                      1e-6 * np.sqrt(np.mean(want * want, axis=1, keepdims=True)))
    else:
        assert np.max(np.abs(got - want)) <= 1e-5
    if cfg.shared_I:
        # the shared expert over every token (one expert, C = T, rows = x)
        layer.shared_expert(x)
        torch.cuda.synchronize()
        _check_y(cfg, to_np(layer.buf.sh_y)[0], ref.y_shared, f"{name}: shared expert")
        # combine adding the (fp32-stored) shared rows
        ysh = ref.y_shared.astype(np.float32)
        y2 = ops.moe_combine(to_dev(ydisp_store, torch.float32),
                             to_dev(ref.disp.slot.astype(np.int32), torch.int32),
                             to_dev(w32.astype(np.float32), torch.float32),
                             y_shared=to_dev(ysh, torch.float32), out_dtype=tdt)
        torch.cuda.synchronize()
        want2 = want + ysh.astype(np.float64)
        got2 = to_np(y2)
        assert np.all(np.abs(got2 - want2) <= 2.0 ** -8 * np.abs(want2) + 1e-30 +
                      1e-6 * np.sqrt(np.mean(want2 * want2, axis=1, keepdims=True)))


# Expert row counts whose last row tile is thin (at most 64 of 256 rows):
# the products schedule those tiles after all others.  Last row tiles of 8,
# 64 (the bound), 1 and 44 rows, an expert with only a thin tile, one with no
# rows, and last tiles of 65 and 128 rows that stay in place; then a shape
# whose other tiles fill exactly one round of 256 workgroups, so that with a
# workspace the 96 thin tiles are the round cut along K.
THIN_LAST = {
    "mixed-swiglu": (MoEConfig("t-mix", "bf16", T=64, H=512, I=512, E=8, k=2, cf=1.0, seed=51),
                     640, [520, 64, 1, 0, 300, 576, 577, 640]),
    "mixed-gelu": (MoEConfig("t-mix-ge", "bf16", T=64, H=512, I=512, E=8, k=2, cf=1.0,
                             act="gelu", seed=52),
                   640, [520, 64, 1, 0, 300, 576, 577, 640]),
    "one-round-swiglu": (MoEConfig("t-round", "bf16", T=64, H=256, I=4096, E=8, k=2, cf=1.0,
                                   seed=53),
                         320, [273, 256, 256, 257, 256, 256, 289, 256]),
}


@pytest.mark.parametrize("ws_on", [True, False], ids=["split", "whole"])
@pytest.mark.parametrize("name", list(THIN_LAST))
def test_thin_last_row_tiles(name, ws_on):
    cfg, C, kept_l = THIN_LAST[name]
    log(f"[thin-last] {name} ({'split' if ws_on else 'whole'}): kept {kept_l}")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(cfg.seed + 1)
    xd_bits = f32_to_bf16_bits(rng.standard_normal((cfg.E, C, cfg.H), dtype=np.float32))
    xd = bf16_bits_to_f32(xd_bits).astype(np.float64)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=False)
    x_disp = torch.from_numpy(xd_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kept = to_dev(np.array(kept_l, dtype=np.int32), torch.int32)
    ws = (torch.zeros(ops.moe_expert_ffn_ws_bytes(), dtype=torch.uint8, device=DEV)
          if ws_on else None)
    y, h = ops.moe_expert_ffn(x_disp, kept, layer.w1, layer.w3, layer.w2, layer.b1, layer.b2,
                              act=cfg.act, ws=ws)
    torch.cuda.synchronize()
    yn, hn = _rows_np(y, kept_l), _rows_np(h, kept_l)
    for e, n in enumerate(kept_l):
        if n == 0:
            continue
        hr, yr = M.expert_forward(inp, cfg.act, e, xd[e, :n])
        _check_h(cfg, hn[e], hr, f"{name}: h[{e}]")
        _check_y(cfg, yn[e], yr, f"{name}: y_disp[{e}]")


def test_split_tiles_leave_counters_zero():
    """The pieces of a split tile count themselves in the workspace; the piece
    that completes a tile resets its counter.  Calls with different kept[]
    (other tiles split) on one workspace: a repeat of the first call gives the
    same bits, and every counter ends at zero."""
    cfg, C, kept_a = THIN_LAST["mixed-swiglu"]
    kept_b = [640, 640, 0, 65, 1, 300, 128, 129]
    log(f"[split counters] kept {kept_a}, then {kept_b}, then {kept_a} on one workspace")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(cfg.seed + 1)
    xd_bits = f32_to_bf16_bits(rng.standard_normal((cfg.E, C, cfg.H), dtype=np.float32))
    xd = bf16_bits_to_f32(xd_bits).astype(np.float64)
    layer = MoELayerGPU(cfg, inp, DEV, fused_gather=False)
    x_disp = torch.from_numpy(xd_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    nbytes = ops.moe_expert_ffn_ws_bytes()
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    tile = 256 * 256 * 4
    counters = ws[(nbytes // tile) * tile:]

    def run(kept_l):
        kept = to_dev(np.array(kept_l, dtype=np.int32), torch.int32)
        y, h = ops.moe_expert_ffn(x_disp, kept, layer.w1, layer.w3, layer.w2, act=cfg.act, ws=ws)
        torch.cuda.synchronize()
        assert int(counters.count_nonzero()) == 0, "tile counters left non-zero"
        return to_np(y).copy(), h.view(torch.int16).cpu().numpy().copy()

    y1, h1 = run(kept_a)
    y2, _ = run(kept_b)
    y3, h3 = run(kept_a)
    for e, n in enumerate(kept_a):
        assert np.array_equal(y3[e, :n].view(np.uint32), y1[e, :n].view(np.uint32)), f"y[{e}]"
        assert np.array_equal(h3[e, :n], h1[e, :n]), f"h[{e}]"
    for e, n in enumerate(kept_b):
        if n == 0:
            continue
        hr, yr = M.expert_forward(inp, cfg.act, e, xd[e, :n])
        _check_y(cfg, y2[e, :n], yr, f"second call: y_disp[{e}]")


# ---------------------------------------------------------- edge cases ----
def test_empty_and_degenerate_calls():
    log("[edge] T = 0, C = 0, zero-token experts")
    H, E, k = 256, 4, 2
    x = torch.zeros((0, H), dtype=torch.bfloat16, device=DEV)
    w_r = torch.zeros((H, E), dtype=torch.bfloat16, device=DEV)
    idx, w, p, _ = ops.moe_route(x, w_r, None, k)
    counts, f, pp, l_aux = ops.moe_aux_stats(idx, p, E, 0.01)
    x_disp, slot, slot_token, kept, dropped = ops.moe_dispatch(x, idx, E, 3)
    y = ops.moe_combine(torch.zeros((0, H), dtype=torch.float32, device=DEV), slot, w)
    fused = ops.moe_dispatch_aux(x, idx, p, E, 3, 0.01)
    torch.cuda.synchronize()
    assert y.shape == (0, H)
    assert to_np(counts).tolist() == [0] * E and float(to_np(l_aux)[0]) == 0.0
    assert to_np(kept).tolist() == [0] * E and int(to_np(dropped)[0]) == 0
    assert np.all(to_np(slot_token) == -1)
    _, _, st_f, kept_f, drop_f, cnt_f, f_f, p_f, la_f = fused
    assert np.all(to_np(st_f) == -1) and to_np(kept_f).tolist() == [0] * E
    assert int(to_np(drop_f)[0]) == 0 and to_np(cnt_f).tolist() == [0] * E
    assert np.all(to_np(f_f) == 0) and np.all(to_np(p_f) == 0) and float(to_np(la_f)[0]) == 0.0
    # C = 0: everything dropped, outputs exactly zero
    cfg = MoEConfig("c0", "bf16", T=40, H=256, I=128, E=4, k=2, cf=1.0, seed=3)
    inp = make_inputs(cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    xx = x_to_device(inp, cfg, DEV)
    layer.route(xx)
    x_disp, slot, slot_token, kept, dropped = ops.moe_dispatch(xx, layer.buf.topk_idx, 4, 0)
    torch.cuda.synchronize()
    assert np.all(to_np(slot) == -1) and int(to_np(dropped)[0]) == 80
    # (every slot is -1, so no expert row is read; one dummy row stands for y_disp)
    y = ops.moe_combine(torch.zeros((1, 256), dtype=torch.float32, device=DEV), slot,
                        layer.buf.topk_w)
    torch.cuda.synchronize()
    assert np.all(to_np(y) == 0.0)
    # zero-token experts: a zero router sends every token to experts 0..k-1
    inp2 = dict(inp, w_r=np.zeros_like(inp["w_r"]))
    ref = M.forward(inp2, cfg)
    layer2 = MoELayerGPU(cfg, inp2, DEV)
    y2, _ = layer2.forward(xx)
    torch.cuda.synchronize()
    assert to_np(layer2.buf.kept).tolist() == ref.disp.kept.tolist() == [20, 20, 0, 0]
    np.testing.assert_array_equal(to_np(layer2.buf.topk_idx), ref.route.idx)
    _check_y(cfg, to_np(y2), ref.y, "zero-router y", layer_out=True)


@pytest.mark.parametrize("T,E,k,cf", [(8192, 8, 2, 1.25), (8193, 8, 2, 1.25), (5461, 5, 3, 0.8),
                                       (5462, 5, 3, 0.8), (1024, 64, 8, 1.0), (1025, 64, 8, 1.0),
                                       (2048, 32, 2, 2.0), (2049, 32, 2, 2.0)])
def test_dispatch_and_aux_both_sizes(T, E, k, cf):
    """Dispatch and aux statistics on either side of the size where the aux
    statistics switch from one workgroup to the multi-block kernels (65536
    probabilities), with skewed loads so that some experts overflow:
    bit-exact integers, 1e-5 floats, x_disp rows exact copies."""
    log(f"[sizes] T={T} E={E} k={k} cf={cf}")
    rng = np.random.default_rng(T * 131 + E)
    skew = np.linspace(2.0, 0.0, E)              # uneven load, so some experts overflow
    keys = rng.standard_normal((T, E)) + skew
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    probs = np.exp(keys - keys.max(axis=1, keepdims=True))
    probs = (probs / probs.sum(axis=1, keepdims=True)).astype(np.float32)
    C = M.capacity(T, k, E, cf)
    H = 64
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV)
    idx_d, probs_d = to_dev(idx, torch.int32), to_dev(probs, torch.float32)
    x_disp, slot, slot_token, kept, dropped = ops.moe_dispatch(x, idx_d, E, C)
    counts, f, p, l_aux = ops.moe_aux_stats(idx_d, probs_d, E, 0.01)
    torch.cuda.synchronize()
    d = M.dispatch(idx.astype(np.int64), E, C)
    _dispatch_compare((to_np(slot), to_np(slot_token), to_np(kept), to_np(dropped)), d,
                      f"sizes T={T}")
    a = M.aux_stats(idx.astype(np.int64), probs.astype(np.float64), E, 0.01)
    np.testing.assert_array_equal(to_np(counts), a.counts)
    assert_rel(to_np(f), a.f, 1e-5, "f")
    assert_rel(to_np(p), a.P, 1e-5, "p")
    assert_rel(to_np(l_aux), [a.l_aux], 1e-5, "L_aux")
    xd = to_np(x_disp).reshape(E * C, H)
    st = d.slot_token.reshape(-1)
    rows = np.where(st >= 0)[0]
    np.testing.assert_array_equal(xd[rows], to_np(x)[st[rows]])
    # the fused pass (dispatch and statistics from the same launches)
    xf, slf, stf, kf, df, cf_, ff, pf, lf = ops.moe_dispatch_aux(x, idx_d, probs_d, E, C, 0.01)
    torch.cuda.synchronize()
    _dispatch_compare((to_np(slf), to_np(stf), to_np(kf), to_np(df)), d, f"fused T={T}")
    np.testing.assert_array_equal(to_np(cf_), a.counts)
    np.testing.assert_array_equal(to_np(ff), to_np(f))   # the same count / (T k)
    assert_rel(to_np(pf), a.P, 1e-5, "fused p")
    assert_rel(to_np(lf), [a.l_aux], 1e-5, "fused L_aux")
    np.testing.assert_array_equal(to_np(xf).reshape(E * C, H)[rows], to_np(x)[st[rows]])


def _skewed_routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((T, E)) + np.linspace(2.0, 0.0, E)   # some experts overflow
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    probs = np.exp(keys - keys.max(axis=1, keepdims=True))
    return idx, (probs / probs.sum(axis=1, keepdims=True)).astype(np.float32)


# 8192 assignments: 16 blocks of one 512-assignment pass; 16386: 33 blocks;
# 32770: 33 blocks of 512 x 2 (ranks in registers); 131072: 64 blocks of 4
# passes; 131074: 52 blocks of 5; then 10 and 13 passes at 16 and 64 experts
# (ranks recomputed after the block's first rows are known).  Up to 4096
# assignments one workgroup does it all (the small and decode cases).
@pytest.mark.parametrize("T,E,k,cf", [(4096, 8, 2, 1.25), (8192, 8, 2, 1.25),
                                       (8193, 8, 2, 1.25), (16385, 8, 2, 1.25),
                                       (65536, 8, 2, 1.25), (65537, 8, 2, 1.25),
                                       (150000, 16, 2, 1.0), (100000, 64, 4, 1.0)])
def test_dispatch_many_blocks_and_passes(T, E, k, cf):
    """The dispatch on both sides of the one-workgroup limit and with several
    512-assignment passes per block, in registers and recomputed: maps
    bit-exact against the oracle's walk, statistics within 1e-5."""
    log(f"[passes] T={T} E={E} k={k} cf={cf}")
    idx, probs = _skewed_routing(T, E, k, T + E)
    C = M.capacity(T, k, E, cf)
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device=DEV)
    idx_d, probs_d = to_dev(idx, torch.int32), to_dev(probs, torch.float32)
    _, slf, stf, kf, df, cnt, ff, pf, lf = ops.moe_dispatch_aux(x, idx_d, probs_d, E, C, 0.01,
                                                                copy=False)
    torch.cuda.synchronize()
    d = M.dispatch(idx.astype(np.int64), E, C)
    _dispatch_compare((to_np(slf), to_np(stf), to_np(kf), to_np(df)), d, f"passes T={T}")
    a = M.aux_stats(idx.astype(np.int64), probs.astype(np.float64), E, 0.01)
    np.testing.assert_array_equal(to_np(cnt), a.counts)
    assert_rel(to_np(ff), a.f, 1e-5, "f")
    assert_rel(to_np(pf), a.P, 1e-5, "p")
    assert_rel(to_np(lf), [a.l_aux], 1e-5, "L_aux")
    assert int(to_np(df)[0]) > 0, "the case should drop some assignments"


# the multi-block dispatch (more than 4096 assignments) at its degenerate
# cases: no capacity, one row per expert, one expert, every expert chosen
@pytest.mark.parametrize("T,E,k,C", [(5000, 8, 2, 0), (5000, 8, 2, 1), (9000, 1, 1, 9000),
                                     (700, 8, 8, 700), (3000, 64, 2, 37)])
def test_dispatch_degenerate_many_blocks(T, E, k, C):
    """Maps, kept, dropped and statistics bit-exact / within 1e-5 against the
    oracle's walk in the one-launch dispatch's multi-block form."""
    log(f"[degenerate] T={T} E={E} k={k} C={C}")
    idx, probs = _skewed_routing(T, E, k, 3 * T + E)
    x = torch.zeros((T, 64), dtype=torch.bfloat16, device=DEV)
    idx_d, probs_d = to_dev(idx, torch.int32), to_dev(probs, torch.float32)
    _, slf, stf, kf, df, cnt, ff, pf, lf = ops.moe_dispatch_aux(x, idx_d, probs_d, E, C, 0.01,
                                                                copy=False)
    _, sl2, st2, k2, d2 = ops.moe_dispatch(x, idx_d, E, C, copy=False)
    torch.cuda.synchronize()
    d = M.dispatch(idx.astype(np.int64), E, C)
    _dispatch_compare((to_np(slf), to_np(stf), to_np(kf), to_np(df)), d, f"aux T={T} C={C}")
    _dispatch_compare((to_np(sl2), to_np(st2), to_np(k2), to_np(d2)), d, f"maps T={T} C={C}")
    a = M.aux_stats(idx.astype(np.int64), probs.astype(np.float64), E, 0.01)
    np.testing.assert_array_equal(to_np(cnt), a.counts)
    assert_rel(to_np(pf), a.P, 1e-5, "p")
    assert_rel(to_np(lf), [a.l_aux], 1e-5, "L_aux")


def test_dispatch_workspace_shared_across_shapes():
    """One zero-filled workspace, sized for the largest call, shared by
    moe_aux_stats, moe_dispatch and moe_dispatch_aux at different shapes in
    turn: every output bitwise equal to the same call on a fresh workspace,
    and after every call the whole workspace (counters, count and sum words)
    is zero again."""
    shapes = [(40000, 16, 2), (3000, 8, 2), (20000, 64, 3), (9000, 16, 2), (40000, 16, 2)]
    ws = torch.zeros(max(ops.moe_workspace_bytes(T, E, k) for T, E, k in shapes),
                     dtype=torch.uint8, device=DEV)
    for n, (T, E, k) in enumerate(shapes):
        log(f"[shared ws] call {n}: T={T} E={E} k={k}")
        idx, probs = _skewed_routing(T, E, k, 7 * n + 1)
        idx_d, probs_d = to_dev(idx, torch.int32), to_dev(probs, torch.float32)
        C = M.capacity(T, k, E, 1.0)
        x = torch.zeros((T, 64), dtype=torch.bfloat16, device=DEV)
        for kind in ("aux", "dispatch", "dispatch_aux"):
            if kind == "aux":
                got = ops.moe_aux_stats(idx_d, probs_d, E, 0.01, ws=ws)
                want = ops.moe_aux_stats(idx_d, probs_d, E, 0.01)
            elif kind == "dispatch":
                got = ops.moe_dispatch(x, idx_d, E, C, ws=ws, copy=False)[1:]
                want = ops.moe_dispatch(x, idx_d, E, C, copy=False)[1:]
            else:
                got = ops.moe_dispatch_aux(x, idx_d, probs_d, E, C, 0.01, ws=ws, copy=False)[1:]
                want = ops.moe_dispatch_aux(x, idx_d, probs_d, E, C, 0.01, copy=False)[1:]
            torch.cuda.synchronize()
            for g, w in zip(got, want):
                assert torch.equal(g, w), f"call {n} {kind}: outputs differ"
            words = ws[:256].cpu().numpy()
            assert not words.any(), f"call {n} {kind}: counters not cleared"
            assert not ws[256:].cpu().numpy().any(), f"call {n} {kind}: words not cleared"


@pytest.mark.parametrize("T", [1, 16, 64, 256])
def test_decode_drop_free(T):
    """Drop-free decode steps (C = T): nothing dropped, every token's output
    within tolerance; T = 1 gives each selected expert a single row."""
    cfg = drop_free(MoEConfig("decode", "bf16", T=T, H=512, I=512, E=8, k=2, cf=1.0,
                              batch=T, seq=1, seed=20 + T))
    log(f"[decode] T={T} C={M.capacity(T, cfg.k, cfg.E, cfg.cf)}")
    inp = make_inputs(cfg)
    ref = M.forward(inp, cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    assert layer.C == T
    x = x_to_device(inp, cfg, DEV)
    y, _ = layer.forward(x)
    torch.cuda.synchronize()
    b = layer.buf
    assert int(to_np(b.dropped)[0]) == 0 and ref.disp.dropped == 0
    same = _route_compare(cfg, to_np(b.topk_idx), to_np(b.topk_w), to_np(b.probs), None,
                          ref.route, f"decode T={T}")
    _check_y(cfg, to_np(y)[same], ref.y[same], f"decode T={T}: y", layer_out=True)


def test_decode_config_full_size():
    """The 64-token drop-free decode step on the full-size layer (H 2048,
    I 4096, E 8): the workload `bench.py --config 6` times."""
    cfg = CONFIGS[6]
    log(f"[decode] config 6 {cfg.name}")
    inp = make_inputs(cfg)
    ref = M.forward(inp, cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    x = x_to_device(inp, cfg, DEV)
    y, l_aux = layer.forward(x)
    torch.cuda.synchronize()
    b = layer.buf
    assert int(to_np(b.dropped)[0]) == 0
    same = _route_compare(cfg, to_np(b.topk_idx), to_np(b.topk_w), to_np(b.probs), None,
                          ref.route, "config 6")
    assert_rel(to_np(l_aux), [ref.aux.l_aux], 1e-5, "config 6: L_aux")
    worst = _check_y(cfg, to_np(y)[same], ref.y[same], "config 6: y", layer_out=True)
    log(f"[decode] config 6: worst err/rms {worst:.3e}")


def test_deterministic_bitwise():
    cfg = SMALL["bf16-swiglu-e8"]
    log("[det] two runs bitwise identical")
    inp = make_inputs(cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    x = x_to_device(inp, cfg, DEV)
    y1, a1 = layer.forward(x)
    torch.cuda.synchronize()
    snap = {n: getattr(layer.buf, n).clone() for n in ("topk_idx", "topk_w", "probs", "slot",
                                                       "slot_token", "kept", "y", "l_aux", "p")}
    layer.forward(x)
    torch.cuda.synchronize()
    for n, t in snap.items():
        assert torch.equal(t, getattr(layer.buf, n)), n


# ---------------------------------------------------- full-size configs ----
def _rows_np(t: torch.Tensor, kept) -> list:
    """Per expert, the first kept[e] rows of a [E, C, N] buffer as float64
    (rows past kept[e] are never written and are not converted)."""
    return [to_np(t[e, :int(n)]) for e, n in enumerate(kept)]


def _check_expert_rows(cfg, inp, yd_rows, st_gpu, d_ref, ref_ydisp, what):
    """Every kept row of every expert: GPU y_disp against the oracle's
    expert output for the token in that row (rows whose token differs from
    the oracle's dispatch, after a near-tie flip upstream, are recomputed by
    the oracle for the GPU's token).  Returns the worst err / RMS(row)."""
    x = inp["x"]
    worst = 0.0
    for e, rows in enumerate(yd_rows):
        n = rows.shape[0]
        if n == 0:
            continue
        want = np.zeros_like(rows)
        same = np.zeros(n, dtype=bool)
        m = min(n, int(d_ref.kept[e]))
        same[:m] = st_gpu[e, :m] == d_ref.slot_token[e, :m]
        want[same] = ref_ydisp[e, :n][same]
        if not same.all():
            _, ye = M.expert_forward(inp, cfg.act, e, M.widen(x[st_gpu[e, :n][~same]]))
            want[~same] = ye
        worst = max(worst, _check_y(cfg, rows, want, f"{what}: y_disp[{e}]"))
    return worst


def test_full_config2_with_shared_expert():
    """The 4096-token layer plus a shared expert of intermediate size 4096
    (enqueued first on the same stream as the routed path): every row."""
    cfg = CONFIGS[2].with_(shared_I=4096)
    log("[full] config 2 + shared expert (I_s 4096), every row")
    inp = make_inputs(cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    x = x_to_device(inp, cfg, DEV)
    y, _ = layer.forward(x)
    torch.cuda.synchronize()
    b = layer.buf
    ref = M.forward(inp, cfg)
    same = np.all(to_np(b.topk_idx) == ref.route.idx, axis=1)
    ok = same & np.all(to_np(b.slot) == ref.disp.slot, axis=1)
    _check_y(cfg, to_np(b.sh_y)[0], ref.y_shared, "config 2: shared expert (every row)")
    worst = _check_y(cfg, to_np(y)[ok], ref.y[ok], "config 2 + shared: y", layer_out=True)
    log(f"[full] config 2 + shared: {int(ok.sum())}/{cfg.T} rows, worst err/rms {worst:.3e}")


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_config(cid):
    """A full-size workload in the launch configuration the benchmark times
    (fused gather, split tail rounds), against the whole oracle forward:
    routing, statistics and dispatch on every token, every kept expert row of
    y_disp, and every row of y whose routing agrees (the others are near
    ties, counted; their expert rows are still checked)."""
    cfg = CONFIGS[cid]
    log(f"[full] config {cid} {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} "
        f"k={cfg.k} cf={cfg.cf} {cfg.act} {cfg.route}")
    inp = make_inputs(cfg)
    layer = MoELayerGPU(cfg, inp, DEV)
    x = x_to_device(inp, cfg, DEV)
    y, l_aux = layer.forward(x, keys=True)
    torch.cuda.synchronize()
    log(f"[full] config {cid}: GPU forward done")
    assert layer.buf.x_disp is None   # the fused-gather path, as the benchmark runs it
    b = layer.buf
    ref = M.forward(inp, cfg)
    log(f"[full] config {cid}: oracle forward done ({sum(ref.timings.values()):.1f} s)")
    r = ref.route
    same = _route_compare(cfg, to_np(b.topk_idx), to_np(b.topk_w), to_np(b.probs), to_np(b.keys),
                          r, f"config {cid}")
    gidx = to_np(b.topk_idx).astype(np.int64)
    C = M.capacity(cfg.T, cfg.k, cfg.E, cfg.cf)
    assert C == layer.C
    d_gpu = M.dispatch(gidx, cfg.E, C)
    st_gpu = to_np(b.slot_token)
    _dispatch_compare((to_np(b.slot), st_gpu, to_np(b.kept), to_np(b.dropped)), d_gpu,
                      f"config {cid}")
    assert_rel(to_np(l_aux), [ref.aux.l_aux], 1e-5, f"config {cid}: L_aux")
    assert_rel(to_np(b.p), ref.aux.P, 1e-5, f"config {cid}: p", atol=1e-12)
    if same.all():
        np.testing.assert_array_equal(to_np(b.counts), ref.aux.counts)
    kept = to_np(b.kept)
    w1 = _check_expert_rows(cfg, inp, _rows_np(b.y_disp, kept), st_gpu, ref.disp, ref.y_disp,
                            f"config {cid}")
    ok = same & np.all(to_np(b.slot) == ref.disp.slot, axis=1)
    w2 = _check_y(cfg, to_np(y)[ok], ref.y[ok], f"config {cid}: y", layer_out=True)
    log(f"[full] config {cid}: dropped {d_gpu.dropped}, y compared on {int(ok.sum())}/{cfg.T} "
        f"rows, every kept expert row compared; worst err/rms y_disp {w1:.3e}, y {w2:.3e}")


@pytest.mark.parametrize("cid", [2, 4])
def test_full_config_expert_stages(cid):
    """The expert products at full size fed the oracle's dispatch, with and
    without the split-tail workspace: h and y_disp on every kept row of
    every expert (workload 2: ragged experts with thin last row tiles and a
    split last round; workload 4: the GELU expert with both biases at
    I = 16384).  Then the combine of the oracle's expert outputs, every row."""
    cfg = CONFIGS[cid]
    log(f"[full stages] config {cid} {cfg.name}")
    inp = make_inputs(cfg)
    ref = M.forward(inp, cfg, keep_h=True)
    layer = MoELayerGPU(cfg, inp, DEV)
    x = x_to_device(inp, cfg, DEV)
    st = to_dev(ref.disp.slot_token.astype(np.int32), torch.int32)
    kept = to_dev(ref.disp.kept.astype(np.int32), torch.int32)
    for ws in (layer.buf.ffn_ws, None):
        yg, hg = ops.moe_expert_ffn_gather(x, st, kept, layer.w1, layer.w3, layer.w2, layer.b1,
                                           layer.b2, act=cfg.act, ws=ws)
        torch.cuda.synchronize()
        tag = "split tails" if ws is not None else "whole tiles"
        for e, n in enumerate(ref.disp.kept):
            n = int(n)
            if n == 0:
                continue
            _check_h(cfg, to_np(hg[e, :n]), ref.h[e, :n], f"config {cid} ({tag}): h[{e}]")
            _check_y(cfg, to_np(yg[e, :n]), ref.y_disp[e, :n], f"config {cid} ({tag}): y_disp[{e}]")
        log(f"[full stages] config {cid} ({tag}): h and y_disp on every kept row")
        del yg, hg
    ydisp_store = ref.y_disp.astype(np.float32)
    w32 = ref.route.w.astype(np.float32)
    y = ops.moe_combine(to_dev(ydisp_store, torch.float32),
                        to_dev(ref.disp.slot.astype(np.int32), torch.int32),
                        to_dev(w32, torch.float32), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = M.combine(ydisp_store.astype(np.float64), ref.disp.slot, w32.astype(np.float64), cfg.H)
    got = to_np(y)
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-30 +
                  1e-6 * np.sqrt(np.mean(want * want, axis=1, keepdims=True))), "combine"
