"""Benchmark: one sparse-MoE FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--gpus 1]

A step is one whole layer forward (route, dispatch of the row maps with the
aux statistics in the same pass, the grouped expert GEMM whose first product
gathers its rows from x, combine) over one batch of synthetic input that is
already resident in HBM.
The default workload is the 2 x 2048-token layer (hidden 2048, SwiGLU
intermediate 4096, 8 experts, top-2, capacity factor 1.25, bf16 with fp32
accumulation); --config 6 is the drop-free 64-token decode step on the same
layer.  Prints one JSON line.

Timing:
  * the timed region is exactly K whole-layer forwards, bracketed by device
    synchronisation, with nothing else enqueued (it sets ms_per_step and
    value);
  * K more steps follow with HIP events on the launch stream between the
    phases, so each phase's average duration is reported too (the expert
    phase dominates and gives `roofline`, against the matrix-core peak or,
    when its weights take longer to stream than its FLOP to compute, against
    HBM);
  * memory-bound phases are also timed in isolation after a 1 GiB write that
    flushes the 256 MB Infinity Cache, so their bytes come from HBM;
  * the CPU oracle (float64, the reference implementation) is timed on the
    host cores on one full layer forward of the same workload.

Further measurements, each added to the same JSON line: --backward (a
training step: forward keeping the dispatched rows, then the combine, expert,
dispatch and router backward, per phase), --weights fp8 (the layer on 8-bit
e4m3 expert weights), --shared I_S (the layer plus a shared expert of
intermediate size I_S), --copy-calibration (three plain 256 MiB device
copies, the reference for the HBM traffic counters).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + grouped-GEMM % MFMA peak, dispatch % HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--iso-reps", type=int, default=10)
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (combine, expert FFN, dispatch and router "
                         "backward) after a forward that keeps the dispatched rows")
    ap.add_argument("--weights", choices=["bf16", "fp8"], default="bf16",
                    help="expert weight storage: bf16, or 8-bit e4m3 codes with per-expert, "
                         "per-column scales (quantised on the device before timing)")
    ap.add_argument("--shared", type=int, default=0, metavar="I_S",
                    help="also time the layer with a shared expert of intermediate size I_S "
                         "(every token, weight 1)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three plain 256 MiB device copies (read 256 MiB, write "
                         "256 MiB each), the reference for HBM traffic counters")
    return ap.parse_args()


def algorithmic_work(cfg, kept: np.ndarray, dropped: int, weights: str = "bf16"):
    """Bytes and FLOP each phase must move / compute at minimum."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    esz = 2 if cfg.dtype == "bf16" else 4
    wsz = 1 if weights == "fp8" else esz
    n_kept = int(kept.sum())
    mult = 6 if cfg.act == "swiglu" else 4
    ffn_flop = mult * H * I * n_kept
    # expert phase: the weights of every expert that has rows (read once),
    # the gathered x rows, h written and read back, fp32 y_disp written
    n_mats = 3 if cfg.act == "swiglu" else 2
    active = int((kept > 0).sum())
    ffn_bytes = (active * n_mats * H * I * wsz + n_kept * H * esz + 2 * n_kept * I * esz
                 + n_kept * H * 4)
    if weights == "fp8":  # the per-column fp32 scales
        ffn_bytes += active * ((n_mats - 1) * I + H) * 4
    route_bytes = T * H * esz + H * E * esz + T * k * 8 + T * E * 4
    # fused-gather layer: dispatch only maps rows (idx read, slot + slot_token
    # written; the row copy happens inside the first expert product's loads),
    # and it computes the aux statistics in the same pass (probs read once)
    dispatch_bytes = T * k * 4 + T * k * 4 + n_kept * 4 + T * E * 4
    # kept expert rows (fp32) read once, y written once, slot + weights read
    combine_bytes = n_kept * H * 4 + T * H * esz + T * k * 8
    return dict(n_kept=n_kept, ffn_flop=ffn_flop, ffn_bytes=ffn_bytes, route_bytes=route_bytes,
                dispatch_bytes=dispatch_bytes, combine_bytes=combine_bytes, dropped=dropped)


TRAFFIC_PROFILES = {
    "layer-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_layer_bf16_4096tok_traffic.md"),
    "decode-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_decode_bf16_64tok_traffic.md"),
}
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_08_amd", "csrc", "expert_ffn.hip")


def measured_traffic(cfg):
    """HBM bytes per expert phase from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when that summary is
    for another workload or for another version of the GEMM source."""
    import re
    path = TRAFFIC_PROFILES.get(cfg.name)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_layer_call:\s*(\d+)", text)
    m_h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m_b or not m_h:
        return None
    if gemm_source_digest() != m_h.group(1):
        return None
    return int(m_b.group(1))


def gemm_source_digest() -> str:
    """sha256 of the GEMM source with comments and blank space removed, so
    that only a change to the code itself invalidates recorded counters."""
    import hashlib
    import re
    text = open(GEMM_SOURCE).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def cpu_baseline(cfg, inputs):
    """The CPU oracle as it stands, timed on one full layer forward."""
    from oracle import moe_oracle as M
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    threads = max([n for _, n in blas if n] or [1])
    # repeat whole forwards until about 10 s of CPU work has been timed
    runs, dt = 0, 0.0
    while True:
        t0 = time.perf_counter()
        res = M.forward(inputs, cfg)
        dt += time.perf_counter() - t0
        runs += 1
        if dt >= 10.0 or runs >= 50:
            break
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(runs * cfg.T / dt, 3), "unit": "tokens/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{runs} full layer forwards of the same workload ({cfg.T} tokens each), "
                  f"float64 numpy with BLAS products; {dt:.2f} s in total",
        "affinity_cores": len(os.sched_getaffinity(0)), "cpu": cpu_model, "blas": blas,
        "phase_s": {k: round(v, 4) for k, v in res.timings.items()},
    }


def bench_backward(cfg, inputs, dev, args):
    """Training step: the training forward (dispatched rows and the first
    expert product's planes kept) + backward, with per-phase events."""
    import torch
    from mixture_experts_layer_08_amd import ops
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
    layer = MoELayerGPU(cfg, inputs, dev, fused_gather=False)
    x = x_to_device(inputs, cfg, dev)
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    dy = torch.randn((cfg.T, cfg.H), generator=g).to(layer.tdtype).to(dev)
    b = layer.buf
    stream = torch.cuda.current_stream()

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        rec(0)
        layer.forward_train(x)
        rec(1)
        dy_disp, dw = ops.moe_combine_bwd(dy, b.y_disp, b.slot, b.topk_w)
        rec(2)
        gr = ops.moe_expert_ffn_bwd(b.x_disp, b.kept, layer.w1, layer.w3, layer.w2, layer.b1,
                                    dy_disp, act=cfg.act, has_b2=layer.b2 is not None,
                                    ws=layer.bws, saved=True)
        rec(3)
        dx = ops.moe_dispatch_bwd(gr["dx_disp"], b.slot)
        rec(4)
        ops.moe_route_bwd(x, layer.w_r, b.probs, b.topk_idx, b.topk_w, dw, b.f, alpha=cfg.alpha,
                          dl_aux=1.0, mode=cfg.route, seq_len=cfg.seq_len, dx=dx,
                          bias=layer.b_r is not None)
        rec(5)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    K = max(1, args.steps // 2)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    t0 = time.perf_counter()
    for s_ in range(K):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K
    names = ["forward", "combine_bwd", "expert_ffn_bwd", "dispatch_bwd", "route_bwd"]
    ph = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    n_kept = int(b.kept.cpu().numpy().sum())
    # dh + dX + the weight gradients (the first product's planes come from
    # the training forward, so the backward does not recompute them)
    mult = 12 if cfg.act == "swiglu" else 8
    bwd_flop = mult * cfg.H * cfg.I * n_kept
    tf = bwd_flop / (ph["expert_ffn_bwd"] * 1e-3) / 1e12
    return {"train_step_ms": round(wall * 1e3, 5), "train_tokens_per_s": round(cfg.T / wall, 1),
            "steps": K, "phases_ms": {k: round(v, 5) for k, v in ph.items()},
            "expert_ffn_bwd": {"flop": bwd_flop, "TFLOP/s": round(tf, 2),
                               "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def bench_shared(cfg, dev, args):
    """The layer plus a shared expert of intermediate size args.shared: the
    whole forward, and the shared expert's own launches alone."""
    import torch
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
    from mixture_experts_layer_08_amd.synth import make_inputs
    scfg = cfg.with_(shared_I=args.shared)
    inputs = make_inputs(scfg)
    layer = MoELayerGPU(scfg, inputs, dev)
    x = x_to_device(inputs, scfg, dev)
    stream = torch.cuda.current_stream()

    res = {}
    for name, fn in (("layer", lambda: layer.forward(x)), ("shared", lambda: layer.shared_expert(x))):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        K = max(1, args.steps)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / K
    n_kept = int(layer.buf.kept.cpu().numpy().sum())
    per_row = (6 if cfg.act == "swiglu" else 4) * cfg.H
    flop = per_row * (cfg.I * n_kept + args.shared * cfg.T)
    ms = res["layer"]
    sh_flop = per_row * args.shared * cfg.T
    return {"shared_intermediate": args.shared, "ms_per_step": round(ms, 5),
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "expert_flop": flop,
            "shared_expert_ms": round(res["shared"], 5),
            "shared_expert_TFLOP/s": round(sh_flop / (res["shared"] * 1e-3) / 1e12, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
    from mixture_experts_layer_08_amd.synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    print(f"[bench] generating inputs for {cfg.name}", file=sys.stderr, flush=True)
    inputs = make_inputs(cfg)
    dev = "cuda:0"
    layer = MoELayerGPU(cfg, inputs, dev, weights=args.weights)
    x = x_to_device(inputs, cfg, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    K = args.steps
    # the timed region: K whole-layer forwards, nothing else enqueued
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        layer.forward(x)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K steps again with HIP events between the phases (on the launch
    # stream) for the per-phase times; the events add a little time per step,
    # so this loop does not set ms_per_step
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        layer.route(x)
        e[1].record(stream)
        layer.dispatch_aux(x)
        e[2].record(stream)
        layer.experts(x)
        e[3].record(stream)
        layer.combine()
        e[4].record(stream)
    torch.cuda.synchronize()
    names = ["route", "dispatch", "expert_ffn", "combine"]
    ph = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)]))
          for i, n in enumerate(names)}
    dev_ms = float(np.mean([ev[s][0].elapsed_time(ev[s][4]) for s in range(K)]))
    ms_per_step = wall * 1e3 / K
    print(f"[bench] timed {K} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    kept = layer.buf.kept.cpu().numpy()
    dropped = int(layer.buf.dropped.cpu()[0])
    work = algorithmic_work(cfg, kept, dropped, args.weights)

    # memory-bound phases in isolation, after flushing the Infinity Cache
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    iso = {}
    for n, fn in (("route", lambda: layer.route(x)), ("dispatch", lambda: layer.dispatch_aux(x)),
                  ("combine", layer.combine)):
        ts = []
        for _ in range(args.iso_reps):
            flush.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        iso[n] = float(np.median(ts))
    del flush
    layer.forward(x)        # leave buffers consistent
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    gemm_ms = ph["expert_ffn"]
    achieved_tflops = work["ffn_flop"] / (gemm_ms * 1e-3) / 1e12
    phases = {}
    for n, key in (("route", "route_bytes"), ("dispatch", "dispatch_bytes"),
                   ("combine", "combine_bytes")):
        gbs = work[key] / (ph[n] * 1e-3) / 1e9
        phases[n] = {"ms": round(ph[n], 5), "bytes": work[key], "GB/s": round(gbs, 1),
                     "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        if n in iso:
            g2 = work[key] / (iso[n] * 1e-3) / 1e9
            phases[n].update({"ms_cold": round(iso[n], 5), "GB/s_cold": round(g2, 1),
                              "hbm_frac_cold": round(g2 / PEAK_HBM_GBS, 4)})
    ffn_gbs = work["ffn_bytes"] / (gemm_ms * 1e-3) / 1e9
    phases["expert_ffn"] = {"ms": round(gemm_ms, 5), "flop": work["ffn_flop"],
                            "TFLOP/s": round(achieved_tflops, 2),
                            "mfma_frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                            "bytes": work["ffn_bytes"], "GB/s": round(ffn_gbs, 1),
                            "hbm_frac": round(ffn_gbs / PEAK_HBM_GBS, 4)}
    # the expert phase is bound by whichever peak it would take longer at:
    # the matrix cores for many rows per expert, HBM (the weights) for few
    t_mfma = work["ffn_flop"] / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = work["ffn_bytes"] / (PEAK_HBM_GBS * 1e9)
    kernel = ("grouped expert GEMM (moe_expert_ffn_gather" +
              ("_fp8, e4m3 weights" if args.weights == "fp8" else "") + ": " +
              ("gate/up product with SwiGLU epilogue" if cfg.act == "swiglu" else
               "first product with bias + GELU epilogue") +
              ", then down product; split last rounds finished in-kernel)")
    if t_hbm > t_mfma:
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(ffn_gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ffn_gbs / PEAK_HBM_GBS, 4),
                    "bytes_per_launch": work["ffn_bytes"]}
    else:
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved_tflops, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved_tflops / PEAK_BF16_TFLOPS, 4),
                    "flop_per_launch": work["ffn_flop"]}
    roofline.update({"traffic": measured_traffic(cfg) if args.weights == "bf16" else None,
                     "traffic_unit": "HBM bytes per expert phase (rocprofv3 FETCH_SIZE x2.0 + "
                                     "WRITE_SIZE x1.0, copy-calibrated)",
                     "avg_ms": round(gemm_ms, 5)})

    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one MoE FFN layer forward, T={cfg.T} "
                               f"({cfg.batch}x{cfg.seq_len}), H={cfg.H}, I={cfg.I}, E={cfg.E}, "
                               f"top-{cfg.k}, cf={cfg.cf}, {cfg.act}, {cfg.route} router" +
                               (", e4m3 expert weights with per-column scales"
                                if args.weights == "fp8" else ""),
                   "expert_weights": args.weights,
                   "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E,
                   "top_k": cfg.k, "capacity_factor": cfg.cf,
                   "capacity": layer.C, "kept_rows": work["n_kept"], "dropped": dropped,
                   "path": "route, dispatch (row maps) with aux statistics, gather-fused expert products, "
                           "combine"},
        "roofline": roofline,
        "phases": phases,
        "device_ms_per_step": round(dev_ms, 5),
    }
    if args.backward:
        out["backward"] = bench_backward(cfg, inputs, dev, args)
    if args.shared:
        out["shared_expert"] = bench_shared(cfg, dev, args)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
