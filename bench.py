"""Benchmark: one sparse-MoE FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 5] [--also 2,3,4] [--gpus 1]

A step is one whole layer forward (route, dispatch of the row maps with the
aux statistics in the same pass, the grouped expert GEMM whose first product
gathers its rows from x, combine) over one batch of synthetic input that is
already resident in HBM.

The headline workload is the largest one: the long-context layer (T = 32768
tokens in one sequence, hidden 2048, SwiGLU intermediate 5632, 32 experts,
top-2 Gumbel hard routing at temperature 1 + 1e-4 * 32768, capacity factor
1.25, bf16 with fp32 accumulation).  The other workloads (--also, default the
4096-token layer, the skewed 16384-token layer and the wide GELU layer) are
measured the same way in the same process and reported as sub-records of the
one JSON line ("workloads").  --config 6 is the drop-free 64-token decode step.

Timing, per workload:
  * the timed region is exactly K whole-layer forwards, bracketed by device
    synchronisation; HIP events recorded on the launch stream between the
    phases inside that region give each phase's average duration, so
    `value` (tokens per second of the region) and `roofline` (the expert
    phase: both grouped-GEMM launches) come from the same steps;
  * the same K steps without events follow (`ms_per_step_no_events`: what
    the events cost);
  * the GPU shader clock is sampled during the timed region where the
    driver exposes it (sysfs pp_dpm_sclk);
  * memory-bound phases are also timed alone after a 1 GiB write that
    flushes the 256 MB Infinity Cache, so their bytes come from HBM; the
    dispatch that copies rows into the per-expert buffer (the unfused path)
    is timed the same way, as the HBM figure of dispatch;
  * the CPU oracle (float64, the reference implementation) is timed on the
    host cores on one or more full layer forwards of the same workload.

Further measurements, each added to the same JSON line: --backward (a
training step: forward keeping the dispatched rows, then the combine, expert,
dispatch and router backward, per phase), --weights fp8 (the layer on 8-bit
e4m3 expert weights), --shared I_S (the layer plus a shared expert of
intermediate size I_S), --graph (the forward captured into a HIP graph and
replayed), --copy-calibration (three plain 256 MiB device
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
    ap.add_argument("--config", type=int, default=5,
                    help="headline workload (default 5, the long-context 32768-token layer)")
    ap.add_argument("--also", default="2,3,4",
                    help="other workloads measured in the same run, comma-separated ids "
                         "('' for none); each becomes a sub-record of the JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer forward captured into a HIP graph and replayed")
    ap.add_argument("--no-fused-combine", action="store_true",
                    help="skip the sub-record of the layer with the combine fused into the "
                         "down product")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle forwards are repeated until this much CPU time is timed")
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
    # the unfused dispatch also copies the kept rows: x read once, N_kept rows
    # written, on top of the maps
    copy_dispatch_bytes = T * H * esz + n_kept * H * esz + T * k * 4 + T * k * 4 + n_kept * 4
    # kept expert rows (fp32) read once, y written once, slot + weights read
    combine_bytes = n_kept * H * 4 + T * H * esz + T * k * 8
    return dict(n_kept=n_kept, ffn_flop=ffn_flop, ffn_bytes=ffn_bytes, route_bytes=route_bytes,
                dispatch_bytes=dispatch_bytes, copy_dispatch_bytes=copy_dispatch_bytes,
                combine_bytes=combine_bytes, dropped=dropped)


TRAFFIC_PROFILES = {
    "layer-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_layer_bf16_4096tok_traffic.md"),
    "skewed-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_skewed_bf16_16384tok_traffic.md"),
    "wide-gelu-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_wide_gelu_bf16_8192tok_traffic.md"),
    "long-gumbel-bf16": os.path.join(ROOT, "profiles",
                                     "grouped_gemm_long_gumbel_bf16_32768tok_traffic.md"),
    "decode-bf16": os.path.join(ROOT, "profiles", "grouped_gemm_decode_bf16_64tok_traffic.md"),
}
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_08_amd", "csrc", f)
                for f in ("expert_ffn.hip", "gemm_common.h")]


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
    """sha256 of the GEMM sources with comments and blank space removed, so
    that only a change to the code itself invalidates recorded counters."""
    import hashlib
    import re
    text = "\n".join(open(p).read() for p in GEMM_SOURCES)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def cpu_baseline(cfg, inputs, seconds: float = 10.0):
    """The CPU oracle as it stands, timed on whole layer forwards of the
    workload (all T tokens each), repeated until `seconds` of CPU time have
    been timed (at least one)."""
    from oracle import moe_oracle as M
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    threads = max([n for _, n in blas if n] or [1])
    runs, dt = 0, 0.0
    res = None
    while True:
        t0 = time.perf_counter()
        res = M.forward(inputs, cfg)
        dt += time.perf_counter() - t0
        runs += 1
        if dt >= seconds or runs >= 50:
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
        "sample": f"{runs} full layer forward(s) of the same workload ({cfg.T} tokens each), "
                  f"float64 numpy with BLAS products; {dt:.2f} s in total",
        "affinity_cores": len(os.sched_getaffinity(0)), "cpu": cpu_model, "blas": blas,
        "phase_s": {k: round(v, 4) for k, v in res.timings.items()},
    }


class ClockSampler:
    """Samples the GPU shader clock (the active level of sysfs pp_dpm_sclk)
    from a host thread while the timed region runs; empty where the driver
    does not expose it."""

    def __init__(self, period_s: float = 0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import re
        for p in self.paths:
            try:
                for line in open(p):
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            return int(m.group(1))
            except OSError:
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self.paths:
            self._thr.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thr.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.array(self.samples)
        return {"samples": int(a.size), "mhz_median": float(np.median(a)),
                "mhz_min": int(a.min()), "mhz_max": int(a.max()),
                "source": "sysfs pp_dpm_sclk, active level"}


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


def bench_fused_combine(cfg, inputs, dev, args, plain_ms):
    """The same forward with the combine fused into the down product
    (moe_expert_ffn_gather_combine): K steps with events around route,
    dispatch and the fused expert call, then K steps with nothing else
    enqueued.  plain_ms: the unfused layer's expert + combine phases."""
    import torch
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device

    layer = MoELayerGPU(cfg, inputs, dev, fused_combine=True)
    x = x_to_device(inputs, cfg, dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t0 = time.perf_counter()
    for s_ in range(K):
        e = ev[s_]
        e[0].record(stream)
        layer.route(x)
        e[1].record(stream)
        layer.dispatch_aux(x)
        e[2].record(stream)
        layer.experts_combine(x)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fused_ms = float(np.mean([ev[s_][2].elapsed_time(ev[s_][3]) for s_ in range(K)]))
    t0 = time.perf_counter()
    for _ in range(K):
        layer.forward(x)
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / K
    del layer, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    ms = wall * 1e3 / K
    print(f"[bench] {cfg.name}: fused combine {ms:.4f} ms/step ({ms_plain:.4f} without events), "
          f"expert products + combine {fused_ms:.4f} ms (unfused {plain_ms:.4f})",
          file=sys.stderr, flush=True)
    return {"value": round(cfg.T / (ms_plain * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms, 5), "ms_per_step_no_events": round(ms_plain, 5),
            "experts_and_combine_ms": round(fused_ms, 5),
            "unfused_experts_and_combine_ms": round(plain_ms, 5),
            "path": "route, dispatch with aux statistics, gather-fused expert products with the "
                    "combine in the down product's epilogue (moe_expert_ffn_gather_combine)"}


def bench_graph(cfg, inputs, dev, args, eager_ms):
    """The same forward captured into a HIP graph (MoELayerGPU.graph) and
    replayed: K replays between two synchronisations.  eager_ms: the eager
    layer's ms per step without events."""
    import torch
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device

    layer = MoELayerGPU(cfg, inputs, dev, weights=args.weights)
    x = x_to_device(inputs, cfg, dev)
    g = layer.graph(x)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    del g, layer, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"[bench] {cfg.name}: graph replay {ms:.4f} ms/step (eager {eager_ms:.4f})",
          file=sys.stderr, flush=True)
    return {"value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 5),
            "eager_ms_per_step": round(eager_ms, 5),
            "path": "the layer forward captured once into a HIP graph, replayed K times"}


def workload_name(cfg, weights):
    return (f"{cfg.name}: one MoE FFN layer forward, T={cfg.T} ({cfg.batch}x{cfg.seq_len}), "
            f"H={cfg.H}, I={cfg.I}, E={cfg.E}, top-{cfg.k}, cf={cfg.cf}, {cfg.act}, "
            f"{cfg.route} router" + (", router bias +2 on expert 0" if cfg.router_bias0 else "")
            + (", e4m3 expert weights with per-column scales" if weights == "fp8" else ""))


def run_workload(cid, args, with_cpu: bool):
    """Measure one workload; returns its record (the fields of the JSON line)."""
    import torch
    from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
    from mixture_experts_layer_08_amd.synth import CONFIGS, make_inputs

    cfg = CONFIGS[cid]
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inputs = make_inputs(cfg)
    dev = "cuda:0"
    layer = MoELayerGPU(cfg, inputs, dev, weights=args.weights)
    x = x_to_device(inputs, cfg, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    K = args.steps
    # the timed region: K whole-layer forwards, with HIP events between the
    # phases on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for s_ in range(K):
            e = ev[s_]
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
        wall = time.perf_counter() - t0
    names = ["route", "dispatch", "expert_ffn", "combine"]
    ph = {n: float(np.mean([ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(K)]))
          for i, n in enumerate(names)}
    dev_ms = float(np.mean([ev[s_][0].elapsed_time(ev[s_][4]) for s_ in range(K)]))
    ms_per_step = wall * 1e3 / K
    # the same K steps with nothing but the layer enqueued
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        layer.forward(x)
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / K
    print(f"[bench] {cfg.name}: timed {K} steps: {ms_per_step:.4f} ms/step "
          f"({ms_plain:.4f} without events)", file=sys.stderr, flush=True)

    kept = layer.buf.kept.cpu().numpy()
    dropped = int(layer.buf.dropped.cpu()[0])
    work = algorithmic_work(cfg, kept, dropped, args.weights)

    # memory-bound phases in isolation, after flushing the Infinity Cache by
    # reading 1 GiB (a read leaves clean lines behind: a write-based flush
    # would leave dirty lines whose write-back the timed phase would pay)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # fp32 sum: no conversion pass
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def cold(fn):
        ts = []
        for _ in range(args.iso_reps):
            torch.sum(flush, dim=0, out=sink)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    iso = {"route": cold(lambda: layer.route(x)), "dispatch": cold(lambda: layer.dispatch_aux(x)),
           "combine": cold(layer.combine)}
    # the unfused dispatch that copies the kept rows into x_disp [E, C, H]
    copy_layer_buf = torch.empty((cfg.E, layer.C, cfg.H), dtype=layer.tdtype, device=dev)
    from mixture_experts_layer_08_amd import ops
    b = layer.buf

    def copy_dispatch():
        ops.moe_dispatch_aux(x, b.topk_idx, b.probs, cfg.E, layer.C, cfg.alpha, ws=b.ws,
                             x_disp=copy_layer_buf, slot=b.slot, slot_token=b.slot_token,
                             kept=b.kept, dropped=b.dropped, counts=b.counts, f=b.f, p=b.p,
                             l_aux=b.l_aux, copy=True)
    iso["dispatch_copy"] = cold(copy_dispatch)
    del flush, sink, copy_layer_buf
    layer.forward(x)        # leave buffers consistent
    torch.cuda.synchronize()

    gemm_ms = ph["expert_ffn"]
    achieved_tflops = work["ffn_flop"] / (gemm_ms * 1e-3) / 1e12
    phases = {}
    for n, key in (("route", "route_bytes"), ("dispatch", "dispatch_bytes"),
                   ("combine", "combine_bytes")):
        gbs = work[key] / (ph[n] * 1e-3) / 1e9
        g2 = work[key] / (iso[n] * 1e-3) / 1e9
        phases[n] = {"ms": round(ph[n], 5), "bytes": work[key], "GB/s": round(gbs, 1),
                     "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "ms_cold": round(iso[n], 5),
                     "GB/s_cold": round(g2, 1), "hbm_frac_cold": round(g2 / PEAK_HBM_GBS, 4)}
    phases["dispatch"]["note"] = ("index-only dispatch of the fused-gather layer (maps and aux "
                                  "statistics, no row copy): a latency, not an HBM stream")
    gcp = work["copy_dispatch_bytes"] / (iso["dispatch_copy"] * 1e-3) / 1e9
    phases["dispatch_copy"] = {"ms_cold": round(iso["dispatch_copy"], 5),
                               "bytes": work["copy_dispatch_bytes"], "GB/s_cold": round(gcp, 1),
                               "hbm_frac_cold": round(gcp / PEAK_HBM_GBS, 4),
                               "note": "dispatch with the row copy into [E, C, H] (x read once, "
                                       "kept rows written), timed alone after a cache flush"}
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
              ", then down product; both launches, timed together inside the timed region)")
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
    rec = {
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_no_events": round(ms_plain, 5),
        "dtype": cfg.dtype,
        "config": {"workload": workload_name(cfg, args.weights),
                   "expert_weights": args.weights,
                   "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E,
                   "top_k": cfg.k, "capacity_factor": cfg.cf,
                   "capacity": layer.C, "kept_rows": work["n_kept"], "dropped": dropped,
                   "path": "route, dispatch (row maps) with aux statistics, gather-fused expert "
                           "products, combine"},
        "roofline": roofline,
        "phases": phases,
        "device_ms_per_step": round(dev_ms, 5),
        "gpu_clock": clk.summary(),
    }
    if args.weights == "bf16" and not args.no_fused_combine:
        rec["fused_combine"] = bench_fused_combine(cfg, inputs, dev, args,
                                                   ph["expert_ffn"] + ph["combine"])
    if args.graph:
        rec["graph"] = bench_graph(cfg, inputs, dev, args, ms_plain)
    if args.backward:
        rec["backward"] = bench_backward(cfg, inputs, dev, args)
    if args.shared:
        rec["shared_expert"] = bench_shared(cfg, dev, args)
    del layer, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if with_cpu:
        print(f"[bench] {cfg.name}: timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, inputs, args.cpu_seconds)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs the layer on one GPU; --gpus {args.gpus} is not "
              "supported (the layer has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch

    also = [int(c) for c in args.also.split(",") if c.strip()] if args.also else []
    also = [c for c in also if c != args.config]
    head = run_workload(args.config, args, not args.no_cpu_baseline)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    subs = {}
    for c in also:
        subs[str(c)] = run_workload(c, args, not args.no_cpu_baseline)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
    }
    for key in ("config", "roofline", "cpu_baseline", "phases", "ms_per_step_no_events",
                "device_ms_per_step", "gpu_clock", "backward", "shared_expert"):
        if key in head:
            out[key] = head[key]
    if subs:
        out["workloads"] = subs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
