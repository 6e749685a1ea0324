"""Seeded synthetic workloads for the sparse-MoE FFN forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it without sharing any method code.

Workload shapes follow the pages:
  * hidden 2048 / intermediate 4096 / 8 experts / top-2 / alpha 0.01 / init
    std 0.02 is the configuration dataclass of the LLaMA4-MoE guide
    (dpshk.com/news/5809432, section 2.1);
  * the flattened [8, 4096, 16384] expert pool with per-expert biases is the
    "Flatten the Experts" layout (discosf.com/news/5228035, section 2.1) with
    the biased GELU expert of the minimal MoELayer (dpshk.com/news/6005940,
    section 3.1);
  * 32 experts at sequence 32768 with Gumbel hard top-k and temperature
    1 + 1e-4 * seq_len is the long-context router (2kiu.com/news/5130654,
    sections 2 and 5.2).

Draw recipe (fixed so that a run is reproducible anywhere):
  generator  numpy.random.Generator(PCG64(seed)), seed = 1000 + config id;
  order      x, W_r, then for each expert e in turn: W_gate[e] (W1[e]),
             W_up[e] (SwiGLU only), W_down[e] (W2[e]), b1[e], b2[e] (GELU only);
  values     standard_normal(shape, float32) * std with std 1 for x, 0.02
             for weights, 0.01 for biases;
  storage    rounded once to bfloat16 with round-to-nearest-even (kept as the
             uint16 bit pattern), or left in float32 for fp32 workloads.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

ACT_SWIGLU = "swiglu"
ACT_GELU = "gelu"
ROUTE_SOFTMAX = "softmax"
ROUTE_GUMBEL = "gumbel"


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    dtype: str          # "bf16" or "f32"
    T: int              # tokens = batch * seq
    H: int              # hidden size
    I: int              # expert intermediate size
    E: int              # number of experts
    k: int              # experts per token
    cf: float           # capacity factor
    alpha: float = 0.01
    act: str = ACT_SWIGLU
    route: str = ROUTE_SOFTMAX
    router_bias0: float = 0.0   # bias added to expert 0's logit (0 = no bias)
    batch: int = 1
    seq: int = 0        # sequence length (sets the Gumbel temperature)
    seed: int = 0
    shared_I: int = 0   # intermediate size of the shared expert (0 = none)

    @property
    def seq_len(self) -> int:
        return self.seq if self.seq else self.T // self.batch

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# The five named workloads.  Config 2 is the one throughput is quoted on.
CONFIGS: Dict[int, MoEConfig] = {
    1: MoEConfig("tiny-fp32", "f32", T=64, H=128, I=256, E=4, k=2, cf=1.25,
                 batch=1, seq=64, seed=1001),
    2: MoEConfig("layer-bf16", "bf16", T=4096, H=2048, I=4096, E=8, k=2,
                 cf=1.25, batch=2, seq=2048, seed=1002),
    3: MoEConfig("skewed-bf16", "bf16", T=16384, H=2048, I=4096, E=8, k=2,
                 cf=1.0, router_bias0=2.0, batch=1, seq=16384, seed=1003),
    4: MoEConfig("wide-gelu-bf16", "bf16", T=8192, H=4096, I=16384, E=8, k=2,
                 cf=1.25, act=ACT_GELU, batch=1, seq=8192, seed=1004),
    5: MoEConfig("long-gumbel-bf16", "bf16", T=32768, H=2048, I=5632, E=32,
                 k=2, cf=1.25, route=ROUTE_GUMBEL, batch=1, seq=32768,
                 seed=1005),
    # Drop-free decode step: 64 sequences x 1 new token on the config-2 layer.
    # cf = E / k makes C = T, the most rows one expert can receive when a
    # token's k experts are distinct, so nothing is ever dropped.
    6: MoEConfig("decode-bf16", "bf16", T=64, H=2048, I=4096, E=8, k=2,
                 cf=4.0, batch=64, seq=1, seed=1006),
}


def drop_free(cfg: MoEConfig) -> MoEConfig:
    """The same workload with capacity C = T (cf = E / k): no drops."""
    return cfg.with_(cf=cfg.E / cfg.k)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(cfg: MoEConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of one layer call.

    Returns a dict with x [T,H], w_r [H,E], b_r [E] (float32, or None),
    and per-expert stacks: SwiGLU -> w_gate [E,H,I], w_up [E,H,I],
    w_down [E,I,H]; GELU -> w1 [E,H,I], w2 [E,I,H], b1 [E,I], b2 [E,H].
    With cfg.shared_I > 0, the shared expert's weights follow under the same
    names prefixed "shared_", as one-expert stacks of intermediate size
    shared_I (drawn after everything else, so the routed inputs do not
    depend on it).  bf16 arrays are uint16 bit patterns; f32 arrays are
    float32.
    """
    seed = cfg.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed))
    dt = cfg.dtype
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    out: Dict[str, np.ndarray] = {}
    out["x"] = _store(g.standard_normal((T, H), dtype=np.float32), dt)
    out["w_r"] = _store(g.standard_normal((H, E), dtype=np.float32) * np.float32(0.02), dt)
    if cfg.router_bias0 != 0.0:
        b = np.zeros(E, dtype=np.float32)
        b[0] = cfg.router_bias0
        out["b_r"] = b
    else:
        out["b_r"] = None
    sw = np.float32(0.02)
    sb = np.float32(0.01)
    if cfg.act == ACT_SWIGLU:
        shp_in, shp_out = (E, H, I), (E, I, H)
        edt = np.uint16 if dt == "bf16" else np.float32
        wg = np.empty(shp_in, edt)
        wu = np.empty(shp_in, edt)
        wd = np.empty(shp_out, edt)
        for e in range(E):
            wg[e] = _store(g.standard_normal((H, I), dtype=np.float32) * sw, dt)
            wu[e] = _store(g.standard_normal((H, I), dtype=np.float32) * sw, dt)
            wd[e] = _store(g.standard_normal((I, H), dtype=np.float32) * sw, dt)
        out.update(w_gate=wg, w_up=wu, w_down=wd)
    elif cfg.act == ACT_GELU:
        edt = np.uint16 if dt == "bf16" else np.float32
        w1 = np.empty((E, H, I), edt)
        w2 = np.empty((E, I, H), edt)
        b1 = np.empty((E, I), edt)
        b2 = np.empty((E, H), edt)
        for e in range(E):
            w1[e] = _store(g.standard_normal((H, I), dtype=np.float32) * sw, dt)
            w2[e] = _store(g.standard_normal((I, H), dtype=np.float32) * sw, dt)
            b1[e] = _store(g.standard_normal((I,), dtype=np.float32) * sb, dt)
            b2[e] = _store(g.standard_normal((H,), dtype=np.float32) * sb, dt)
        out.update(w1=w1, w2=w2, b1=b1, b2=b2)
    else:
        raise ValueError(f"unknown activation {cfg.act!r}")
    Is = cfg.shared_I
    if Is:
        edt = np.uint16 if dt == "bf16" else np.float32
        if cfg.act == ACT_SWIGLU:
            for name, shp in (("w_gate", (H, Is)), ("w_up", (H, Is)), ("w_down", (Is, H))):
                a = np.empty((1,) + shp, edt)
                a[0] = _store(g.standard_normal(shp, dtype=np.float32) * sw, dt)
                out["shared_" + name] = a
        else:
            for name, shp, sd in (("w1", (H, Is), sw), ("w2", (Is, H), sw), ("b1", (Is,), sb),
                                  ("b2", (H,), sb)):
                a = np.empty((1,) + shp, edt)
                a[0] = _store(g.standard_normal(shp, dtype=np.float32) * sd, dt)
                out["shared_" + name] = a
    return out


def to_f64(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact widening of a stored array (bf16 bits or float32) to float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)

