"""moe_dispatch_aux_noalloc (the library's static device workspace in place
of a workspace argument) against moe_dispatch_aux on the same inputs: two
calls in a row on one GPU, the second smaller, every output bitwise equal
(the same kernels run on the same inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_layer_08_amd import ops
from mixture_experts_layer_08_amd._lib import lib

from parity_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((T, E)) + np.linspace(1.5, 0.0, E)   # uneven: some experts overflow
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    pr = np.exp(keys - keys.max(axis=1, keepdims=True))
    pr = (pr / pr.sum(axis=1, keepdims=True)).astype(np.float32)
    x = rng.standard_normal((T, 256)).astype(np.float32)
    return (torch.from_numpy(x).to(torch.bfloat16).to(DEV), torch.from_numpy(idx).to(DEV),
            torch.from_numpy(pr).to(DEV))


NAMES = ("x_disp", "slot", "slot_token", "kept", "dropped", "counts", "f", "p", "l_aux")


def _compare(got, want, what, kept):
    for n, g, w in zip(NAMES, got, want):
        if n == "x_disp":
            assert (g is None) == (w is None), f"{what}: x_disp"
            for e, m in enumerate(kept if g is not None else []):
                assert torch.equal(g[e, :m], w[e, :m]), f"{what}: x_disp[{e}]"
            continue
        assert torch.equal(g, w), f"{what}: {n}"


@pytest.mark.parametrize("copy", [False, True], ids=["maps", "copy"])
def test_noalloc_matches_workspace_entry(copy):
    E, k, alpha = 16, 2, 0.01
    for i, (T, cf) in enumerate(((9000, 1.0), (1234, 0.75))):   # the second call smaller
        C = ops.moe_capacity(T, k, E, cf)
        log(f"[noalloc] call {i + 1}: T={T} E={E} k={k} C={C} copy={copy}")
        x, idx, pr = _routing(T, E, k, 100 + i)
        want = ops.moe_dispatch_aux(x, idx, pr, E, C, alpha, copy=copy)
        # outputs preallocated, so the no-allocation call allocates nothing at all
        outs = dict(x_disp=torch.empty((E, C, 256), dtype=torch.bfloat16, device=DEV) if copy
                    else None,
                    slot=torch.empty((T, k), dtype=torch.int32, device=DEV),
                    slot_token=torch.empty((E, C), dtype=torch.int32, device=DEV),
                    kept=torch.empty(E, dtype=torch.int32, device=DEV),
                    dropped=torch.empty(1, dtype=torch.int32, device=DEV),
                    counts=torch.empty(E, dtype=torch.int32, device=DEV),
                    f=torch.empty(E, dtype=torch.float32, device=DEV),
                    p=torch.empty(E, dtype=torch.float32, device=DEV),
                    l_aux=torch.empty(1, dtype=torch.float32, device=DEV))
        got = ops.moe_dispatch_aux_noalloc(x, idx, pr, E, C, alpha, copy=copy, **outs)
        torch.cuda.synchronize()
        kept = want[3].cpu().numpy().tolist()
        assert int(want[4].cpu()[0]) > 0, "the case should drop some assignments"
        _compare(got, want, f"call {i + 1}", kept)

