"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
from __future__ import annotations

import sys

import numpy as np
import torch


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_round_np(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (through torch, nearest-even) -> float64."""
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy() \
        .astype(np.float64)


def to_dev(a: np.ndarray, dtype: torch.dtype, dev="cuda:0") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(dev)


def assert_rows_close(got: np.ndarray, want: np.ndarray, rel_rms: float, what: str,
                      abs_floor: float = 0.0, stored_bf16: bool = False) -> float:
    """max |got - want| <= rel_rms * RMS(want row) (+ abs_floor), row by row.

    stored_bf16: `got` is a layer output stored in bf16 (rounded once, to
    nearest even, after the fp32 computation).  That final rounding moves a
    value by at most the bf16 unit roundoff 2^-8 of the stored value, which
    for an element several times the row RMS is itself close to 2e-2 RMS; it
    is added to the bound, which then bounds the computation before the
    output's own rounding.  Returns the worst err / RMS(row) (rounding
    included)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    err = np.abs(got - want)
    bound = rel_rms * rms + abs_floor
    if stored_bf16:
        bound = bound + 2.0 ** -8 * np.abs(got)
    bad = err > bound
    worst = float(np.max(err / np.maximum(rms, 1e-300))) if want.size else 0.0
    if bad.any():
        r = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at "
                             f"{tuple(r)} got {got[tuple(r)]} want {want[tuple(r)]} "
                             f"(rms {rms[tuple(r[:-1])][0]}), worst err/rms {worst:.3e}")
    return worst


def assert_rel(got, want, rtol: float, what: str, atol: float = 0.0) -> None:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = err > rtol * np.abs(want) + atol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} out of tolerance; first at {tuple(i)} "
                             f"got {got[tuple(i)]} want {want[tuple(i)]}")
