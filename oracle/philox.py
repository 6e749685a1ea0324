"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY: this file belongs to the CPU oracle.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import it.

Definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11, section 3.2 and table 2):
  state      four 32-bit counter words (c0, c1, c2, c3), two key words (k0, k1);
  one round  (hi0, lo0) = 0xD2511F53 * c0 as a 64-bit product split in halves,
             (hi1, lo1) = 0xCD9E8D57 * c2 likewise, then
             (c0, c1, c2, c3) <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
  key bump   between rounds k0 += 0x9E3779B9, k1 += 0xBB67AE85 (mod 2^32);
  output     the counter after 10 rounds.

The long-context page keys its Gumbel noise to uniform draws
(2kiu.com/news/5130654, section 2, where u comes from rand_like); the draw for
(token t, expert e) is word 0 of Philox4x32-10 with counter (t, e, 0, 0) and
key (seed mod 2^32, seed >> 32), mapped to u = (word + 0.5) * 2^-32 in (0, 1).
"""
from __future__ import annotations

import numpy as np

_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over uint32-valued arrays (broadcastable)."""
    m = np.uint64(_MASK)
    c0 = np.asarray(c0, dtype=np.uint64) & m
    c1 = np.asarray(c1, dtype=np.uint64) & m
    c2 = np.asarray(c2, dtype=np.uint64) & m
    c3 = np.asarray(c3, dtype=np.uint64) & m
    k0 = np.asarray(k0, dtype=np.uint64) & m
    k1 = np.asarray(k1, dtype=np.uint64) & m
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(_W0)) & m
            k1 = (k1 + np.uint64(_W1)) & m
        p0 = np.uint64(_M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return (c0.astype(np.uint32), c1.astype(np.uint32),
            c2.astype(np.uint32), c3.astype(np.uint32))


def gumbel_words(seed: int, T: int, E: int) -> np.ndarray:
    """uint32 word 0 of Philox4x32-10 at counter (t, e, 0, 0), shape [T, E]."""
    t = np.arange(T, dtype=np.uint64)[:, None]
    e = np.arange(E, dtype=np.uint64)[None, :]
    k0 = seed & _MASK
    k1 = (seed >> 32) & _MASK
    w0, _, _, _ = philox4x32_10(t, e, 0, 0, k0, k1)
    return np.broadcast_to(w0, (T, E)).copy()


def gumbel_uniform(seed: int, T: int, E: int) -> np.ndarray:
    """u[t, e] = (word + 0.5) * 2^-32, exactly representable in float64."""
    return (gumbel_words(seed, T, E).astype(np.float64) + 0.5) * 2.0 ** -32


def gumbel_noise(seed: int, T: int, E: int) -> np.ndarray:
    """g = -log(-log u): standard Gumbel noise in float64."""
    u = gumbel_uniform(seed, T, E)
    return -np.log(-np.log(u))
