"""CPU oracle for 8-bit expert weights: the e4m3 float format, per-channel
quantisation and dequantisation, in plain numpy.

TEST INFRASTRUCTURE ONLY, like the rest of the oracle: imported by the test
suite and the benchmark's CPU leg, never by the product path; it shares no
code with the HIP library.

Source: [P4] long-context page (2kiu.com/news/5130654) section 3 stores the
expert weights in 8 bits and turns them back into 16-bit floats with a
scale, and insists that the scale be computed per expert and per dimension
(one global scale costs accuracy); [P1] section 5.2 and [P5] section 5.1
name low-bit weights for inference.

Readings (the page's code is int8 with a constant scale):
  * the 8-bit code is the OCP float8 e4m3 format ("e4m3fn": 1 sign bit,
    4 exponent bits with bias 7, 3 mantissa bits, no infinities, the one
    NaN pattern S.1111.111, largest finite 448, subnormals m * 2^-9);
  * one fp32 scale per expert and per output column n of W [K, N]:
    s = max_k |W[k, n]| / 448 (s = 1 for an all-zero column), so the column's
    largest weight maps to 448;
  * code = the e4m3 value nearest to the fp32 quotient W / s (both the
    division and the comparison in float32 arithmetic, as the GPU does it),
    ties to the even code, magnitudes past 448 saturating to 448;
  * the dequantised weight is decode(code) * s, exactly (in float64).
The codes are stored transposed, [E, N, K] (each output column's K codes
contiguous), the scales as [E, N].
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

E4M3_MAX = 448.0


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """float64 value of each e4m3 code (NaN for the NaN patterns)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes 0x00 .. 0x7e, in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode_e4m3(_POS_CODES)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code to each float32 value (ties to the even code,
    magnitudes past 448 saturate to 448; NaN maps to the NaN code).  The
    magnitude is placed in the sorted table of the 127 non-negative finite
    values and the nearer of its two neighbours taken."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = np.abs(a - _POS_VALUES[lo])
    dhi = np.abs(_POS_VALUES[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = _POS_CODES[pick]
    code = np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_weight(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """w [E, K, N] (float32 values) -> codes [E, N, K] uint8, scales [E, N]
    float32 ([P4] section 3: a scale per expert and per dimension)."""
    w = np.asarray(w, dtype=np.float32)
    absmax = np.max(np.abs(w), axis=1)                        # [E, N]
    scale = np.where(absmax > 0, absmax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (w / scale[:, None, :]).astype(np.float32)            # float32 division
    codes = encode_e4m3(q)                                    # [E, K, N]
    return np.ascontiguousarray(codes.transpose(0, 2, 1)), scale


def dequantize_weight(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [E, N, K], scales [E, N] -> W [E, K, N] float64 (exact)."""
    vals = decode_e4m3(codes)                                 # [E, N, K]
    w = vals * np.asarray(scale, dtype=np.float64)[:, :, None]
    return np.ascontiguousarray(w.transpose(0, 2, 1))


# the expert weights each activation quantises: name -> (K, N) orientation
# of the stored [E, K, N] tensor
_WEIGHTS = {"swiglu": ("w_gate", "w_up", "w_down"), "gelu": ("w1", "w2")}


def quantize_inputs(inputs: Dict[str, np.ndarray], act: str) -> Dict[str, np.ndarray]:
    """Codes and scales of every routed expert weight: '<name>_q' [E, N, K]
    and '<name>_s' [E, N]."""
    out = {}
    for name in _WEIGHTS[act]:
        w = inputs[name]
        w32 = (w.astype(np.uint32) << np.uint32(16)).view(np.float32) if w.dtype == np.uint16 \
            else np.asarray(w, dtype=np.float32)
        out[name + "_q"], out[name + "_s"] = quantize_weight(w32)
    return out


def dequantized_inputs(inputs: Dict[str, np.ndarray], q: Dict[str, np.ndarray],
                       act: str) -> Dict[str, np.ndarray]:
    """The layer's inputs with every routed expert weight replaced by its
    dequantised value (float64): the layer the 8-bit weights compute."""
    out = dict(inputs)
    for name in _WEIGHTS[act]:
        out[name] = dequantize_weight(q[name + "_q"], q[name + "_s"])
    return out
