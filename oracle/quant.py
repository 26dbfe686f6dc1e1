"""Plain CPU definition of the fp8 row quantisation of the fp8 attention path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path never imports it and shares no code with it.

Reduced-bitwidth attention after reordering is the subject of "PAROAttention:
Pattern-Aware ReOrdering for Efficient Sparse and Quantized Attention in
Visual Generation Models" (abstract, INT8/INT4); the fp8 path uses the OCP
FP8 E4M3 format (4 exponent bits with bias 7, 3 mantissa bits, largest
finite value 448, no infinities). Each row gets one power-of-two scale:
2^e with e the smallest integer for which max|x| 2^-e <= 448, but no less
than -127, the smallest E8M0 scale (e = 0 for an all-zero row), stored as the
E8M0 code e + 127; the row divided by its scale
is rounded to nearest even E4M3. torch's float8_e4m3fn cast serves as the
rounding step (a library primitive); the scale is computed here from its
definition with exact power-of-two arithmetic.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["E4M3_MAX", "row_exponent", "quantize_rows", "dequantize_rows", "e4m3_decode"]

E4M3_MAX = 448.0


def row_exponent(amax: float) -> int:
    """Smallest integer e >= -127 with amax * 2^-e <= 448 (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = 0
    while amax * 2.0 ** (-e) > E4M3_MAX:    # too big: larger scale
        e += 1
    while e > -127 and amax * 2.0 ** (-(e - 1)) <= E4M3_MAX:  # a smaller scale still fits
        e -= 1
    return e


def quantize_rows(x: np.ndarray):
    """x: float32 [n, d] (bf16 values are exact in float32) ->
    (codes uint8 [n, d], scales uint8 [n] = e + 127)."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(n, dtype=np.uint8)
    for r in range(n):
        e = row_exponent(np.abs(x[r]).max())
        y = np.ldexp(x[r], -e).astype(np.float32)  # exact: a power-of-two scaling
        codes[r] = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scales[r] = e + 127
    return codes, scales


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 bytes -> float64, from the format definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (ex - 7.0))
    val = np.where((ex == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)[:, None]
