"""FP8 KV quantization: per-(token, head) tiles of e4m3 codes with fp32 scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the Baidu Day0 article on hybrid linear + sparse attention models,
"Layered quantization", point 2: the KV cache is stored in FP8, quantized per
token, per head and per tile of 128 elements, each tile with its own scale.
The vLLM MiniMax M3 post runs the MI355X serving stack with an fp8 KV cache.

Readings taken where the pages leave a step open:

* The FP8 format is OCP e4m3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3
  fraction bits, subnormals below 2^-6 in steps of 2^-9, largest finite 448,
  code 0x7F / 0xFF NaN, no infinities.
* A tile of a row x (the min(128, d) elements of one token and head) is
  quantized with amax = max |x|, scale = amax / 448 and inv = 448 / amax, both
  fp32 divisions rounded to nearest; each element becomes the e4m3 code of the
  fp32 product x * inv, rounded to nearest with ties to an even fraction and
  saturated at 448.  amax = 0 gives scale 0, inv 0, all codes 0.  The
  decisions (division, product, rounding) are made in fp32 on both sides.
* Dequantized value = e4m3 value of the code * scale; the attention oracle
  runs in fp64 on these values.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of an e4m3 code from the format's definition."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_scalar(y: float) -> int:
    """Nearest e4m3 code to y by direct search over the finite codes (ties to
    the code with an even fraction), saturating at +-448."""
    y = float(y)
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = min(abs(y), E4M3_MAX)
    best, best_d = 0, math.inf
    for c in range(0x7F):                  # non-negative finite codes 0x00..0x7E
        d = abs(E4M3_TABLE[c] - a)
        if d < best_d or (d == best_d and (c & 1) == 0):
            best, best_d = c, d
    return sign | best


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Vectorised e4m3 encoding of fp32 values (same rule as the scalar
    search): exponent from frexp, fraction rounded half to even."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    sub = a < 2.0 ** -6
    code = np.zeros(a.shape, dtype=np.int64)
    # subnormal range: units of 2^-9 (q = 8 is the smallest normal, code 0x08)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    m, e = np.frexp(a[~sub])               # a = m * 2^e, 0.5 <= m < 1
    q = np.rint((2 * m - 1) * 8).astype(np.int64)   # 3-bit fraction, ties to even
    field = (e - 1 + 7).astype(np.int64)
    code[~sub] = field * 8 + q             # q == 8 carries into the exponent
    return (sign | code).astype(np.uint8)


def quantize_rows(x) -> tuple:
    """Quantize rows x [..., n] (n <= 128, one tile per row) given as fp32
    values (bf16 inputs convert exactly).  Returns (codes uint8 [..., n],
    scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] > 128:
        raise ValueError("one tile holds at most 128 elements")
    amax = np.max(np.abs(x), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """fp64 values code * scale (exact: a 4-bit significand times an fp32)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)] * \
        np.asarray(scale, dtype=np.float64)[..., None]
