"""Pins of the oracle's FP8 KV quantization (oracle/fp8.py).

* The e4m3 value table against facts of the format: 448 the largest finite
  value, 2^-6 the smallest normal, 2^-9 the smallest subnormal, 1 and 2 at
  their exponent fields, NaN only at 0x7F / 0xFF, finite codes strictly
  increasing.
* The vectorised encoder against a brute-force nearest-code search over the
  table on exact ties, neighbours of every tie, subnormals, zeros and values
  beyond 448 (saturation), plus encode(value(c)) == c for every finite code.
* Row quantization: the largest element maps to +-448, the dequantized
  error is within half an e4m3 step times the scale, all-zero rows give
  zero codes and scale.
"""
import math

import numpy as np
import pytest

from oracle import fp8 as F


def test_value_table_facts():
    assert F.e4m3_value(0x7E) == 448.0 and F.e4m3_value(0xFE) == -448.0
    assert F.e4m3_value(0x08) == 2.0 ** -6
    assert F.e4m3_value(0x01) == 2.0 ** -9
    assert F.e4m3_value(0x38) == 1.0 and F.e4m3_value(0x40) == 2.0
    assert F.e4m3_value(0xB8) == -1.0
    assert F.e4m3_value(0x00) == 0.0 and math.copysign(1, F.e4m3_value(0x80)) < 0
    nans = [c for c in range(256) if math.isnan(F.e4m3_value(c))]
    assert nans == [0x7F, 0xFF]
    pos = [F.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))


def _probe_values():
    pos = [F.e4m3_value(c) for c in range(0x7F)]
    vals = []
    for a, b in zip(pos, pos[1:]):
        mid = (a + b) / 2                  # exact tie (fp32 represents it)
        vals += [mid, np.nextafter(np.float32(mid), np.float32(0)),
                 np.nextafter(np.float32(mid), np.float32(1e9)), a, b]
    rng = np.random.default_rng(0)
    vals += list(rng.standard_normal(2000) * 10.0 ** rng.uniform(-4, 3, 2000))
    vals += [0.0, -0.0, 447.9, 448.0, 455.9, 464.0, 500.0, 1e30, 2.0 ** -10, 2.0 ** -12]
    v = np.array(vals, dtype=np.float32)
    return np.concatenate([v, -v])


def test_vector_encoder_matches_nearest_code_search():
    v = _probe_values()
    got = F.e4m3_encode(v)
    exp = np.array([F.e4m3_encode_scalar(float(x)) for x in v], dtype=np.uint8)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(exp[i])) for i in bad[:5]]


def test_encode_of_every_finite_value_is_its_code():
    codes = [c for c in range(256) if not math.isnan(F.e4m3_value(c))]
    vals = np.array([F.e4m3_value(c) for c in codes], dtype=np.float32)
    assert F.e4m3_encode(vals).tolist() == codes


def test_quantize_rows_bounds():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((500, 128)) * 10.0 ** rng.uniform(-3, 2, (500, 1))).astype(np.float32)
    x = x.astype(np.float32)
    codes, scale = F.quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    top = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(F.E4M3_TABLE[codes[np.arange(500), top]]) == 448.0)
    deq = F.dequantize_rows(codes, scale)
    # half a step of the e4m3 grid at the element's magnitude, in scaled units
    y = np.abs(x.astype(np.float64)) / scale[:, None]
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 3))
    bound = 0.5 * step * scale[:, None] * (1 + 1e-6) + 1e-12
    assert np.all(np.abs(deq - x) <= bound)


def test_zero_row():
    codes, scale = F.quantize_rows(np.zeros((2, 64), np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)
    assert np.all(F.dequantize_rows(codes, scale) == 0)
