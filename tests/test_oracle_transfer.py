"""Pins of the oracle's window-masked transfer (oracle/transfer.py).

* The SWA mask it moves equals the set of positions that keep an SWA entry
  in the dual-pool simulator after eviction (MiMo page, sec. 2.1: transfers
  go by the SWA mask) -- a second, independent derivation of the same set.
* Byte counts against the closed form min(L, W - 1) * Hkv * d * 4 per SWA
  layer and L * Hkv * d * 4 per Full layer.
* The V format conversion (bf16 -> fp16, round to nearest even) against an
  fp16 encoder written from the IEEE 754 binary16 definition, including
  subnormal results and exact ties.
* FP8 pages: byte counts against the closed form (2 code bytes per element
  plus 8 scale bytes per (token, head)); the packed codes times their scales
  give back every moved input within the e4m3 rounding bound (half a unit
  of the 3-bit fraction, or half the subnormal step 2^-9 of the tile's
  scale), K from K and V from V, in sequence and position order.
"""
import math
import random

import numpy as np
import pytest

from oracle import transfer as T
from oracle.pool import PoolSim


@pytest.mark.parametrize("seed", range(6))
def test_swa_mask_is_the_resident_set_after_eviction(seed):
    rnd = random.Random(seed)
    W = rnd.choice([1, 2, 16, 128])
    C = 16 * (-(-(W + 40) // 16))
    S = 4
    sim = PoolSim(W, C, S, 64, S * 64, list(range(S * 64)), list(range(S * C // 16)))
    for _ in range(30):
        b = rnd.randrange(S)
        n = rnd.randint(0, 40)
        if sim.length[b] + n > 64 * 16:
            continue
        sim.alloc([b], [n])
        sim.evict([b])
        for q in range(S):
            resident = [p for p in range(sim.length[q])
                        if sim.full_slot(q, p) in sim.map]
            assert resident == list(T.transfer_positions(T.SWA, sim.length[q], W))
            assert list(T.transfer_positions(T.FULL, sim.length[q], W)) == \
                list(range(sim.length[q]))


def test_byte_counts_closed_form():
    lens = [0, 1, 5, 127, 128, 129, 4096, 32768]
    W, hkv, d = 128, 8, 128
    assert T.transfer_counts(T.SWA, lens, W) == [min(L, W - 1) for L in lens]
    assert T.transfer_bytes(T.SWA, lens, W, hkv, d) == sum(min(L, 127) for L in lens) * 4096
    assert T.transfer_bytes(T.FULL, lens, W, hkv, d) == sum(lens) * 4096
    # window 1: the query is its own window, nothing cached moves
    assert T.transfer_counts(T.SWA, lens, 1) == [0] * len(lens)


def _fp16_bits(x: float) -> int:
    """IEEE 754 binary16 encoding of a finite float, round to nearest even,
    written from the format's definition (1 sign, 5 exponent bits with bias
    15, 10 fraction bits; subnormals below 2^-14)."""
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    m, e = math.frexp(a)          # a = m * 2^e, 0.5 <= m < 1
    exp = e - 1                   # a = (2m) * 2^exp, 1 <= 2m < 2
    if exp < -14:                 # subnormal: units of 2^-24
        units = a / 2.0 ** -24
    else:
        units = (2 * m) * 2 ** 10  # significand in units of 2^-10, 1024..2047
    lo = math.floor(units)
    frac = units - lo
    q = lo + (1 if frac > 0.5 or (frac == 0.5 and lo % 2 == 1) else 0)
    if exp < -14:
        return sign | q            # q == 1024 rolls into the smallest normal
    if q == 2048:                  # rounding carried into the next binade
        q, exp = 1024, exp + 1
    if exp > 15:
        raise OverflowError
    return sign | ((exp + 15) << 10) | (q - 1024)


def _bf16_bits(x: float) -> int:
    return int(np.array([x], np.float32).view(np.uint32)[0] >> 16)


def test_v_conversion_matches_binary16_definition():
    rnd = random.Random(5)
    vals = [0.0, -0.0, 1.0, -2.5, 65280.0, 2.0 ** -14, 2.0 ** -15, 2.0 ** -24, 3 * 2.0 ** -25,
            2.0 ** -25, 1.0 + 2.0 ** -10, 1.0 + 2.0 ** -11]
    vals += [rnd.gauss(0, 1) for _ in range(300)] + [rnd.gauss(0, 1) * 1e-5 for _ in range(300)]
    bits = np.array([_bf16_bits(v) for v in vals], np.uint16)   # bf16 truncation of the draw
    k = bits.reshape(-1, 1, 1)
    hk, hv = T.host_image(T.FULL, 128, [(k, k)])
    assert np.array_equal(hk.reshape(-1), bits)
    for b, got in zip(bits, hv.reshape(-1)):
        x = float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])
        assert int(got) == _fp16_bits(x), (hex(int(b)), x)


def test_host_image_packs_windows_in_order():
    rng = np.random.default_rng(0)

    def draw(n):  # bf16 bit patterns of N(0, 1) values
        x = rng.standard_normal((n, 2, 4)).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    a, b = draw(10), draw(3)
    hk, _ = T.host_image(T.SWA, 4, [(a, a), (b, b)])
    assert np.array_equal(hk, np.concatenate([a[7:10], b[0:3]]))
    hk, _ = T.host_image(T.FULL, 4, [(a, a), (b, b)])
    assert np.array_equal(hk, np.concatenate([a, b]))


def test_fp8_byte_counts_closed_form():
    lens = [0, 1, 5, 127, 128, 129, 4096]
    W, hkv = 128, 8
    for d in (64, 128):
        per_tok = hkv * d * 2 + hkv * 8
        assert T.transfer_bytes_fp8(T.SWA, lens, W, hkv, d) == \
            sum(min(L, 127) for L in lens) * per_tok
        assert T.transfer_bytes_fp8(T.FULL, lens, W, hkv, d) == sum(lens) * per_tok


def test_host_image_fp8_packs_windows_in_order():
    rng = np.random.default_rng(3)
    lens, W, hkv, d = [10, 3, 0, 25], 4, 2, 16
    ks = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    vs = [(3 * rng.standard_normal((L, hkv, d))).astype(np.float32) for L in lens]
    for kind in (T.FULL, T.SWA):
        ck, cv, sk, sv = T.host_image_fp8(kind, W, zip(ks, vs))
        sel = [T.transfer_positions(kind, L, W) for L in lens]
        want_k = np.concatenate([k[r.start:r.stop] for k, r in zip(ks, sel)])
        want_v = np.concatenate([v[r.start:r.stop] for v, r in zip(vs, sel)])
        n = sum(len(r) for r in sel)
        assert ck.shape == cv.shape == (n, hkv, d) and sk.shape == sv.shape == (n, hkv)
        for codes, scale, want in ((ck, sk, want_k), (cv, sv, want_v)):
            # e4m3 value of each code: sign, 4-bit exponent (bias 7), 3-bit
            # fraction; exponent field 0 is subnormal, units of 2^-9
            c = codes.astype(np.int64)
            e, f = (c >> 3) & 15, c & 7
            mag = np.where(e == 0, f * 2.0 ** -9, (1 + f / 8) * 2.0 ** (e - 7))
            got = np.where(c & 0x80, -mag, mag) * scale[..., None].astype(np.float64)
            bound = np.abs(want) * 2.0 ** -4 + scale[..., None] * 2.0 ** -10
            assert np.all(np.abs(got - want) <= bound * (1 + 1e-6) + 1e-30), kind
            # the largest element of each row maps to the largest code
            assert np.all(np.max(mag, axis=-1) == 448.0), kind
