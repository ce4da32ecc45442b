"""Pins of the fp64 attention oracle and the closed forms to facts outside it.

Each test checks the oracle against something it does not share code with:
a library routine (torch's scaled_dot_product_attention in fp64 on the CPU,
given an explicit boolean band mask), brute force with math.fsum, special
cases with exact answers, and the figures of the MiMo-V2.5 inference page
(sections 1.1, 1.2 and 2.1) stored in tests/golden/page_facts.json.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import closed_forms as CF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa_reference(q, k, v, kind, window, scale=None):
    """torch SDPA in fp64 with an explicit band mask and expanded KV heads."""
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, n, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    i = torch.arange(n).unsqueeze(1) + (L - n)
    j = torch.arange(L).unsqueeze(0)
    mask = j <= i
    if kind == A.SWA:
        mask = mask & (j > i - window)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("kind,window", [(A.FULL, 0), (A.SWA, 1), (A.SWA, 5),
                                         (A.SWA, 16), (A.SWA, 300)])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 16), (4, 4, 8), (6, 1, 32)])
def test_matches_torch_sdpa_fp64(kind, window, hq, hkv, d):
    L = 97
    q = _rand((L, hq, d), 1)
    k = _rand((L, hkv, d), 2)
    v = _rand((L, hkv, d), 3)
    ours = A.attend_sequence(q, k, v, kind, window)
    ref = _sdpa_reference(q, k, v, kind, window)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_explicit_scale_matches_sdpa():
    L, hq, hkv, d = 40, 4, 2, 16
    q, k, v = _rand((L, hq, d), 4), _rand((L, hkv, d), 5), _rand((L, hkv, d), 6)
    ours = A.attend_sequence(q, k, v, A.SWA, 7, scale=0.3)
    ref = _sdpa_reference(q, k, v, A.SWA, 7, scale=0.3)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_chunk_rows_match_sdpa_suffix():
    """Rows of a later chunk (positions 60..96) equal the same rows of the
    whole-sequence reference."""
    L, hq, hkv, d = 97, 8, 2, 16
    q, k, v = _rand((L, hq, d), 7), _rand((L, hkv, d), 8), _rand((L, hkv, d), 9)
    ours = A.attend(q[60:], range(60, L), k, v, A.SWA, 16)
    ref = _sdpa_reference(q[60:], k, v, A.SWA, 16)
    assert np.max(np.abs(ours - ref)) < 1e-12


@pytest.mark.parametrize("window", [1, 2, 5, 16, 64])
def test_brute_force_fsum(window):
    """Pure-Python loops with exact-sum accumulation on a tiny case."""
    L, hq, hkv, d = 23, 4, 2, 4
    q, k, v = _rand((L, hq, d), 10), _rand((L, hkv, d), 11), _rand((L, hkv, d), 12)
    g = hq // hkv
    tau = 1.0 / math.sqrt(d)
    ours = A.attend_sequence(q, k, v, A.SWA, window)
    for i in range(L):
        keys = [j for j in range(L) if j <= i and i - j < window]
        for h in range(hq):
            kv = h // g
            s = [tau * math.fsum(q[i, h, t] * k[j, kv, t] for t in range(d)) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            for t in range(d):
                o = math.fsum(w[a] * v[j, kv, t] for a, j in enumerate(keys)) / z
                assert abs(o - ours[i, h, t]) < 1e-13


def test_window_one_returns_own_value():
    L, hq, hkv, d = 30, 8, 2, 16
    q, k, v = _rand((L, hq, d), 13), _rand((L, hkv, d), 14), _rand((L, hkv, d), 15)
    o = A.attend_sequence(q, k, v, A.SWA, 1)
    g = hq // hkv
    for h in range(hq):
        assert np.array_equal(o[:, h], v[:, h // g])


def test_window_at_least_length_is_full():
    L, hq, hkv, d = 50, 4, 2, 8
    q, k, v = _rand((L, hq, d), 16), _rand((L, hkv, d), 17), _rand((L, hkv, d), 18)
    full = A.attend_sequence(q, k, v, A.FULL, 0)
    for w in (L, L + 1, 10 * L):
        assert np.array_equal(A.attend_sequence(q, k, v, A.SWA, w), full)


@pytest.mark.parametrize("kind,window", [(A.FULL, 0), (A.SWA, 6)])
def test_zero_query_gives_window_mean(kind, window):
    """q = 0 makes every score equal, so the output is the mean of V over
    the window; compare with exact sums."""
    L, hq, hkv, d = 40, 4, 2, 8
    q = np.zeros((L, hq, d))
    k, v = _rand((L, hkv, d), 19), _rand((L, hkv, d), 20)
    o = A.attend_sequence(q, k, v, kind, window)
    g = hq // hkv
    for i in range(L):
        lo = 0 if kind == A.FULL else max(0, i - window + 1)
        for h in range(hq):
            for t in range(d):
                mean = math.fsum(v[lo:i + 1, h // g, t]) / (i + 1 - lo)
                assert abs(o[i, h, t] - mean) < 1e-14


def test_one_hot_values_expose_weights():
    """V = one-hot by key position makes o[i, h, j] the softmax weight of
    key j: zero outside the window, summing to 1, with ratios exp(s_j - s_k)."""
    L, hq, hkv, d, W = 24, 2, 1, 32, 5
    q, k = _rand((L, hq, d), 21), _rand((L, hkv, d), 22)
    v = np.zeros((L, hkv, d))
    for j in range(L):
        v[j, 0, j] = 1.0
    o = A.attend_sequence(q, k, v, A.SWA, W)
    tau = 1.0 / math.sqrt(d)
    for i in range(L):
        lo = max(0, i - W + 1)
        for h in range(hq):
            p = o[i, h]
            assert np.all(p[:lo] == 0.0) and np.all(p[i + 1:] == 0.0)
            assert abs(math.fsum(p[lo:i + 1]) - 1.0) < 1e-14
            s = [tau * math.fsum(q[i, h, t] * k[j, 0, t] for t in range(d))
                 for j in range(lo, i + 1)]
            for a in range(1, len(s)):
                assert abs(p[lo + a] / p[lo] - math.exp(s[a] - s[0])) < 1e-11 * math.exp(abs(s[a] - s[0]))


def test_out_of_window_keys_do_not_matter():
    """NaN-poisoning every key/value outside each query's window leaves SWA
    outputs bitwise unchanged (checked one query at a time)."""
    L, hq, hkv, d, W = 60, 8, 2, 16, 9
    q, k, v = _rand((L, hq, d), 23), _rand((L, hkv, d), 24), _rand((L, hkv, d), 25)
    base = A.attend_sequence(q, k, v, A.SWA, W)
    for i in (0, 3, 8, 9, 30, 59):
        lo = max(0, i - W + 1)
        kp, vp = k.copy(), v.copy()
        kp[:lo] = np.nan
        vp[:lo] = np.nan
        kp[i + 1:] = np.nan
        vp[i + 1:] = np.nan
        o = A.attend(q[i:i + 1], [i], kp, vp, A.SWA, W)
        assert np.array_equal(o[0], base[i])


def test_gqa_groups_are_contiguous():
    """Changing KV head 1 changes exactly query heads g..2g-1."""
    L, hq, hkv, d = 20, 6, 3, 8
    q, k, v = _rand((L, hq, d), 26), _rand((L, hkv, d), 27), _rand((L, hkv, d), 28)
    base = A.attend_sequence(q, k, v, A.FULL, 0)
    v2 = v.copy()
    v2[:, 1] += 1.0
    o = A.attend_sequence(q, k, v2, A.FULL, 0)
    changed = [h for h in range(hq) if not np.array_equal(o[:, h], base[:, h])]
    assert changed == [2, 3]
    # adding a constant to V shifts the convex combination by that constant
    assert np.max(np.abs(o[:, 2:4] - base[:, 2:4] - 1.0)) < 1e-13


@pytest.mark.parametrize("window", [1, 2, 7, 128])
def test_valid_length_and_pair_counts(window):
    for n in list(range(0, 40)) + [127, 128, 129, 300]:
        lens = [A.valid_length(i, A.SWA, window) for i in range(n)]
        assert sum(lens) == CF.pairs_swa(n, window)
        assert sum(A.valid_length(i, A.FULL, 0) for i in range(n)) == CF.pairs_full(n)
        # brute-force mask count
        if n <= 40:
            cnt = sum(1 for i in range(n) for j in range(n) if j <= i and i - j < window)
            assert cnt == CF.pairs_swa(n, window)


def test_page_facts_one_seventh_and_seven_x():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["facts"]
    nl = facts["num_layers"]["value"]
    nf = facts["num_full_layers"]["value"]
    ns = facts["num_swa_layers"]["value"]
    W = facts["window"]["value"]
    assert nf + ns == nl
    assert ns * facts["swa_layer_share"]["value"][1] == nl * facts["swa_layer_share"]["value"][0]
    lim = facts["compute_ratio_approx"]["value"][0] / facts["compute_ratio_approx"]["value"][1]
    # the page's ratios are long-sequence statements: within 3% at 64k tokens,
    # and converging to exactly 1/7 (and 7x) as the sequence grows
    for n in (65536, 262144):
        assert abs(CF.stack_pair_ratio(n, ns, nf, W) - lim) / lim < 0.03
        assert abs(CF.stack_kv_ratio(n, ns, nf, W) - lim) / lim < 0.03
        assert abs(CF.capacity_gain(n, ns, nf, W) - facts["capacity_gain_approx"]["value"]) < 0.2
    big = 10 ** 9
    assert abs(CF.stack_pair_ratio(big, ns, nf, W) - lim) < 1e-6
    assert abs(CF.stack_kv_ratio(big, ns, nf, W) - lim) < 1e-6
    assert abs(CF.capacity_gain(big, ns, nf, W) - 7.0) < 1e-5
    # ratios decrease monotonically towards the limit
    rs = [CF.stack_pair_ratio(n, ns, nf, W) for n in (1024, 4096, 65536, 1 << 20)]
    assert all(a > b for a, b in zip(rs, rs[1:])) and rs[-1] > lim


def test_short_sequences_have_no_saving():
    """Below the window every layer is effectively Full (ratio 1)."""
    for n in (1, 17, 128):
        assert CF.stack_pair_ratio(n, 60, 10, 128) == 1.0
        assert CF.stack_kv_ratio(n, 60, 10, 128) == 1.0


def test_flop_count():
    # one query, one key, d=2, one head: QK^T is 2 MACs and PV is 2 MACs = 8 flops
    assert CF.attention_flops(1, 1, 2) == 8
    assert CF.attention_flops(CF.pairs_swa(1024, 128), 8, 64) == 4 * 64 * 8 * 122944


def test_rejects_bad_arguments():
    q = np.zeros((2, 4, 8))
    k = np.zeros((2, 3, 8))
    with pytest.raises(ValueError):
        A.attend_sequence(q, k, k, A.FULL, 0)
    with pytest.raises(ValueError):
        A.key_range(3, A.SWA, 0)
    with pytest.raises(ValueError):
        A.attend(np.zeros((1, 2, 8)), [5], np.zeros((3, 1, 8)), np.zeros((3, 1, 8)), A.FULL, 0)
