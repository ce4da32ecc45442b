"""GPU parity of chunked prefill over FP8 pages (Baidu Day0 hybrid-attention
article, Layered quantization, point 2: FP8 KV per token, head and
128-element tile; "MiMo-V2.5 Series Inference Full-Link Optimization" sec.
1.1, chunked prefill of SWA and Full layers).

``hswa_prefill_chunk`` with ``k_scale``/``v_scale`` quantizes each chunk's
K/V into the pages and attends over them.  Every output row is within 4e-3
of the fp64 oracle evaluated on the oracle's own dequantization of the same
bf16 rows (code value x scale).  Pools start with NaN codes (0x7F) and NaN
scales, and the ring slots of evicted positions are set back to NaN after
every chunk, so a read of a slot outside a row's keys shows up.  Cases: SWA
and Full layers, d 64 and 128, 1 to 8 query heads per KV head, chunk starts
on and off page boundaries, chunks of one row, a ring of one page, and 12
seeded random configurations.  Every finite e4m3 code also comes back
exactly through the prefill path.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle import fp8 as F8

from harness import TOL, dev, make_seqs

pytestmark = pytest.mark.gpu

# kind, window, head_dim, hq, hkv, sequence lengths, chunk, ring slots
CASES = [
    (H.SWA, 128, 128, 64, 8, [400, 177, 33], 128, 256),
    (H.SWA, 37, 128, 16, 2, [300, 129, 5], 50, 96),
    (H.SWA, 16, 64, 8, 8, [150, 64], 7, 32),
    (H.SWA, 5, 64, 2, 1, [70, 17], 1, 16),
    (H.SWA, 20, 128, 4, 4, [150], 33, 64),
    (H.FULL, 64, 128, 64, 8, [300, 150, 31], 100, 176),
    (H.FULL, 16, 64, 4, 2, [130, 77], 24, 48),
    (H.FULL, 16, 128, 2, 2, [97], 1, 32),
]


def _deq(x):
    """fp64 values the pages hold for bf16 rows [L, Hkv, d]."""
    codes, scale = F8.quantize_rows(x.float().numpy())
    return F8.dequantize_rows(codes, scale)


def _run(case, seed):
    kind, W, d, hq, hkv, lens, chunk, C = case
    B = len(lens)
    maxp = max(lens) // 16 + 2
    npages = B * maxp if kind == H.FULL else B * C // 16
    seqs = make_seqs(lens, hq, hkv, d, seed)
    free = synth.permutation(B * maxp, seed, 1)
    ring = synth.permutation(B * C // 16, seed, 2)
    pool = H.hswa_pool_create(W, C, B, maxp, B * maxp, free, ring, device=dev())
    view = H.hswa_pool_get_view(pool)
    kc, vc, ks, vs = H.kv_cache_alloc_fp8(npages, hkv, d, dev(), 0x7F)
    ring_pages = ring.reshape(B, C // 16)
    outs = [np.full((L, hq, d), np.nan) for L in lens]
    done = [0] * B
    while any(done[b] < lens[b] for b in range(B)):
        act = [b for b in range(B) if done[b] < lens[b]]
        n = [min(chunk, lens[b] - done[b]) for b in act]
        H.hswa_pool_alloc(pool, act, n)
        rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
        q = torch.cat([seqs[b].q[a:e] for b, a, e in rows]).to(dev())
        kn = torch.cat([seqs[b].k[a:e] for b, a, e in rows]).to(dev())
        vn = torch.cat([seqs[b].v[a:e] for b, a, e in rows]).to(dev())
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        sid = torch.tensor(act, dtype=torch.int32, device=dev())
        out = torch.full((q.shape[0], hq, d), float("nan"), dtype=torch.float32, device=dev())
        H.hswa_prefill_chunk(kind, W, q, kn, vn, sid, cu, max(n), view, kc, vc, out,
                             k_scale=ks, v_scale=vs)
        _, cnt = H.hswa_pool_evict(pool, act)
        torch.cuda.synchronize()
        o = out.cpu().double().numpy()
        r = 0
        for (b, a, e), c in zip(rows, cnt):
            outs[b][a:e] = o[r:r + e - a]
            r += e - a
            if kind == H.SWA and c > 0:
                # NaN into the ring slots of the positions that just left
                pos = np.arange(e - W + 1 - c, e - W + 1) % C
                pg = torch.as_tensor(ring_pages[b][pos // 16].astype(np.int64), device=dev())
                off = torch.as_tensor((pos % 16).astype(np.int64), device=dev())
                kc[pg, :, off, :] = 0x7F
                vc[pg, :, :, off] = 0x7F
                ks[pg, :, off] = float("nan")
                vs[pg, :, off] = float("nan")
        for b, k in zip(act, n):
            done[b] += k
    worst = 0.0
    for b, s in enumerate(seqs):
        L = lens[b]
        want = OA.attend(synth.to_f64(s.q), list(range(L)), _deq(s.k), _deq(s.v), kind, W)
        assert np.all(np.isfinite(outs[b])), f"sequence {b}: non-finite output"
        worst = max(worst, float(np.max(np.abs(outs[b] - want))))
    assert worst < TOL, f"max-abs error {worst:.3e}"
    return worst


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fp8_chunked_prefill_matches_oracle(gpu, case):
    _run(CASES[case], 960 + case)


@pytest.mark.parametrize("kind", [H.FULL, H.SWA])
def test_prefill_reads_every_e4m3_code_exactly(gpu, kind):
    """Every finite e4m3 code, through the prefill path, comes back as its
    exact value.  One stored key's V codes are all 254 finite codes (two KV
    heads x 128 dims) with V scale 1 (code x scale is then exact in fp16);
    its K codes are 448 and the new row's Q is all ones, so its score exceeds
    the new row's own key (K = 0) by thousands: weight 1 against 0.  The
    output is that key's V, code by code, bit for bit."""
    from test_fp8_decode_gpu import Fp8Pool
    hkv, d, W = 2, 128, 128
    P = Fp8Pool([1], hkv, d, W, 62)
    codes = np.arange(256, dtype=np.uint8).reshape(hkv, d)
    codes[(codes & 0x7F) == 0x7F] &= 0x80     # the two NaN codes -> +-0
    kc, vc, ks, vs = P.bufs(kind)
    s = P.slot(kind, 0, 0)
    pg, off = s // 16, s % 16
    kc[pg, :, off, :] = 0x7E
    vc[pg, :, :, off] = torch.as_tensor(codes, device=dev())
    ks[pg, :, off] = 1.0
    vs[pg, :, off] = 1.0
    H.hswa_pool_alloc(P.pool, [0], [1])
    q = torch.ones((1, hkv, d), dtype=torch.bfloat16, device=dev())
    zero = torch.zeros((1, hkv, d), dtype=torch.bfloat16, device=dev())
    cu = torch.tensor([0, 1], dtype=torch.int32, device=dev())
    out = torch.full((1, hkv, d), float("nan"), dtype=torch.float32, device=dev())
    H.hswa_prefill_chunk(kind, W, q, zero, zero, P.sid, cu, 1, P.view, kc, vc, out,
                         k_scale=ks, v_scale=vs)
    want = F8.E4M3_TABLE[codes].astype(np.float32)
    got = out.cpu().numpy()[0]
    assert np.array_equal(got.view(np.uint32) & 0x7FFFFFFF, want.view(np.uint32) & 0x7FFFFFFF) \
        and np.array_equal(got, want), np.argwhere(got != want)[:5]


def _random_case(seed):
    import random
    rnd = random.Random(7000 + seed)
    kind = rnd.choice([H.SWA, H.FULL])
    d = rnd.choice([64, 128])
    hkv = rnd.choice([1, 2, 4])
    g = rnd.choice([1, 2, 4, 8])
    W = rnd.choice([1, 3, 16, 31, 64, 128, 200])
    chunk = rnd.choice([1, 5, 16, 33, 64, 100])
    C = 16 * (-(-(W - 1 + chunk) // 16) + rnd.choice([0, 0, 1]))
    lens = [rnd.randint(1, 260) for _ in range(rnd.randint(1, 3))]
    return (kind, W, d, g * hkv, hkv, lens, chunk, C)


@pytest.mark.parametrize("seed", range(12))
def test_fp8_chunked_prefill_random_configuration(gpu, seed):
    """Seeded random shapes: SWA or Full, d, KV heads 1-4, GQA 1-8, windows
    1-200, chunks 1-100 rows, rings from the smallest that holds W - 1 +
    chunk (down to one page), 1-3 sequences of 1-260 tokens."""
    _run(_random_case(seed), 980 + seed)
