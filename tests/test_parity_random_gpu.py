"""GPU parity on seeded random configurations: layer kind, head dim, GQA
group, KV heads, window, chunk, ring slack, lengths, softmax scale and output
type are drawn per case; each case runs a chunked prefill of every sequence
and then multi-row decode steps (1-4 rows per sequence, ragged) with eviction
after each, and compares every output row with the fp64 oracle and every
valid length with its definition.  32 more cases run over FP8 pages, against
the oracle on the dequantized K/V."""
import random

import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
from oracle import attention as OA

from harness import TOL, SeqData, Setup, chunked_prefill, dev, make_seqs, oracle_rows

pytestmark = pytest.mark.gpu

CASES = 128


def _draw(case, base=7000):
    rnd = random.Random(base + case)
    c = dict(
        kind=rnd.choice([H.SWA, H.FULL]),
        d=rnd.choice([64, 128]),
        g=rnd.choice([1, 2, 4, 8]),
        hkv=rnd.choice([1, 2, 3]),
        W=rnd.choice([1, 2, 5, 16, 33, 64, 127, 128, 200]),
        chunk=rnd.choice([1, 7, 16, 31, 64, 100, 128, 257]),
        slack=rnd.choice([0, 0, 16, 48]),
        lens=[rnd.randint(1, 520) for _ in range(rnd.randint(1, 4))],
        scale=rnd.choice([0.0, 0.0, 0.05, 0.2]),
        out=rnd.choice([torch.float32, torch.float32, torch.float16]),
        steps=rnd.randint(1, 3),
        seed=100 + case,
    )
    c["rows"] = [[rnd.randint(1, 4) for _ in c["lens"]] for _ in range(c["steps"])]
    return c


def _tau(scale, d):
    return None if scale == 0.0 else scale


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration(gpu, case):
    _run(_draw(case), case, fp8=False)


@pytest.mark.parametrize("case", range(32))
def test_random_configuration_fp8_pages(gpu, case):
    """The same scenarios over FP8 pages (the appends quantize, prefill and
    decode read codes and scales), against the oracle on the dequantized
    K/V."""
    _run(_draw(case, base=7200), case, fp8=True)


def _run(c, case, fp8):
    kind, d, hkv, W = c["kind"], c["d"], c["hkv"], c["W"]
    hq = c["g"] * hkv
    lens, B = c["lens"], len(c["lens"])
    grow = [sum(r[b] for r in c["rows"]) for b in range(B)]
    total = [L + k for L, k in zip(lens, grow)]
    print(f"case {case}: fp8 {fp8} {c}", flush=True)
    seqs = make_seqs(total, hq, hkv, d, c["seed"])
    # the ring holds the W - 1 resident positions plus the largest append
    C = -(-(W - 1 + max(c["chunk"], 4)) // 16) * 16 + c["slack"]
    maxp = max(total) // 16 + 2
    st = Setup(kind, W, C, B, maxp, B * maxp + 3, hkv, d, c["seed"], fp8=fp8)
    tau = _tau(c["scale"], d)

    # chunked prefill of the first lens[b] positions
    pre = [SeqData(s.q[:L], s.k[:L], s.v[:L]) for s, L in zip(seqs, lens)]
    outs, vlens, _ = chunked_prefill(st, pre, c["chunk"], hq, scale=c["scale"],
                                     out_dtype=c["out"])
    for b, s in enumerate(pre):
        got = outs[b].double().numpy()
        exp = oracle_rows(s, list(range(lens[b])), kind, W, tau, fp8)
        assert np.all(np.isfinite(got)), f"prefill: non-finite output in sequence {b}"
        err = float(np.max(np.abs(got - exp)))
        assert err < TOL, f"prefill sequence {b}: max-abs error {err:.3e}"
        assert vlens[b].tolist() == [OA.valid_length(p, kind, W) for p in range(lens[b])]

    # multi-row decode steps, eviction after each
    ids = list(range(B))
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    cur = list(lens)
    for t, n in enumerate(c["rows"]):
        H.hswa_pool_alloc(st.pool, ids, n)
        pos = [list(range(cur[b], cur[b] + n[b])) for b in range(B)]
        flat = [(b, p) for b in range(B) for p in pos[b]]
        q = torch.stack([seqs[b].q[p] for b, p in flat]).to(dev())
        kn = torch.stack([seqs[b].k[p] for b, p in flat]).to(dev())
        vn = torch.stack([seqs[b].v[p] for b, p in flat]).to(dev())
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        T = len(flat)
        maxlen = max(cur[b] + n[b] for b in range(B))
        nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen, total_q=T)
        ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
        out = torch.full((T, hq, d), float("nan"), dtype=c["out"], device=dev())
        vl = torch.full((T,), -1, dtype=torch.int32, device=dev())
        H.hswa_decode(kind, W, q, kn, vn, sid, maxlen, st.view, st.kc, st.vc, out, ws, vl,
                      scale=c["scale"], cu_q=cu, max_q_len=max(n), **st.scales())
        got = out.cpu().double().numpy()
        o = 0
        for b in range(B):
            exp = oracle_rows(seqs[b], pos[b], kind, W, tau, fp8)
            err = float(np.max(np.abs(got[o:o + n[b]] - exp)))
            assert err < TOL, f"decode step {t} sequence {b}: max-abs error {err:.3e}"
            o += n[b]
        assert vl.cpu().tolist() == [OA.valid_length(p, kind, W) for _, p in flat]
        ev, cnt = H.hswa_pool_evict(st.pool, ids)
        for b in range(B):
            L = cur[b] + n[b]
            st.poison_ring_positions(b, list(range(L - W + 1 - cnt[b], L - W + 1)))
            cur[b] = L


@pytest.mark.parametrize("case", range(8))
def test_random_large_configuration(gpu, case):
    """Longer random prefills (up to 6,000 tokens, chunks up to 2,048, up to
    64 query heads) checked on sampled rows: every chunk's first and last
    rows, the window edges, and 200 random rows per sequence."""
    rnd = random.Random(7500 + case)
    kind = rnd.choice([H.SWA, H.FULL])
    d, g, hkv = rnd.choice([64, 128]), rnd.choice([1, 2, 4, 8]), rnd.choice([1, 2, 8])
    W = rnd.choice([16, 100, 128, 129, 256])
    chunk = rnd.choice([256, 1000, 2048])
    lens = [rnd.randint(1, 6000) for _ in range(rnd.randint(1, 3))]
    hq = g * hkv
    print(f"case {case}: kind {kind} d {d} g {g} hkv {hkv} W {W} chunk {chunk} lens {lens}",
          flush=True)
    seqs = make_seqs(lens, hq, hkv, d, 500 + case)
    C = -(-(W - 1 + chunk) // 16) * 16
    maxp = max(lens) // 16 + 2
    st = Setup(kind, W, C, len(lens), maxp, len(lens) * maxp + 3, hkv, d, 500 + case)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    for b, s in enumerate(seqs):
        L = lens[b]
        pick = {0, L - 1, min(L - 1, W - 1), min(L - 1, W)}
        for a in range(0, L, chunk):
            pick |= {a, min(L - 1, a + chunk - 1)}
        pick |= set(rnd.randrange(L) for _ in range(200))
        pos = sorted(pick)
        got = outs[b][pos].double().numpy()
        assert np.all(np.isfinite(got)), f"non-finite output in sequence {b}"
        err = float(np.max(np.abs(got - oracle_rows(s, pos, kind, W))))
        assert err < TOL, f"sequence {b}: max-abs error {err:.3e}"
        assert vlens[b][pos].tolist() == [OA.valid_length(p, kind, W) for p in pos]
