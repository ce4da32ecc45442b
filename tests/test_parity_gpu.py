"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar (fixed by the workload statement): slot maps, eviction sets and valid
window lengths bit-exact; attention outputs from bf16 inputs within max-abs
4e-3 of the oracle.
"""
import random

import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle.pool import NoSpace, PoolSim

from harness import TOL, SeqData, Setup, chunked_prefill, dev, make_seqs, oracle_rows

pytestmark = pytest.mark.gpu


def _check_seq(outs, vlens, seqs, kind, W, scale=None, sample=None):
    worst = 0.0
    for b, s in enumerate(seqs):
        L = s.q.shape[0]
        pos = list(range(L)) if sample is None else sorted(set(p for p in sample(L)))
        exp = oracle_rows(s, pos, kind, W, scale)
        got = outs[b][pos].double().numpy()
        assert np.all(np.isfinite(got)), f"non-finite output in sequence {b}"
        err = float(np.max(np.abs(got - exp)))
        worst = max(worst, err)
        assert err < TOL, f"sequence {b}: max-abs error {err:.3e}"
        vl = vlens[b][pos].numpy()
        want = np.array([OA.valid_length(p, kind, W) for p in pos])
        assert np.array_equal(vl, want)
    return worst


# ---------------------------------------------------------------------------
# Pool tables on the device are bit-exact against the oracle simulator


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pool_device_tables_match_oracle(gpu, seed):
    rnd = random.Random(seed)
    W, C, S, maxp, npages = [(4, 16, 3, 6, 12), (128, 384, 4, 40, 100), (17, 48, 5, 9, 30)][seed]
    free = synth.permutation(npages, seed, 1)
    ring = synth.permutation(S * C // 16, seed, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    t = pool.tables
    for step in range(80):
        ids = rnd.sample(range(S), rnd.randint(1, S))
        r = rnd.random()
        if r < 0.45:
            n = [rnd.choice([0, 1, 3, 16, 40, rnd.randint(0, C)]) for _ in ids]
            try:
                exp = sim.alloc(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_alloc(pool, ids, n)
                continue
            got = H.hswa_pool_alloc(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.8:
            exp = sim.evict(ids)
            got = H.hswa_pool_evict(pool, ids)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.92:
            n = [rnd.randint(0, 3 * W) for _ in ids]
            try:
                exp = sim.import_context(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_import(pool, ids, n)
                continue
            got = H.hswa_pool_import(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        else:
            sim.release(ids)
            H.hswa_pool_release(pool, ids)
        torch.cuda.synchronize()
        assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
        assert t["fpt"].cpu().view(S, maxp).tolist() == sim.fpt_table()
        assert t["map"].cpu().tolist() == sim.map_table()
        assert t["rpt"].cpu().view(S, C // 16).tolist() == sim.rpt_table()


def test_pool_tables_with_lopsided_page_lists(gpu):
    """One sequence with thousands of pages next to many with one: the
    table updates go out in several launches (page lists are padded per
    launch), and every table still matches the oracle simulator."""
    W, C, S = 64, 128, 48
    maxp, npages = 400, 600
    free = synth.permutation(npages, 9, 1)
    ring = synth.permutation(S * C // 16, 9, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    t = pool.tables
    ids = list(range(S))
    n = [6000] + [1] * (S - 2) + [200]
    assert [list(x) for x in H.hswa_pool_import(pool, ids, n)] == \
        [list(x) for x in sim.import_context(ids, n)]
    for step in range(3):
        k = [3] * S
        k[0] = 60
        assert [list(x) for x in H.hswa_pool_alloc(pool, ids, k)] == \
            [list(x) for x in sim.alloc(ids, k)]
        assert [list(x) for x in H.hswa_pool_evict(pool, ids)] == \
            [list(x) for x in sim.evict(ids)]
    torch.cuda.synchronize()
    assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
    assert t["fpt"].cpu().view(S, maxp).tolist() == sim.fpt_table()
    assert t["map"].cpu().tolist() == sim.map_table()


# ---------------------------------------------------------------------------
# SWA single-chunk prefill then decode steps (one sequence, d = 64, g = 4)


def test_swa_single_chunk_then_decode(gpu):
    wl = synth.C1
    L0, steps = wl.prefill_len, wl.decode_steps
    total = L0 + steps
    hq, hkv, d, W = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window
    seqs = make_seqs([total], hq, hkv, d, wl.seed)
    C = W + L0
    # contiguous slot tables: identity page orders
    st = Setup(H.SWA, W, C, 1, total // 16 + 2, total // 16 + 2, hkv, d, wl.seed)
    H.hswa_pool_destroy(st.pool)
    st.pool = H.hswa_pool_create(W, C, 1, total // 16 + 2, total // 16 + 2,
                                 np.arange(total // 16 + 2), np.arange(C // 16), device=dev())
    st.view = H.hswa_pool_get_view(st.pool)
    st.ring_pages = np.arange(C // 16).reshape(1, -1)
    pre = [SeqData(seqs[0].q[:L0], seqs[0].k[:L0], seqs[0].v[:L0])]
    outs, vlens, _ = chunked_prefill(st, pre, L0, hq)
    _check_seq(outs, vlens, pre, OA.SWA, W)
    sid = torch.zeros(1, dtype=torch.int32, device=dev())
    for t in range(steps):
        pos = L0 + t
        H.hswa_pool_alloc(st.pool, [0], [1])
        q = seqs[0].q[pos:pos + 1].to(dev())
        kn = seqs[0].k[pos:pos + 1].to(dev())
        vn = seqs[0].v[pos:pos + 1].to(dev())
        out = torch.full((1, hq, d), float("nan"), dtype=torch.float32, device=dev())
        vl = torch.full((1,), -1, dtype=torch.int32, device=dev())
        ws_bytes = H.hswa_decode_workspace_bytes(H.SWA, W, 1, hq, hkv, d, pos + 1)
        assert ws_bytes == 0
        H.hswa_decode(H.SWA, W, q, kn, vn, sid, pos + 1, st.view, st.kc, st.vc, out, None, vl)
        ev, cnt = H.hswa_pool_evict(st.pool, [0])
        exp = oracle_rows(seqs[0], [pos], OA.SWA, W)
        err = float(np.max(np.abs(out.cpu().double().numpy() - exp)))
        assert err < TOL, f"decode step {t}: {err:.3e}"
        assert int(vl.item()) == W
        assert list(cnt) == [1]


# ---------------------------------------------------------------------------
# Chunked prefill, several sequences, ragged tails, permuted pages, NaN-poisoned
# evicted and unwritten slots


@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_chunked_prefill_ragged(gpu, kind):
    hq, hkv, d, W, chunk = 64, 8, 128, 128, 256
    lens = [700, 333, 1029, 1]
    seqs = make_seqs(lens, hq, hkv, d, 11)
    maxp = max(lens) // 16 + 2
    st = Setup(kind, W, W + chunk, len(lens), maxp, len(lens) * maxp + 5, hkv, d, 11)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    _check_seq(outs, vlens, seqs, kind, W)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_gqa_and_head_dims(gpu, g, d, kind):
    hkv = 2
    hq = g * hkv
    W, chunk = 48, 96
    lens = [200, 77]
    seqs = make_seqs(lens, hq, hkv, d, 100 + g + d)
    maxp = max(lens) // 16 + 2
    st = Setup(kind, W, W + chunk, 2, maxp, 2 * maxp, hkv, d, 5)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    _check_seq(outs, vlens, seqs, kind, W)


def test_window_one_returns_value(gpu):
    hq, hkv, d = 8, 2, 64
    seqs = make_seqs([90], hq, hkv, d, 21)
    st = Setup(H.SWA, 1, 64, 1, 8, 8, hkv, d, 21)
    outs, vlens, _ = chunked_prefill(st, seqs, 32, hq)
    v = seqs[0].v.float()
    for h in range(hq):
        # one key of weight 1: the value itself, up to fp32 rounding of the
        # normaliser and the fp16 subnormal range of the PV operand
        vv = v[:, h // (hq // hkv)]
        err = (outs[0][:, h] - vv).abs() - 1e-6 * vv.abs()
        assert err.max().item() <= 2.0 ** -24
    assert torch.all(vlens[0] == 1)


def test_large_window_equals_full_bitwise(gpu):
    """A SWA layer whose window covers the sequence reads the same logical
    keys as a Full layer; the reduction order depends on logical positions
    only, so the outputs agree bit for bit."""
    hq, hkv, d = 16, 2, 128
    L = 300
    seqs = make_seqs([L], hq, hkv, d, 31)
    a = Setup(H.SWA, 512, 512 + 64, 1, 20, 20, hkv, d, 31)
    oa, va, _ = chunked_prefill(a, seqs, 64, hq)
    b = Setup(H.FULL, 512, 512 + 64, 1, 20, 20, hkv, d, 77)
    ob, vb, _ = chunked_prefill(b, seqs, 64, hq)
    assert torch.equal(oa[0], ob[0])
    assert torch.equal(va[0], vb[0])
    _check_seq(oa, va, seqs, OA.FULL, 0)


@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_page_permutation_bitwise(gpu, kind):
    hq, hkv, d, W = 64, 8, 128, 128
    seqs = make_seqs([450, 260], hq, hkv, d, 41)
    res = []
    for perm_seed in (1, 2):
        st = Setup(kind, W, W + 128, 2, 40, 80, hkv, d, perm_seed)
        outs, vlens, _ = chunked_prefill(st, seqs, 128, hq)
        res.append(outs)
    for x, y in zip(*res):
        assert torch.equal(x, y)


@pytest.mark.parametrize("chunk", [1, 16, 100])
def test_chunk_sizes_agree_with_oracle(gpu, chunk):
    hq, hkv, d, W = 16, 2, 64, 32
    seqs = make_seqs([130, 45], hq, hkv, d, 51)
    st = Setup(H.SWA, W, W + chunk + 16 - (W + chunk) % 16, 2, 20, 40, hkv, d, 51)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    _check_seq(outs, vlens, seqs, OA.SWA, W)


def test_empty_batch_is_noop(gpu):
    st = Setup(H.SWA, 16, 32, 1, 4, 4, 2, 64, 1)
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=dev())
    cu = torch.zeros(1, dtype=torch.int32, device=dev())
    sid = torch.empty(0, dtype=torch.int32, device=dev())
    out = torch.empty((0, 8, 64), dtype=torch.float32, device=dev())
    H.hswa_prefill_chunk(H.SWA, 16, q, None, None, sid, cu, 0, st.view, st.kc, st.vc, out)
    H.hswa_decode(H.SWA, 16, q, None, None, sid, 1, st.view, st.kc, st.vc, out)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Decode over a Full and a SWA layer (mixed batch), contexts restored with
# hswa_pool_import, new token appended each step, eviction each step


def _decode_scenario(ctxs, steps, hq, hkv, d, W, seed, C=None):
    B = len(ctxs)
    total = [c + steps for c in ctxs]
    seqs = make_seqs(total, hq, hkv, d, seed)
    C = C or W
    maxp = max(total) // 16 + 2
    nfull = B * maxp + 8
    full = Setup(H.FULL, W, C, B, maxp, nfull, hkv, d, seed)
    # the SWA layer shares the pool's tables; it only needs its own ring buffers
    skc, svc = H.kv_cache_alloc(B * C // 16, hkv, d, dev(), float("nan"))
    pool, view = full.pool, full.view
    ids = list(range(B))
    H.hswa_pool_import(pool, ids, ctxs)
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    # place the restored context: every position in the Full layer, the
    # in-window positions in the SWA ring
    cu = torch.tensor(np.concatenate([[0], np.cumsum(ctxs)]), dtype=torch.int32, device=dev())
    kf = torch.cat([s.k[:c] for s, c in zip(seqs, ctxs)]).to(dev())
    vf = torch.cat([s.v[:c] for s, c in zip(seqs, ctxs)]).to(dev())
    H.hswa_append_kv(H.FULL, kf, vf, sid, view, full.kc, full.vc, cu, max(ctxs))
    nw = [min(c, W - 1) for c in ctxs]
    cuw = torch.tensor(np.concatenate([[0], np.cumsum(nw)]), dtype=torch.int32, device=dev())
    ksw = torch.cat([s.k[c - k:c] for s, c, k in zip(seqs, ctxs, nw)]).to(dev())
    vsw = torch.cat([s.v[c - k:c] for s, c, k in zip(seqs, ctxs, nw)]).to(dev())
    H.hswa_append_kv(H.SWA, ksw, vsw, sid, view, skc, svc, cuw, max(nw))
    errs = []
    for t in range(steps):
        H.hswa_pool_alloc(pool, ids, [1] * B)
        pos = [c + t for c in ctxs]
        q = torch.stack([s.q[p] for s, p in zip(seqs, pos)]).to(dev())
        kn = torch.stack([s.k[p] for s, p in zip(seqs, pos)]).to(dev())
        vn = torch.stack([s.v[p] for s, p in zip(seqs, pos)]).to(dev())
        maxlen = max(pos) + 1
        for kind, kc, vc in ((H.FULL, full.kc, full.vc), (H.SWA, skc, svc)):
            out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=dev())
            vl = torch.full((B,), -1, dtype=torch.int32, device=dev())
            nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            H.hswa_decode(kind, W, q, kn, vn, sid, maxlen, view, kc, vc, out, ws, vl)
            got = out.cpu().double().numpy()
            for b in range(B):
                exp = oracle_rows(seqs[b], [pos[b]], kind, W)[0]
                err = float(np.max(np.abs(got[b] - exp)))
                errs.append(err)
                assert err < TOL, f"step {t} kind {kind} seq {b}: {err:.3e}"
            assert vl.cpu().tolist() == [OA.valid_length(p, kind, W) for p in pos]
        ev, cnt = H.hswa_pool_evict(pool, ids)
        assert list(cnt) == [1 if p + 1 >= W else 0 for p in pos]
    return max(errs)


def test_decode_mixed_full_and_swa(gpu):
    rng = np.random.default_rng(3)
    ctxs = [int(x) for x in rng.integers(1, 3000, size=12)] + [1, 127, 128, 129]
    _decode_scenario(ctxs, 4, 64, 8, 128, 128, 61)


def test_decode_long_context_splits(gpu):
    """Long contexts force the split-K path (several splits + merge)."""
    _decode_scenario([20000, 7000, 33], 2, 64, 8, 128, 128, 71, C=128 + 256)


def test_decode_small_heads_d64(gpu):
    _decode_scenario([1500, 90, 700], 3, 8, 2, 64, 128, 81)


def test_decode_many_sequences_work_queue(gpu):
    """600 sequences (the work-queue pre-pass scans 256 at a time) with
    contexts from 1 to 6,000 keys: 2 splits of 3,008 keys, the second
    empty for the shorter sequences, so the queue holds a mix of pieces of
    every length (and the bounds of a split: 3,007-3,009)."""
    rng = np.random.default_rng(17)
    ctxs = [int(x) for x in rng.integers(1, 6000, size=595)] + [1, 3007, 3008, 3009, 6000]
    _decode_scenario(ctxs, 2, 16, 2, 64, 64, 171)


def test_decode_skips_sequences_outside_the_pool(gpu):
    """A seq_ids entry outside [0, max_seqs) gets no work (its output rows
    and valid length stay as they were); the other sequences are exact,
    through the split-K work queue and without it."""
    hq, hkv, d, W = 16, 2, 64, 64
    ctxs = [5000, 3000, 40]
    seqs = make_seqs(ctxs, hq, hkv, d, 172)
    B = len(ctxs)
    maxp = max(ctxs) // 16 + 2
    st = Setup(H.FULL, W, W, B, maxp, B * maxp + 8, hkv, d, 172)
    ids = list(range(B))
    H.hswa_pool_import(st.pool, ids, ctxs)
    sid_all = torch.tensor(ids, dtype=torch.int32, device=dev())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(ctxs)]), dtype=torch.int32, device=dev())
    kf = torch.cat([s_.k[:c] for s_, c in zip(seqs, ctxs)]).to(dev())
    vf = torch.cat([s_.v[:c] for s_, c in zip(seqs, ctxs)]).to(dev())
    H.hswa_append_kv(H.FULL, kf, vf, sid_all, st.view, st.kc, st.vc, cu, max(ctxs))
    pos = [c - 1 for c in ctxs]
    q = torch.stack([s_.q[p_] for s_, p_ in zip(seqs, pos)]).to(dev())
    for bad in (B, -1, 1 << 20):
        sid = torch.tensor([0, bad, 2], dtype=torch.int32, device=dev())
        for maxlen in (max(ctxs), 64):   # split-K (work queue), and one split
            out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=dev())
            vl = torch.full((B,), -7, dtype=torch.int32, device=dev())
            nb = H.hswa_decode_workspace_bytes(H.FULL, W, B, hq, hkv, d, maxlen)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            H.hswa_decode(H.FULL, W, q, None, None, sid, maxlen, st.view, st.kc, st.vc, out, ws, vl)
            got = out.cpu().double().numpy()
            for b in (0, 2):
                exp = oracle_rows(seqs[b], [pos[b]], H.FULL, W)[0]
                assert float(np.max(np.abs(got[b] - exp))) < TOL
            assert np.isnan(got[1]).all()
            assert vl.cpu().tolist() == [ctxs[0], -7, ctxs[2]]


# ---------------------------------------------------------------------------
# One GPU's share of an 8-way head split: Hq = 8, Hkv = 1, d = 128


@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_prefill_one_kv_head_share(gpu, kind):
    hq, hkv, d, W, chunk = 8, 1, 128, 128, 256
    lens = [900, 37, 513]
    seqs = make_seqs(lens, hq, hkv, d, 91)
    maxp = max(lens) // 16 + 2
    st = Setup(kind, W, W + chunk, len(lens), maxp, len(lens) * maxp + 5, hkv, d, 91)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    _check_seq(outs, vlens, seqs, kind, W)


def test_decode_one_kv_head_share(gpu):
    _decode_scenario([20000, 4100, 129, 1], 2, 8, 1, 128, 128, 93, C=128 + 256)


# ---------------------------------------------------------------------------
# Evictions on a second stream, overlapping the append and attention


def test_evictions_on_a_second_stream(gpu):
    """Each chunk step's eviction runs on another stream right after the
    step's alloc, beside its append and attention, with no host wait inside
    the loop; the next alloc and the final table read wait for it.  The
    outputs equal the same chunked prefill with evictions on the launch
    stream bitwise, and the device tables equal the oracle simulator's."""
    W, C, hq, hkv, d, chunk = 32, 32 + 128, 8, 2, 64, 128
    lens = [300, 517, 90, 128]
    B = len(lens)
    seqs = make_seqs(lens, hq, hkv, d, seed=41)
    maxp, npages = max(lens) // 16 + 2, B * (max(lens) // 16 + 2)

    def run(side):
        st = Setup(H.SWA, W, C, B, maxp, npages, hkv, d, seed=41)
        main = torch.cuda.current_stream()
        sim = PoolSim(W, C, B, maxp, npages, synth.permutation(npages, 41, 1),
                      synth.permutation(B * C // 16, 41, 2))
        outs = [torch.empty((L, hq, d), dtype=torch.float32, device=dev()) for L in lens]
        vls = [torch.empty(L, dtype=torch.int32, device=dev()) for L in lens]
        done, evicted = [0] * B, None
        while True:
            act = [b for b in range(B) if done[b] < lens[b]]
            if not act:
                break
            n = [min(chunk, lens[b] - done[b]) for b in act]
            if evicted is not None:
                main.wait_event(evicted)
            got = H.hswa_pool_alloc(st.pool, act, n)
            exp = sim.alloc(act, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
            if side is not None:
                allocated = torch.cuda.Event()
                allocated.record(main)
                side.wait_event(allocated)
                got = H.hswa_pool_evict(st.pool, act, stream=side)
                evicted = torch.cuda.Event()
                evicted.record(side)
            rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
            q = torch.cat([seqs[b].q[a:e] for b, a, e in rows]).to(dev())
            kn = torch.cat([seqs[b].k[a:e] for b, a, e in rows]).to(dev())
            vn = torch.cat([seqs[b].v[a:e] for b, a, e in rows]).to(dev())
            cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32,
                              device=dev())
            sid = torch.tensor(act, dtype=torch.int32, device=dev())
            out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device=dev())
            vl = torch.empty(q.shape[0], dtype=torch.int32, device=dev())
            H.hswa_prefill_chunk(H.SWA, W, q, kn, vn, sid, cu, max(n), st.view, st.kc, st.vc,
                                 out, vl)
            if side is None:
                got = H.hswa_pool_evict(st.pool, act)
            exp = sim.evict(act)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
            o = 0
            for b, a, e in rows:
                outs[b][a:e].copy_(out[o:o + e - a])
                vls[b][a:e].copy_(vl[o:o + e - a])
                o += e - a
            for b, k in zip(act, n):
                done[b] += k
        if evicted is not None:
            main.wait_event(evicted)
        torch.cuda.synchronize()
        t = st.pool.tables
        assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
        assert t["fpt"].cpu().view(B, maxp).tolist() == sim.fpt_table()
        assert t["map"].cpu().tolist() == sim.map_table()
        return [x.cpu() for x in outs], [x.cpu() for x in vls]

    base, base_vl = run(None)
    side = torch.cuda.Stream()   # default priority
    overlapped, overlapped_vl = run(side)
    for b in range(B):
        assert torch.equal(base[b], overlapped[b]), f"sequence {b} differs"
        assert torch.equal(base_vl[b], overlapped_vl[b])
    _check_seq(overlapped, overlapped_vl, seqs, H.SWA, W)


# ---------------------------------------------------------------------------
# Row offsets that leave the row buffers: the sequence is skipped


def test_rows_beyond_total_q_are_skipped(gpu):
    """cu_q gives sequence 1 more rows than q / out hold: its append and
    attention are skipped (nothing read or written for it), while sequence
    0 is computed as usual.  Prefill, then a two-row decode."""
    hq, hkv, d, W, C = 8, 2, 64, 4, 32
    seqs = make_seqs([7, 12], hq, hkv, d, 53)
    st = Setup(H.SWA, W, C, 2, 4, 8, hkv, d, 53)
    s0, s1 = seqs
    sid = torch.tensor([0, 1], dtype=torch.int32, device=dev())

    # prefill: sequence 0 has rows [0, 5), sequence 1 claims [5, 12) of 10
    H.hswa_pool_alloc(st.pool, [0, 1], [5, 7])
    q = torch.cat([s0.q[:5], s1.q[:5]]).to(dev())
    kn = torch.cat([s0.k[:5], s1.k[:5]]).to(dev())
    vn = torch.cat([s0.v[:5], s1.v[:5]]).to(dev())
    cu = torch.tensor([0, 5, 12], dtype=torch.int32, device=dev())
    out = torch.full((10, hq, d), 7.0, dtype=torch.float32, device=dev())
    vl = torch.full((10,), -5, dtype=torch.int32, device=dev())
    H.hswa_prefill_chunk(H.SWA, W, q, kn, vn, sid, cu, 7, st.view, st.kc, st.vc, out, vl)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    assert np.all(o[5:] == 7.0) and np.all(vl.cpu().numpy()[5:] == -5)
    assert float(np.max(np.abs(o[:5] - oracle_rows(s0, list(range(5)), OA.SWA, W)))) < TOL
    assert vl.cpu().tolist()[:5] == [OA.valid_length(p, OA.SWA, W) for p in range(5)]
    # sequence 1's ring slots were never written: still the NaN fill
    assert torch.isnan(st.kc[torch.as_tensor(st.ring_pages[1].astype(np.int64))]).all()

    # decode: sequence 0 has rows [0, 2), sequence 1 claims [2, 5) of 4
    H.hswa_pool_evict(st.pool, [0, 1])
    H.hswa_pool_alloc(st.pool, [0, 1], [2, 3])
    q = torch.cat([s0.q[5:7], s1.q[7:9]]).to(dev())
    kn = torch.cat([s0.k[5:7], s1.k[7:9]]).to(dev())
    vn = torch.cat([s0.v[5:7], s1.v[7:9]]).to(dev())
    cu = torch.tensor([0, 2, 5], dtype=torch.int32, device=dev())
    out = torch.full((4, hq, d), 7.0, dtype=torch.float32, device=dev())
    vl = torch.full((4,), -5, dtype=torch.int32, device=dev())
    H.hswa_decode(H.SWA, W, q, kn, vn, sid, 10, st.view, st.kc, st.vc, out, None, vl,
                  cu_q=cu, max_q_len=3)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    assert np.all(o[2:] == 7.0) and np.all(vl.cpu().numpy()[2:] == -5)
    assert float(np.max(np.abs(o[:2] - oracle_rows(s0, [5, 6], OA.SWA, W)))) < TOL
    assert vl.cpu().tolist()[:2] == [W, W]


# ---------------------------------------------------------------------------
# A SWA ring of a single page (C = 16): the ring page index wraps twice per
# 32-key step, so every step must come back to that page


@pytest.mark.parametrize("W,chunk", [(5, 7), (9, 8), (1, 16)])
def test_swa_ring_of_one_page(gpu, W, chunk):
    hq, hkv, d = 4, 2, 64
    lens = [258, 3, 40]
    seqs = make_seqs(lens, hq, hkv, d, 97)
    maxp = max(lens) // 16 + 2
    st = Setup(H.SWA, W, 16, len(lens), maxp, len(lens) * maxp, hkv, d, 97)
    outs, vlens, _ = chunked_prefill(st, seqs, chunk, hq)
    _check_seq(outs, vlens, seqs, H.SWA, W)


@pytest.mark.parametrize("case", range(12))
def test_decode_random_configuration(gpu, case):
    """Seeded random single-row decode over a Full and a SWA layer: contexts
    1-20,000 tokens (several splits), GQA group, KV heads 1-3, d, window
    1-200 (ring slack drawn too)."""
    rnd = random.Random(9700 + case)
    g, hkv = rnd.choice([1, 2, 4, 8]), rnd.choice([1, 2, 3])
    d, W = rnd.choice([64, 128]), rnd.choice([1, 2, 5, 33, 128, 200])
    ctxs = [rnd.randint(1, 20000) for _ in range(rnd.randint(1, 6))]
    C = 16 * (-(-W // 16)) + rnd.choice([0, 16, 64])
    steps = rnd.randint(1, 3)
    print(f"case {case}: g {g} hkv {hkv} d {d} W {W} C {C} ctxs {ctxs} steps {steps}",
          flush=True)
    _decode_scenario(ctxs, steps, g * hkv, hkv, d, W, 900 + case, C=C)


@pytest.mark.parametrize("seed", range(8))
def test_pool_device_tables_random_with_truncate(gpu, seed):
    """Random alloc / evict / import / truncate / release sequences on random
    geometries (windows 1-200, rings from one page): host results and all
    four device tables bit-exact against the oracle simulator after every
    operation, refused operations included."""
    rnd = random.Random(4000 + seed)
    W = rnd.choice([1, 2, 5, 16, 33, 128, 200])
    C = 16 * (-(-W // 16) + rnd.choice([0, 0, 1, 3]))
    S, maxp = rnd.randint(1, 6), rnd.randint(2, 30)
    npages = rnd.randint(2, max(4, S * maxp))
    free = synth.permutation(npages, 40 + seed, 1)
    ring = synth.permutation(S * C // 16, 40 + seed, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    t = pool.tables
    for step in range(100):
        ids = rnd.sample(range(S), rnd.randint(1, S))
        r = rnd.random()
        if r < 0.4:
            n = [rnd.choice([0, 1, 2, 4, 16, rnd.randint(0, C)]) for _ in ids]
            try:
                exp = sim.alloc(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_alloc(pool, ids, n)
                continue
            got = H.hswa_pool_alloc(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.55:
            # cut back up to 4 drafts, or far below the window (refused)
            lens = [max(0, sim.length[i] - rnd.choice([0, 1, 3, 4, W + 5])) for i in ids]
            try:
                sim.truncate(ids, lens)
            except ValueError:
                with pytest.raises(H.HswaError):
                    H.hswa_pool_truncate(pool, ids, lens)
                continue
            H.hswa_pool_truncate(pool, ids, lens)
        elif r < 0.85:
            exp = sim.evict(ids)
            got = H.hswa_pool_evict(pool, ids)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.95:
            n = [rnd.randint(0, 3 * W + 20) for _ in ids]
            try:
                exp = sim.import_context(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_import(pool, ids, n)
                continue
            got = H.hswa_pool_import(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        else:
            sim.release(ids)
            H.hswa_pool_release(pool, ids)
        torch.cuda.synchronize()
        assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
        assert t["fpt"].cpu().view(S, maxp).tolist() == sim.fpt_table()
        assert t["map"].cpu().tolist() == sim.map_table()
        assert t["rpt"].cpu().view(S, C // 16).tolist() == sim.rpt_table()
