"""GPU parity of multi-token decode (one token plus up to three drafts per
sequence, the MTP verification step of the MiMo-V2.5 inference page,
section 5.2) over the dual pool, against the fp64 oracle.

Each step: alloc n_b rows per sequence -> decode both layers with the rows
of every sequence (each row attends causally to its own keys) -> keep the
accepted prefix with hswa_pool_truncate -> evict.  Rows a step rejects are
drawn afresh the next step, so the pool must hold exactly the accepted
history; the slots of dropped rows are NaN-poisoned after the truncate and
the ring slots of evicted positions after the evict, so a read of either
shows up as a non-finite output.

Bar: max-abs error 4e-3 against the oracle, valid lengths and pool tables
bit-exact.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle.pool import PoolSim

from harness import TOL, dev

pytestmark = pytest.mark.gpu


def _poison_slots(kc, vc, slots):
    if len(slots) == 0:
        return
    s = torch.as_tensor(np.asarray(slots, dtype=np.int64), device=dev())
    kc[s // 16, :, s % 16, :] = float("nan")
    vc[s // 16, :, :, s % 16] = float("nan")


def _mtp_scenario(ctxs, steps, hq, hkv, d, W, seed, max_rows=4, check_plain=False):
    B = len(ctxs)
    # the ring holds the window plus the step's rows, in whole pages
    C = 16 * max(-(-(W - 1 + max_rows) // 16), -(-W // 16))
    maxp = (max(ctxs) + steps * max_rows) // 16 + 2
    npages = B * maxp + 8
    free = synth.permutation(npages, seed, 1)
    ring = synth.permutation(B * C // 16, seed, 2)
    pool = H.hswa_pool_create(W, C, B, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, B, maxp, npages, free, ring)
    view = H.hswa_pool_get_view(pool)
    fkc, fvc = H.kv_cache_alloc(npages, hkv, d, dev(), float("nan"))
    skc, svc = H.kv_cache_alloc(B * C // 16, hkv, d, dev(), float("nan"))
    ids = list(range(B))
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    # committed history per sequence (what the oracle sees), bf16 on the host
    hist_k = [synth.bf16_normal((c, hkv, d), seed, 0, b, synth.ROLE_K) for b, c in enumerate(ctxs)]
    hist_v = [synth.bf16_normal((c, hkv, d), seed, 0, b, synth.ROLE_V) for b, c in enumerate(ctxs)]
    # restored contexts: every position in the Full layer, the in-window
    # tail in the SWA ring
    H.hswa_pool_import(pool, ids, ctxs)
    sim.import_context(ids, ctxs)
    live = [b for b in ids if ctxs[b] > 0]
    if live:
        cu = torch.tensor(np.concatenate([[0], np.cumsum([ctxs[b] for b in live])]),
                          dtype=torch.int32, device=dev())
        lid = torch.tensor(live, dtype=torch.int32, device=dev())
        H.hswa_append_kv(H.FULL, torch.cat([hist_k[b] for b in live]).to(dev()),
                         torch.cat([hist_v[b] for b in live]).to(dev()), lid, view, fkc, fvc,
                         cu, max(ctxs))
        nw = [min(ctxs[b], W - 1) for b in live]
        cuw = torch.tensor(np.concatenate([[0], np.cumsum(nw)]), dtype=torch.int32, device=dev())
        H.hswa_append_kv(H.SWA, torch.cat([hist_k[b][ctxs[b] - k:] for b, k in zip(live, nw)]).to(dev()),
                         torch.cat([hist_v[b][ctxs[b] - k:] for b, k in zip(live, nw)]).to(dev()),
                         lid, view, skc, svc, cuw, max(nw))
    worst = 0.0
    for t in range(steps):
        n = synth.uniform_ints(B, 1, max_rows, seed, t, 0)
        acc = [synth.uniform_ints(1, 1, k, seed, t, 1 + b)[0] for b, k in enumerate(n)]
        L0 = list(sim.length)
        full_slots, swa_slots = H.hswa_pool_alloc(pool, ids, n)
        exp_slots = sim.alloc(ids, n)
        assert list(full_slots) == exp_slots[0] and list(swa_slots) == exp_slots[1]
        q = synth.bf16_normal((sum(n), hq, d), seed, 1000 + t, 0, synth.ROLE_Q)
        kn = synth.bf16_normal((sum(n), hkv, d), seed, 1000 + t, 0, synth.ROLE_K)
        vn = synth.bf16_normal((sum(n), hkv, d), seed, 1000 + t, 0, synth.ROLE_V)
        offs = np.concatenate([[0], np.cumsum(n)])
        cu = torch.tensor(offs, dtype=torch.int32, device=dev())
        maxlen = max(L0[b] + n[b] for b in ids)
        qd, knd, vnd = q.to(dev()), kn.to(dev()), vn.to(dev())
        for kind, kc, vc in ((H.FULL, fkc, fvc), (H.SWA, skc, svc)):
            out = torch.full((sum(n), hq, d), float("nan"), dtype=torch.float32, device=dev())
            vl = torch.full((sum(n),), -1, dtype=torch.int32, device=dev())
            nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen, total_q=sum(n))
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            H.hswa_decode(kind, W, qd, knd, vnd, sid, maxlen, view, kc, vc, out, ws, vl,
                          cu_q=cu, max_q_len=max(n))
            got = out.cpu().double().numpy()
            for b in ids:
                a, e = offs[b], offs[b + 1]
                pos = list(range(L0[b], L0[b] + n[b]))
                k_all = synth.to_f64(torch.cat([hist_k[b], kn[a:e]]))
                v_all = synth.to_f64(torch.cat([hist_v[b], vn[a:e]]))
                exp = OA.attend(synth.to_f64(q[a:e]), pos, k_all, v_all, kind, W)
                assert np.all(np.isfinite(got[a:e])), f"step {t} kind {kind} seq {b}: non-finite"
                err = float(np.max(np.abs(got[a:e] - exp)))
                worst = max(worst, err)
                assert err < TOL, f"step {t} kind {kind} seq {b}: {err:.3e}"
            assert vl.cpu().tolist() == [OA.valid_length(p, kind, W)
                                         for b in ids for p in range(L0[b], L0[b] + n[b])]
            if check_plain and max(n) == 1:
                # one row each: the multi-row form and the plain form agree bitwise
                out1 = torch.empty_like(out)
                H.hswa_decode(kind, W, qd, None, None, sid, maxlen, view, kc, vc, out1, ws)
                assert torch.equal(out, out1)
        # keep the accepted prefix; drop (and poison) the rest
        keep = [L0[b] + acc[b] for b in ids]
        dropped_full, dropped_swa = [], []
        for b in ids:
            a = int(offs[b])
            dropped_full += list(full_slots[a + acc[b]:a + n[b]])
            dropped_swa += list(swa_slots[a + acc[b]:a + n[b]])
        H.hswa_pool_truncate(pool, ids, keep)
        sim.truncate(ids, keep)
        torch.cuda.synchronize()
        _poison_slots(fkc, fvc, dropped_full)
        _poison_slots(skc, svc, dropped_swa)
        for b in ids:
            a = int(offs[b])
            hist_k[b] = torch.cat([hist_k[b], kn[a:a + acc[b]]])
            hist_v[b] = torch.cat([hist_v[b], vn[a:a + acc[b]]])
        ev, cnt = H.hswa_pool_evict(pool, ids)
        exp_ev = sim.evict(ids)
        assert list(ev) == exp_ev[0] and list(cnt) == exp_ev[1]
        torch.cuda.synchronize()
        # evicted positions' ring slots: their map entries held the SWA slots
        evicted_swa = []
        for i, b in enumerate(ids):
            evicted_swa += [sim.swa_slot(b, p)
                            for p in range(sim.res_start[b] - int(cnt[i]), sim.res_start[b])]
        _poison_slots(skc, svc, evicted_swa)
        t_ = pool.tables
        assert t_["seq_len"].cpu().tolist() == sim.seq_len_table()
        assert t_["fpt"].cpu().view(B, maxp).tolist() == sim.fpt_table()
        assert t_["map"].cpu().tolist() == sim.map_table()
    return worst


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_mtp_decode_gqa(gpu, g):
    hkv = 2 if g < 8 else 8
    _mtp_scenario([700, 1, 5, 130, 2000, 0], 5, g * hkv, hkv, 128, 128, 600 + g)


def test_mtp_decode_long_contexts_split(gpu):
    """Long Full-layer contexts take the split-K path; rows of one sequence
    whose keys end inside different splits merge correctly."""
    _mtp_scenario([20000, 9000, 70], 3, 64, 8, 128, 128, 611)


def test_mtp_decode_small_heads_d64(gpu):
    _mtp_scenario([1500, 90, 700, 3], 4, 8, 2, 64, 128, 621)


def test_mtp_decode_two_rows_and_small_window(gpu):
    """max_q_len 2 takes the two-row kernel; W = 5 puts most keys of the
    earlier rows outside the later rows' windows."""
    _mtp_scenario([300, 17, 64], 5, 16, 2, 128, 5, 631, max_rows=2)


def test_mtp_decode_one_row_matches_plain_decode(gpu):
    _mtp_scenario([900, 33, 4100], 3, 64, 8, 128, 128, 641, max_rows=1, check_plain=True)


@pytest.mark.parametrize("case", range(12))
def test_mtp_decode_random_configuration(gpu, case):
    """Seeded random shapes for multi-token verification with rejected
    drafts: contexts 0-3,000 tokens, GQA group, KV heads 1-3, d, window
    1-200 (rings down to one page), up to 2-4 rows per step."""
    import random
    rnd = random.Random(9300 + case)
    g, hkv = rnd.choice([1, 2, 4, 8]), rnd.choice([1, 2, 3])
    d, W = rnd.choice([64, 128]), rnd.choice([1, 2, 5, 33, 128, 200])
    ctxs = [rnd.randint(0, 3000) for _ in range(rnd.randint(1, 5))]
    steps, rows = rnd.randint(1, 4), rnd.choice([2, 3, 4])
    print(f"case {case}: g {g} hkv {hkv} d {d} W {W} ctxs {ctxs} steps {steps} rows {rows}",
          flush=True)
    _mtp_scenario(ctxs, steps, g * hkv, hkv, d, W, 700 + case, max_rows=rows)
