"""GPU checks of the q_pos argument (each sequence's first query row given
by the caller instead of read from the pool's seq_len table).

With q_pos, SWA appends and attention read only the fixed ring table, so the
pool calls (alloc, evict, release) may run on a second stream with no waits
between the streams.  A chunked SWA prefill run that way gives bitwise the
outputs of the single-stream run without q_pos, within 4e-3 of the oracle,
and the pool's device tables end equal to the oracle simulator's.  Decode
and Full prefill with q_pos equal the same calls without it, bitwise.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle.pool import PoolSim

from harness import TOL, Setup, dev, make_seqs, oracle_rows

pytestmark = pytest.mark.gpu


def _chunked(st, seqs, chunk, hq, use_qpos, side):
    B = len(seqs)
    lens = [s.q.shape[0] for s in seqs]
    d = st.d
    outs = [torch.empty((L, hq, d), dtype=torch.float32, device=dev()) for L in lens]
    done = [0] * B
    main = torch.cuda.current_stream()
    ps = side if side is not None else main
    while True:
        act = [b for b in range(B) if done[b] < lens[b]]
        if not act:
            break
        n = [min(chunk, lens[b] - done[b]) for b in act]
        H.hswa_pool_alloc(st.pool, act, n, want_slots=False, stream=ps)
        rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
        q = torch.cat([seqs[b].q[a:e] for b, a, e in rows]).to(dev())
        kn = torch.cat([seqs[b].k[a:e] for b, a, e in rows]).to(dev())
        vn = torch.cat([seqs[b].v[a:e] for b, a, e in rows]).to(dev())
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        sid = torch.tensor(act, dtype=torch.int32, device=dev())
        qp = torch.tensor([a for _, a, _ in rows], dtype=torch.int32, device=dev())
        out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device=dev())
        H.hswa_prefill_chunk(st.kind, st.W, q, kn, vn, sid, cu, max(n), st.view, st.kc, st.vc,
                             out, q_pos=qp if use_qpos else None, stream=main)
        o = 0
        for b, a, e in rows:
            outs[b][a:e] = out[o:o + e - a]
            o += e - a
        H.hswa_pool_evict(st.pool, act, want_slots=False, stream=ps)
        for b, k in zip(act, n):
            done[b] += k
    torch.cuda.synchronize()
    return [o.cpu() for o in outs]


def test_swa_prefill_with_pool_calls_on_a_second_stream(gpu):
    hq, hkv, d, W, chunk = 16, 2, 128, 64, 96
    lens = [700, 1, 333, 96, 517]
    B = len(lens)
    C = W + chunk
    C = -(-C // 16) * 16
    seqs = make_seqs(lens, hq, hkv, d, seed=191)
    maxp = max(lens) // 16 + 2
    ref_st = Setup(H.SWA, W, C, B, maxp, B * maxp + 4, hkv, d, seed=191)
    ref = _chunked(ref_st, seqs, chunk, hq, use_qpos=False, side=None)
    st = Setup(H.SWA, W, C, B, maxp, B * maxp + 4, hkv, d, seed=191)
    side = torch.cuda.Stream()        # default priority
    got = _chunked(st, seqs, chunk, hq, use_qpos=True, side=side)
    for b in range(B):
        assert torch.equal(got[b].view(torch.int32), ref[b].view(torch.int32)), b
        exp = oracle_rows(seqs[b], list(range(lens[b])), H.SWA, W)
        assert float(np.max(np.abs(got[b].double().numpy() - exp))) < TOL
    sim = PoolSim(W, C, B, maxp, B * maxp + 4, synth.permutation(B * maxp + 4, 191, 1),
                  synth.permutation(B * C // 16, 191, 2))
    done = [0] * B
    while any(done[b] < lens[b] for b in range(B)):
        act = [b for b in range(B) if done[b] < lens[b]]
        n = [min(chunk, lens[b] - done[b]) for b in act]
        sim.alloc(act, n)
        sim.evict(act)
        for b, k in zip(act, n):
            done[b] += k
    t = st.pool.tables
    assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
    assert t["fpt"].cpu().view(B, maxp).tolist() == sim.fpt_table()
    assert t["map"].cpu().tolist() == sim.map_table()


@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_q_pos_equals_seq_len_rows(gpu, kind):
    """Prefill of a chunk and decode of one row per sequence, with q_pos
    given and without: bitwise equal outputs and valid lengths."""
    hq, hkv, d, W = 8, 2, 64, 32
    lens = [150, 40, 77]
    B = len(lens)
    seqs = make_seqs([L + 1 for L in lens], hq, hkv, d, seed=193)
    maxp = max(lens) // 16 + 3
    st = Setup(kind, W, 160, B, maxp, B * maxp + 4, hkv, d, seed=193)
    ids = list(range(B))
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    # prefill of each whole sequence in one chunk
    H.hswa_pool_alloc(st.pool, ids, lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev())
    q = torch.cat([s.q[:L] for s, L in zip(seqs, lens)]).to(dev())
    kn = torch.cat([s.k[:L] for s, L in zip(seqs, lens)]).to(dev())
    vn = torch.cat([s.v[:L] for s, L in zip(seqs, lens)]).to(dev())
    outs, vls = [], []
    for qp in (None, torch.zeros(B, dtype=torch.int32, device=dev())):
        out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device=dev())
        vl = torch.empty((q.shape[0],), dtype=torch.int32, device=dev())
        H.hswa_prefill_chunk(kind, W, q, kn, vn, sid, cu, max(lens), st.view, st.kc, st.vc, out,
                             vl, q_pos=qp)
        outs.append(out)
        vls.append(vl)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    assert torch.equal(vls[0], vls[1])
    H.hswa_pool_evict(st.pool, ids)
    # one decode row per sequence
    H.hswa_pool_alloc(st.pool, ids, [1] * B)
    qd = torch.stack([s.q[L] for s, L in zip(seqs, lens)]).to(dev())
    kd = torch.stack([s.k[L] for s, L in zip(seqs, lens)]).to(dev())
    vd = torch.stack([s.v[L] for s, L in zip(seqs, lens)]).to(dev())
    maxlen = max(lens) + 1
    nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen)
    ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
    dec = []
    for qp in (None, torch.tensor(lens, dtype=torch.int32, device=dev())):
        out = torch.empty((B, hq, d), dtype=torch.float32, device=dev())
        H.hswa_decode(kind, W, qd, kd, vd, sid, maxlen, st.view, st.kc, st.vc, out, ws, q_pos=qp)
        torch.cuda.synchronize()
        dec.append(out.cpu())
    assert torch.equal(dec[0].view(torch.int32), dec[1].view(torch.int32))
    for b in range(B):
        exp = oracle_rows(seqs[b], [lens[b]], kind, W)[0]
        assert float(np.max(np.abs(dec[1][b].double().numpy() - exp))) < TOL
