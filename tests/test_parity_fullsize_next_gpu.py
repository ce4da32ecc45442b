"""GPU parity at full size for multi-token decode and FP8 decode, in the
launch configuration bench.py times (its `mtp_decode` and `mixed_decode_fp8`
workloads): 256 sequences with 4096..32768 tokens of context, one Full and
one SWA layer, the bench's max_seq_len (hence the same split plan).

Sampled sequences (the shortest, the longest and seeded ones) are checked in
full against the oracle; pool slots, eviction sets and valid lengths are
checked for every sequence.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle import fp8 as F8
from oracle.pool import PoolSim

from harness import TOL, dev

pytestmark = pytest.mark.gpu


def _draw(shape, seed, layer, b, role):
    return synth.bf16_normal(shape, seed, layer, b, role, device=dev())


def _sampled(ctxs, seed, k):
    rng = np.random.default_rng(seed + 5)
    s = {int(np.argmin(ctxs)), int(np.argmax(ctxs))}
    s |= set(int(x) for x in rng.choice(len(ctxs), size=k, replace=False))
    return sorted(s)


def _values(x, fp8):
    """What the oracle attends to for stored rows: the bf16 values, or their
    FP8 dequantization."""
    if not fp8:
        return synth.to_f64(x)
    codes, scale = F8.quantize_rows(x.float().cpu().numpy())
    return F8.dequantize_rows(codes, scale)


def _run(ctxs, W, C, seed, steps, rows, fp8, maxlen, sampled):
    hq, hkv, d = 64, 8, 128
    B = len(ctxs)
    maxp = maxlen // 16 + 2
    nfull = int(sum(c // 16 + 2 for c in ctxs) * 1.1) + B * (maxlen - max(ctxs)) // 16 + 64
    free = synth.permutation(nfull, seed, 1)
    ring = synth.permutation(B * C // 16, seed, 2)
    pool = H.hswa_pool_create(W, C, B, maxp, nfull, free, ring, device=dev())
    sim = PoolSim(W, C, B, maxp, nfull, free, ring)
    view = H.hswa_pool_get_view(pool)
    alloc = (lambda n: H.kv_cache_alloc_fp8(n, hkv, d, dev(), 0x7F)) if fp8 else \
        (lambda n: H.kv_cache_alloc(n, hkv, d, dev(), float("nan")) + (None, None))
    layers = [(H.FULL,) + tuple(alloc(nfull)), (H.SWA,) + tuple(alloc(B * C // 16))]
    ids = list(range(B))
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    assert [list(x) for x in H.hswa_pool_import(pool, ids, ctxs)] == \
        [list(x) for x in sim.import_context(ids, ctxs)]
    hist = {}   # (layer, sampled seq) -> [values of stored positions], fp64
    for li, (kind, kc, vc, ks, vs) in enumerate(layers):
        for b, c in enumerate(ctxs):
            lo = 0 if kind == H.FULL else c - min(c, W - 1)
            k = _draw((c - lo, hkv, d), seed, li, b, synth.ROLE_K)
            v = _draw((c - lo, hkv, d), seed, li, b, synth.ROLE_V)
            one = torch.tensor([b], dtype=torch.int32, device=dev())
            cu = torch.tensor([0, c - lo], dtype=torch.int32, device=dev())
            if c - lo > 0:
                H.hswa_append_kv(kind, k, v, one, view, kc, vc, cu, c - lo, k_scale=ks,
                                 v_scale=vs)
            if b in sampled:
                hist[li, b] = (lo, [_values(k, fp8)], [_values(v, fp8)])
            del k, v
    torch.cuda.synchronize()
    lens = list(ctxs)
    worst = 0.0
    for t in range(steps):
        n = [rows] * B
        full_slots, swa_slots = H.hswa_pool_alloc(pool, ids, n)
        ef, es = sim.alloc(ids, n)
        assert list(full_slots) == ef and list(swa_slots) == es
        T = rows * B
        cu = torch.tensor(np.arange(0, T + 1, rows), dtype=torch.int32, device=dev())
        acc = synth.uniform_ints(B, 1, rows, seed, 700, t) if rows > 1 else [1] * B
        for li, (kind, kc, vc, ks, vs) in enumerate(layers):
            q = _draw((T, hq, d), seed, 50 + li, t, synth.ROLE_Q)
            kn = _draw((T, hkv, d), seed, 50 + li, t, synth.ROLE_K)
            vn = _draw((T, hkv, d), seed, 50 + li, t, synth.ROLE_V)
            out = torch.full((T, hq, d), float("nan"), dtype=torch.float32, device=dev())
            vl = torch.full((T,), -1, dtype=torch.int32, device=dev())
            nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen, total_q=T)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            kw = dict(cu_q=cu, max_q_len=rows) if rows > 1 else {}
            H.hswa_decode(kind, W, q, kn, vn, sid, maxlen, view, kc, vc, out, ws, vl,
                          k_scale=ks, v_scale=vs, **kw)
            want = [OA.valid_length(p, kind, W) for b in ids for p in range(lens[b], lens[b] + rows)]
            assert vl.cpu().tolist() == want
            got = out.cpu().double().numpy()
            for b in sampled:
                lo, hk, hv = hist[li, b]
                r0 = b * rows
                k_all = np.concatenate(hk + [_values(kn[r0:r0 + rows], fp8)])
                v_all = np.concatenate(hv + [_values(vn[r0:r0 + rows], fp8)])
                pos = list(range(lens[b], lens[b] + rows))
                exp = OA.attend(synth.to_f64(q[r0:r0 + rows]), [p - lo for p in pos], k_all,
                                v_all, kind, W)
                assert np.all(np.isfinite(got[r0:r0 + rows]))
                err = float(np.max(np.abs(got[r0:r0 + rows] - exp)))
                worst = max(worst, err)
                assert err < TOL, f"step {t} kind {kind} sequence {b}: max-abs {err:.3e}"
                # the accepted rows join the stored history
                hk.append(_values(kn[r0:r0 + acc[b]], fp8))
                hv.append(_values(vn[r0:r0 + acc[b]], fp8))
        keep = [L + a for L, a in zip(lens, acc)]
        if rows > 1:
            H.hswa_pool_truncate(pool, ids, keep)
            sim.truncate(ids, keep)
        ev, cnt = H.hswa_pool_evict(pool, ids)
        eev, ecnt = sim.evict(ids)
        assert list(cnt) == ecnt and list(ev) == eev
        lens = keep
    t_ = pool.tables
    assert t_["seq_len"].cpu().tolist() == sim.seq_len_table()
    assert t_["map"].cpu().tolist() == sim.map_table()
    return worst


def test_mtp_decode_fullsize(gpu):
    """The mtp_decode workload: four rows per sequence per step (one token and
    three drafts), a seeded accepted prefix kept by truncate, ring W + 16."""
    wl = synth.MTP
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    rows = wl.drafts + 1
    maxlen = max(ctxs) + (32 + 4 + 8) * rows + 1    # bench.py's max_seq_len
    worst = _run(ctxs, wl.window, wl.ring_slots, wl.seed, 3, rows, False, maxlen,
                 _sampled(ctxs, wl.seed, 10))
    print(f"MTP full size: worst max-abs {worst:.3e}")


def test_fp8_decode_fullsize(gpu):
    """The mixed_decode_fp8 workload: FP8 pages, one row per sequence."""
    wl = synth.C3
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    maxlen = max(ctxs) + (32 + 4 + 8) + 1
    worst = _run(ctxs, wl.window, wl.ring_slots, wl.seed, 3, 1, True, maxlen,
                 _sampled(ctxs, wl.seed, 10))
    print(f"FP8 full size: worst max-abs {worst:.3e}")
