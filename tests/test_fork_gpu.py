"""GPU checks of prefix reuse across requests (hswa_pool_fork + hswa_kv_copy).

"MiMo-V2.5 Series Inference Full-Link Optimization" sec. 2.1, "SWA-aware
prefix cache tree", points 1 and 3: a window-safe prefix of one request is
reused by another; the Full part is shared, the SWA window moves with it.

- Device tables: random operation sequences with forks (shared pages,
  forks of forks, refused cuts into shared pages); all four device tables
  bit-exact against the oracle simulator after every operation.
- End to end: a source sequence is prefilled through a Full and a SWA layer
  and evicted; an empty sequence forks its whole length (window-safe) and
  copies the tail K/V of both layers; then both sequences decode different
  continuations.  Every output is within 4e-3 of the oracle evaluated on the
  sequence each one really holds (the shared prefix plus its own tokens);
  the source keeps decoding correctly next to the fork, and the fork keeps
  decoding after the source is released (its shared pages stay held).
"""
import random

import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle.pool import NoSpace, PoolSim

from harness import TOL, dev

pytestmark = pytest.mark.gpu


def _tables_match(pool, sim, S, maxp, C):
    t = pool.tables
    torch.cuda.synchronize()
    assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
    assert t["fpt"].cpu().view(S, maxp).tolist() == sim.fpt_table()
    assert t["map"].cpu().tolist() == sim.map_table()
    assert t["rpt"].cpu().view(S, C // 16).tolist() == sim.rpt_table()


@pytest.mark.parametrize("seed", range(6))
def test_device_tables_with_forks(gpu, seed):
    rnd = random.Random(5000 + seed)
    W = rnd.choice([1, 2, 5, 16, 20, 33])
    C = 16 * (-(-W // 16) + rnd.choice([0, 1, 2]))
    S, maxp = rnd.randint(3, 6), rnd.randint(6, 16)
    npages = rnd.randint(S * maxp // 2, S * maxp)
    free = synth.permutation(npages, 60 + seed, 1)
    ring = synth.permutation(S * C // 16, 60 + seed, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    forks = 0
    for step in range(120):
        r = rnd.random()
        if r < 0.25:
            src = rnd.randrange(S)
            empty = [i for i in range(S) if sim.length[i] == 0 and i != src]
            if not empty or sim.length[src] == 0:
                continue
            dst = rnd.choice(empty)
            want = rnd.randint(1, sim.length[src])
            m = rnd.choice([sim.window_safe_len(src, want, W - 1)] * 3 + [want])
            try:
                exp = sim.fork([src], [dst], [m])
            except (ValueError, NoSpace) as err:
                with pytest.raises(H.NoSpace if isinstance(err, NoSpace) else H.HswaError):
                    H.hswa_pool_fork(pool, [src], [dst], [m])
                continue
            ff, sf = H.hswa_pool_fork(pool, [src], [dst], [m])
            assert ff.tolist() == exp[0] and sf.tolist() == exp[1]
            forks += 1
        elif r < 0.5:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            n = [rnd.choice([0, 1, 3, 16, 30]) for _ in ids]
            try:
                exp = sim.alloc(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_alloc(pool, ids, n)
                continue
            got = H.hswa_pool_alloc(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.7:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            exp = sim.evict(ids)
            got = H.hswa_pool_evict(pool, ids)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.8:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            n = [rnd.randint(0, 2 * W + 40) for _ in ids]
            try:
                exp = sim.import_context(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_import(pool, ids, n)
                continue
            got = H.hswa_pool_import(pool, ids, n)
            assert list(got[0]) == exp[0] and list(got[1]) == exp[1]
        elif r < 0.9:
            ids = [rnd.randrange(S)]
            lens = [max(0, sim.length[ids[0]] - rnd.choice([1, 2, 17, 40, 100]))]
            try:
                sim.truncate(ids, lens)
            except ValueError:
                with pytest.raises(H.HswaError):
                    H.hswa_pool_truncate(pool, ids, lens)
                continue
            H.hswa_pool_truncate(pool, ids, lens)
        else:
            ids = rnd.sample(range(S), rnd.randint(1, 2))
            sim.release(ids)
            H.hswa_pool_release(pool, ids)
        _tables_match(pool, sim, S, maxp, C)
    assert forks >= 3


def _oracle_row(k, v, q, pos, kind, W):
    return OA.attend(synth.to_f64(q), [pos], synth.to_f64(k), synth.to_f64(v), kind, W)[0]


def test_fork_then_decode_both_sequences(gpu):
    hq, hkv, d, W, chunk = 16, 2, 128, 48, 64
    C = W + chunk + 16                      # ring slots, a multiple of 16
    Ls, steps = 333, 6
    S, maxp = 3, (Ls + steps + 16) // 16 + 2
    npages = S * maxp
    # the source's tokens (prefix and its own continuation) and the fork's
    # continuation, drawn independently
    src_q = synth.bf16_normal((Ls + steps, hq, d), 81, 0, 0, synth.ROLE_Q)
    src_k = synth.bf16_normal((Ls + steps, hkv, d), 81, 0, 0, synth.ROLE_K)
    src_v = synth.bf16_normal((Ls + steps, hkv, d), 81, 0, 0, synth.ROLE_V)
    new_q = synth.bf16_normal((steps, hq, d), 81, 0, 1, synth.ROLE_Q)
    new_k = synth.bf16_normal((steps, hkv, d), 81, 0, 1, synth.ROLE_K)
    new_v = synth.bf16_normal((steps, hkv, d), 81, 0, 1, synth.ROLE_V)
    free = synth.permutation(npages, 82, 1)
    ring = synth.permutation(S * C // 16, 82, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    view = H.hswa_pool_get_view(pool)
    layers = {H.FULL: H.kv_cache_alloc(npages, hkv, d, dev(), float("nan")),
              H.SWA: H.kv_cache_alloc(S * C // 16, hkv, d, dev(), float("nan"))}

    # prefill the source through both layers, chunk by chunk, with eviction
    sid0 = torch.zeros(1, dtype=torch.int32, device=dev())
    for a in range(0, Ls, chunk):
        e = min(Ls, a + chunk)
        H.hswa_pool_alloc(pool, [0], [e - a])
        sim.alloc([0], [e - a])
        cu = torch.tensor([0, e - a], dtype=torch.int32, device=dev())
        for kind, (kc, vc) in layers.items():
            out = torch.empty((e - a, hq, d), dtype=torch.float32, device=dev())
            H.hswa_prefill_chunk(kind, W, src_q[a:e].to(dev()), src_k[a:e].to(dev()),
                                 src_v[a:e].to(dev()), sid0, cu, e - a, view, kc, vc, out)
        H.hswa_pool_evict(pool, [0])
        sim.evict([0])
    _tables_match(pool, sim, S, maxp, C)

    # fork the whole source (window-safe: eviction keeps its last W - 1)
    m = int(H.hswa_pool_match_len(pool, [0], [Ls])[0])
    assert m == Ls
    ff, sf = H.hswa_pool_fork(pool, [0], [1], [m])
    exp = sim.fork([0], [1], [m])
    assert ff.tolist() == exp[0] and sf.tolist() == exp[1]
    assert sf[0] == m - W + 1 and ff[0] == 16 * ((m - W + 1) // 16)
    _tables_match(pool, sim, S, maxp, C)
    t = H.hswa_pool_read_tables(pool)
    assert (t["fpt"][1][:ff[0] // 16] == t["fpt"][0][:ff[0] // 16]).all()   # shared pages
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev())
    for kind, first in ((H.FULL, int(ff[0])), (H.SWA, int(sf[0]))):
        kc, vc = layers[kind]
        H.hswa_kv_copy(kind, i32([0]), i32([1]), i32([first]), i32([m]), m - first, view, kc,
                       vc)

    def decode(b, q, k, v, ws_len):
        """One decode step of sequence b over both layers; returns outputs."""
        H.hswa_pool_alloc(pool, [b], [1])
        sim.alloc([b], [1])
        sid = i32([b])
        res = {}
        for kind, (kc, vc) in layers.items():
            out = torch.full((1, hq, d), float("nan"), dtype=torch.float32, device=dev())
            nb = H.hswa_decode_workspace_bytes(kind, W, 1, hq, hkv, d, ws_len)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            H.hswa_decode(kind, W, q.to(dev()), k.to(dev()), v.to(dev()), sid, ws_len, view, kc,
                          vc, out, ws)
            res[kind] = out
        H.hswa_pool_evict(pool, [b])
        sim.evict([b])
        torch.cuda.synchronize()
        return {kind: o.cpu().double().numpy()[0] for kind, o in res.items()}

    def check(outs, k_all, v_all, q, pos):
        for kind in (H.FULL, H.SWA):
            want = _oracle_row(k_all, v_all, q, pos, kind, W)
            err = float(np.max(np.abs(outs[kind] - want)))
            assert err < TOL, f"kind {kind} position {pos}: {err:.3e}"

    # both sequences decode side by side, each its own continuation
    for t_ in range(steps - 2):
        pos = m + t_
        o1 = decode(1, new_q[t_:t_ + 1], new_k[t_:t_ + 1], new_v[t_:t_ + 1], pos + 1)
        k1 = torch.cat([src_k[:m], new_k[:t_ + 1]])
        v1 = torch.cat([src_v[:m], new_v[:t_ + 1]])
        check(o1, k1, v1, new_q[t_:t_ + 1], pos)
        o0 = decode(0, src_q[pos:pos + 1], src_k[pos:pos + 1], src_v[pos:pos + 1], pos + 1)
        check(o0, src_k[:pos + 1], src_v[:pos + 1], src_q[pos:pos + 1], pos)
        _tables_match(pool, sim, S, maxp, C)
    # the source ends; the fork keeps its shared pages and decodes on
    H.hswa_pool_release(pool, [0])
    sim.release([0])
    _tables_match(pool, sim, S, maxp, C)
    for t_ in range(steps - 2, steps):
        pos = m + t_
        o1 = decode(1, new_q[t_:t_ + 1], new_k[t_:t_ + 1], new_v[t_:t_ + 1], pos + 1)
        k1 = torch.cat([src_k[:m], new_k[:t_ + 1]])
        v1 = torch.cat([src_v[:m], new_v[:t_ + 1]])
        check(o1, k1, v1, new_q[t_:t_ + 1], pos)
    H.hswa_pool_release(pool, [1])
    sim.release([1])
    _tables_match(pool, sim, S, maxp, C)
    assert sorted(H.hswa_pool_read_tables(pool)["free"].tolist()) == list(range(npages))
