"""GPU checks of hswa_pool_evict_alloc: a chunk step's eviction and the next
step's alloc as one operation with one device-table update.

"MiMo-V2.5 Series Inference Full-Link Optimization" sec. 2.1 ("KVCache Dual
Pool"; "SWA-aware prefix cache tree", point 2: out-of-window SWA entries are
released per chunk).  The operation is, by definition, the eviction followed
by the alloc, so the oracle simulator runs those two in order.

- Random operation sequences (allocs, evictions, combined operations with
  overlapping and disjoint id lists, imports, releases) on random pool
  geometries: all four device tables bit-exact against the simulator after
  every operation, and a failed combined operation changes no table.
- A chunked SWA prefill driven by combined operations gives bitwise the
  outputs of the same prefill driven by separate evictions and allocs.
"""
import copy
import random

import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle.pool import NoSpace, PoolSim

from harness import dev

pytestmark = pytest.mark.gpu


def _tables_match(pool, sim, S, maxp, C):
    t = pool.tables
    torch.cuda.synchronize()
    assert t["seq_len"].cpu().tolist() == sim.seq_len_table()
    assert t["fpt"].cpu().view(S, maxp).tolist() == sim.fpt_table()
    assert t["map"].cpu().tolist() == sim.map_table()
    assert t["rpt"].cpu().view(S, C // 16).tolist() == sim.rpt_table()


@pytest.mark.parametrize("seed", range(6))
def test_device_tables_with_combined_ops(gpu, seed):
    rnd = random.Random(7000 + seed)
    W = rnd.choice([1, 2, 5, 16, 20, 33, 128])
    C = 16 * (-(-W // 16) + rnd.choice([0, 1, 2, 4]))
    S, maxp = rnd.randint(2, 6), rnd.randint(6, 24)
    npages = rnd.randint(S * maxp // 2, S * maxp)
    free = synth.permutation(npages, 90 + seed, 1)
    ring = synth.permutation(S * C // 16, 90 + seed, 2)
    pool = H.hswa_pool_create(W, C, S, maxp, npages, free, ring, device=dev())
    sim = PoolSim(W, C, S, maxp, npages, free, ring)
    combined = 0
    for step in range(100):
        r = rnd.random()
        if r < 0.5:
            ev_ids = rnd.sample(range(S), rnd.randint(0, S))
            al_ids = rnd.sample(range(S), rnd.randint(0, S))
            n = [rnd.choice([0, 1, 3, 16, 30, C]) for _ in al_ids]
            snap = copy.deepcopy(sim)
            try:
                e_ev = sim.evict(ev_ids)
                e_al = sim.alloc(al_ids, n)
            except NoSpace:
                sim = snap
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_evict_alloc(pool, ev_ids, al_ids, n)
                _tables_match(pool, sim, S, maxp, C)
                continue
            ev, cnt, full, swa = H.hswa_pool_evict_alloc(pool, ev_ids, al_ids, n)
            assert ev.tolist() == e_ev[0] and cnt.tolist() == e_ev[1]
            assert full.tolist() == e_al[0] and swa.tolist() == e_al[1]
            combined += 1
        elif r < 0.7:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            n = [rnd.choice([0, 1, 3, 16]) for _ in ids]
            try:
                sim.alloc(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_alloc(pool, ids, n)
                continue
            H.hswa_pool_alloc(pool, ids, n)
        elif r < 0.8:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            sim.evict(ids)
            H.hswa_pool_evict(pool, ids)
        elif r < 0.9:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            n = [rnd.randint(0, 2 * W + 40) for _ in ids]
            try:
                sim.import_context(ids, n)
            except NoSpace:
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_import(pool, ids, n)
                continue
            H.hswa_pool_import(pool, ids, n)
        else:
            ids = rnd.sample(range(S), rnd.randint(1, 2))
            sim.release(ids)
            H.hswa_pool_release(pool, ids)
        _tables_match(pool, sim, S, maxp, C)
    assert combined >= 10


def _chunked_swa_prefill(combined):
    """8 sequences of 200-700 tokens in 64-token chunks through one SWA layer
    (W 48, 16 query / 2 KV heads, d 128); pool calls as separate evictions
    and allocs, or as combined operations at the chunk boundaries."""
    hq, hkv, d, W, chunk = 16, 2, 128, 48, 64
    lens = [200, 700, 333, 64, 65, 512, 257, 640]
    B, C = len(lens), W + chunk + 16
    maxp = max(lens) // 16 + 2
    npages = B * maxp
    pool = H.hswa_pool_create(W, C, B, maxp, npages, synth.permutation(npages, 95, 1),
                              synth.permutation(B * C // 16, 95, 2), device=dev())
    view = H.hswa_pool_get_view(pool)
    kc, vc = H.kv_cache_alloc(B * C // 16, hkv, d, dev(), float("nan"))
    outs = []
    done = [0] * B
    prev = []
    while True:
        act = [b for b in range(B) if done[b] < lens[b]]
        n = [min(chunk, lens[b] - done[b]) for b in act]
        if combined:
            H.hswa_pool_evict_alloc(pool, prev, act, n)
        else:
            H.hswa_pool_evict(pool, prev)
            H.hswa_pool_alloc(pool, act, n)
        if not act:
            break
        rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
        q = torch.cat([synth.bf16_normal((lens[b], hq, d), 96, 0, b, synth.ROLE_Q)[a:e]
                       for b, a, e in rows]).to(dev())
        k = torch.cat([synth.bf16_normal((lens[b], hkv, d), 96, 0, b, synth.ROLE_K)[a:e]
                       for b, a, e in rows]).to(dev())
        v = torch.cat([synth.bf16_normal((lens[b], hkv, d), 96, 0, b, synth.ROLE_V)[a:e]
                       for b, a, e in rows]).to(dev())
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        sid = torch.tensor(act, dtype=torch.int32, device=dev())
        out = torch.empty((q.shape[0], hq, d), dtype=torch.float32, device=dev())
        H.hswa_prefill_chunk(H.SWA, W, q, k, v, sid, cu, max(n), view, kc, vc, out)
        outs.append(out.cpu())
        for b, k_ in zip(act, n):
            done[b] += k_
        prev = act
    H.hswa_pool_release(pool, list(range(B)))
    return outs


def test_chunked_prefill_with_combined_ops_is_bitwise_equal(gpu):
    a, b = _chunked_swa_prefill(False), _chunked_swa_prefill(True)
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
