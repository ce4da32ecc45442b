"""Pins of the oracle's dual-pool simulator.

* hand-worked fixtures (tests/golden/pool_small.json) from the rules of the
  MiMo-V2.5 inference page, section 2.1;
* a second simulator written in a different style (position-keyed dicts,
  slot formulas evaluated from scratch) run on seeded random operation
  sequences;
* invariants the page states: SWA residency bounded by the window, Full
  index authoritative (map keys are Full slots of resident positions only),
  a failed joint capacity check changes nothing.
"""
import copy
import json
import os
import random

import pytest

from oracle.pool import NoSpace, PoolSim

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _state(p: PoolSim):
    return (p.seq_len_table(), p.fpt_table(), p.map_table(), p.free_pages(),
            list(p.res_start))


def _run_fixture(sc):
    c = sc["create"]
    p = PoolSim(c["window"], c["ring_slots"], c["max_seqs"], c["max_pages_per_seq"],
                c["num_full_pages"], c["free_order"], c["ring_pages"])
    for op in sc["ops"]:
        if op["op"] in ("alloc", "import"):
            fn = p.alloc if op["op"] == "alloc" else p.import_context
            if op.get("nospace"):
                before = _state(p)
                with pytest.raises(NoSpace):
                    fn(op["seq_ids"], op["n"])
                assert _state(p) == before
            else:
                full, swa = fn(op["seq_ids"], op["n"])
                assert full == op["full"] and swa == op["swa"], op
        elif op["op"] == "evict":
            ev, cnt = p.evict(op["seq_ids"])
            assert ev == op["evicted"] and cnt == op["counts"], op
        elif op["op"] == "release":
            p.release(op["seq_ids"])
        elif op["op"] == "match":
            assert p.window_safe_len(op["seq"], op["m"], op["tail"]) == op["expect"], op
        elif op["op"] == "truncate":
            if op.get("invalid"):
                before = _state(p)
                with pytest.raises(ValueError):
                    p.truncate(op["seq_ids"], op["new_len"])
                assert _state(p) == before
            else:
                p.truncate(op["seq_ids"], op["new_len"])
        else:
            raise AssertionError(f"unknown fixture op {op['op']}")
    f = sc["final"]
    assert p.seq_len_table() == f["seq_len"]
    assert p.fpt_table() == f["fpt"]
    assert p.free_pages() == f["free"]
    m = p.map_table()
    nonneg = {str(i): s for i, s in enumerate(m) if s >= 0}
    assert nonneg == f["map_nonneg"]


def test_hand_worked_fixtures():
    data = json.load(open(os.path.join(GOLDEN, "pool_small.json")))
    for sc in data["scenarios"]:
        _run_fixture(sc)


class DictPool:
    """Second simulator: positions keyed in dicts, nothing shared with PoolSim."""

    def __init__(self, W, C, max_seqs, max_pages, npages, free_order, ring_pages):
        self.W, self.C, self.maxp = W, C, max_pages
        self.free = list(free_order)
        self.ring = {b: list(ring_pages[b * (C // 16):(b + 1) * (C // 16)]) for b in range(max_seqs)}
        self.page_of = {b: {} for b in range(max_seqs)}   # logical page -> physical
        self.alive = {b: set() for b in range(max_seqs)}  # resident positions
        self.n = {b: 0 for b in range(max_seqs)}
        self.npages = npages

    def fslot(self, b, pos):
        return self.page_of[b][pos // 16] * 16 + pos % 16

    def sslot(self, b, pos):
        r = pos % self.C
        return self.ring[b][r // 16] * 16 + r % 16

    def _need(self, ids, ns):
        tot = 0
        for b, k in zip(ids, ns):
            have = len(self.page_of[b])
            want = (self.n[b] + k + 15) // 16
            if want > self.maxp:
                return None
            tot += max(0, want - have)
        return tot

    def alloc(self, ids, ns, importing=False):
        need = self._need(ids, ns)
        if need is None or need > len(self.free):
            raise NoSpace()
        if not importing:
            for b, k in zip(ids, ns):
                if len(self.alive[b]) + k > self.C:
                    raise NoSpace()
        fo, so = [], []
        for b, k in zip(ids, ns):
            end = self.n[b] + k
            if importing:
                self.alive[b] = {p for p in self.alive[b] if p > end - self.W}
            for pos in range(self.n[b], end):
                if pos // 16 not in self.page_of[b]:
                    self.page_of[b][pos // 16] = self.free.pop(0)
                fo.append(self.fslot(b, pos))
                if importing and pos <= end - self.W:
                    so.append(-1)
                else:
                    so.append(self.sslot(b, pos))
                    self.alive[b].add(pos)
            self.n[b] = end
        return fo, so

    def evict(self, ids):
        out, cnt = [], []
        for b in ids:
            gone = sorted(p for p in self.alive[b] if p <= self.n[b] - self.W)
            out += [self.fslot(b, p) for p in gone]
            cnt.append(len(gone))
            self.alive[b] -= set(gone)
        return out, cnt

    def release(self, ids):
        for b in ids:
            self.free += [self.page_of[b][i] for i in sorted(self.page_of[b])]
            self.page_of[b] = {}
            self.alive[b] = set()
            self.n[b] = 0

    def truncate(self, ids, lens):
        for b, n in zip(ids, lens):
            lo = min(self.alive[b]) if self.alive[b] else self.n[b]
            if n < 0 or n > self.n[b] or lo > max(0, n - self.W + 1):
                raise ValueError()
        for b, n in zip(ids, lens):
            self.alive[b] = {p for p in self.alive[b] if p < n}
            gone = sorted(lp for lp in self.page_of[b] if lp * 16 >= n)
            self.free = [self.page_of[b].pop(lp) for lp in gone] + self.free
            self.n[b] = n

    def match(self, b, m, tail):
        # walk back from the end of the match to the first position that lost
        # its SWA entry; the match may end no later than tail past it
        k = min(m, self.n[b])
        hole = -1
        for p in range(k - 1, -1, -1):
            if p not in self.alive[b]:
                hole = p
                break
        while k > 0 and max(0, k - tail) <= hole:
            k -= 1
            hole = max((p for p in range(k) if p not in self.alive[b]), default=-1)
        return k

    def map_table(self):
        t = [-1] * (self.npages * 16)
        for b in self.alive:
            for p in self.alive[b]:
                t[self.fslot(b, p)] = self.sslot(b, p)
        return t


def _check_invariants(p: PoolSim, just_evicted):
    m = p.map_table()
    res_slots = []
    for b in range(p.max_seqs):
        L = p.length[b]
        res = p.resident(b)
        if b in just_evicted:
            assert len(res) == min(L, p.W - 1)
        assert len(res) <= p.C
        for pos in range(L):
            fs = p.full_slot(b, pos)
            if pos in res:
                assert m[fs] == p.swa_slot(b, pos)
                res_slots.append(m[fs])
            else:
                assert m[fs] == -1
        if b in just_evicted and L > 0:
            # every position the next query can see (its W-1 predecessors) is resident
            for pos in range(max(0, L - p.W + 1), L):
                assert m[p.full_slot(b, pos)] >= 0
    # map injective on resident tokens
    assert len(res_slots) == len(set(res_slots))
    # Full pages are conserved
    used = sum(len(x) for x in p.pages)
    assert used + len(p.free) == p.num_full_pages
    assert len(set(p.free) | {q for x in p.pages for q in x}) == p.num_full_pages


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_against_second_simulator(seed):
    rnd = random.Random(seed)
    W = rnd.choice([1, 2, 5, 16, 33, 128])
    C = 16 * rnd.randint(max(1, -(-W // 16)), max(1, -(-W // 16)) + 3)
    S = rnd.randint(1, 5)
    maxp = rnd.randint(2, 12)
    npages = rnd.randint(3, S * maxp)
    free_order = list(range(npages))
    rnd.shuffle(free_order)
    ring = list(range(S * C // 16))
    rnd.shuffle(ring)
    a = PoolSim(W, C, S, maxp, npages, free_order, ring)
    b = DictPool(W, C, S, maxp, npages, free_order, ring)
    for step in range(120):
        ids = rnd.sample(range(S), rnd.randint(1, S))
        r = rnd.random()
        just_evicted = set()
        if r < 0.45:
            ns = [rnd.choice([0, 1, 1, 2, 5, 16, rnd.randint(0, C)]) for _ in ids]
            try:
                exp = b.alloc(ids, ns)
            except NoSpace:
                before = _state(a)
                with pytest.raises(NoSpace):
                    a.alloc(ids, ns)
                assert _state(a) == before
                continue
            assert a.alloc(ids, ns) == exp
        elif r < 0.8:
            assert a.evict(ids) == b.evict(ids)
            just_evicted = set(ids)
        elif r < 0.86:
            # cut back by up to 4 positions (rejected drafts), sometimes far
            # below the resident window (refused, nothing changes)
            lens = [max(0, a.length[i] - rnd.choice([0, 1, 3, 4, W + 5])) for i in ids]
            try:
                b.truncate(ids, lens)
            except ValueError:
                before = _state(a)
                with pytest.raises(ValueError):
                    a.truncate(ids, lens)
                assert _state(a) == before
                continue
            a.truncate(ids, lens)
        elif r < 0.94:
            ns = [rnd.randint(0, 3 * W + 20) for _ in ids]
            try:
                exp = b.alloc(ids, ns, importing=True)
            except NoSpace:
                before = _state(a)
                with pytest.raises(NoSpace):
                    a.import_context(ids, ns)
                assert _state(a) == before
                continue
            assert a.import_context(ids, ns) == exp
            just_evicted = {i for i, n in zip(ids, ns) if n > 0}
        else:
            a.release(ids)
            b.release(ids)
        assert a.map_table() == b.map_table()
        assert a.free_pages() == b.free
        _check_invariants(a, just_evicted)
        for i in ids:
            m, tail = rnd.randint(0, a.length[i] + 3), rnd.choice([0, 1, W - 1, W, W + 2])
            assert a.window_safe_len(i, m, tail) == b.match(i, m, tail)


def test_decode_steps_evict_one_token_each():
    W, C = 8, 16
    p = PoolSim(W, C, 1, 64, 64, list(range(64)), [0])
    p.alloc([0], [3])
    assert p.evict([0])[1] == [0]
    counts = []
    for _ in range(40):
        p.alloc([0], [1])
        counts.append(p.evict([0])[1][0])
    # lengths 4..43: nothing evicted while L < W, then exactly one per step
    assert counts == [0] * (W - 4) + [1] * (40 - (W - 4))
    assert len(p.resident(0)) == W - 1


def test_rejects_invalid():
    with pytest.raises(ValueError):
        PoolSim(4, 8, 1, 4, 4, [0, 1, 2, 3], [0])        # ring not a multiple of 16
    with pytest.raises(ValueError):
        PoolSim(32, 16, 1, 4, 4, [0, 1, 2, 3], [0])      # ring smaller than window
    with pytest.raises(ValueError):
        PoolSim(4, 16, 1, 4, 4, [0, 1, 2, 2], [0])       # free order not a permutation
    p = PoolSim(4, 16, 2, 4, 4, [0, 1, 2, 3], [0, 1])
    with pytest.raises(ValueError):
        p.alloc([0, 0], [1, 1])
    with pytest.raises(ValueError):
        p.alloc([2], [1])
    with pytest.raises(ValueError):
        p.alloc([0], [-1])
    with pytest.raises(NoSpace):
        p.alloc([0], [17])                               # more than the ring holds
    with pytest.raises(NoSpace):
        p.import_context([0], [16 * 5])                  # more pages than a row holds
