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
        elif op["op"] == "fork":
            full_from, swa_from = p.fork(op["src"], op["dst"], op["m"])
            assert full_from == op["full_from"] and swa_from == op["swa_from"], op
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
        self.holders = {}                                 # physical page -> sequences

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
                    self.holders[self.page_of[b][pos // 16]] = {b}
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

    def _let_go(self, b, pg):
        self.holders[pg].discard(b)
        return not self.holders[pg]

    def release(self, ids):
        for b in ids:
            self.free += [self.page_of[b][i] for i in sorted(self.page_of[b])
                          if self._let_go(b, self.page_of[b][i])]
            self.page_of[b] = {}
            self.alive[b] = set()
            self.n[b] = 0

    def truncate(self, ids, lens):
        for b, n in zip(ids, lens):
            lo = min(self.alive[b]) if self.alive[b] else self.n[b]
            if n < 0 or n > self.n[b] or lo > max(0, n - self.W + 1):
                raise ValueError()
            # no page another sequence holds may lose or change positions
            if n < self.n[b] and any(len(self.holders[pg]) > 1 and (lp + 1) * 16 > n
                                     for lp, pg in self.page_of[b].items()):
                raise ValueError()
        for b, n in zip(ids, lens):
            self.alive[b] = {p for p in self.alive[b] if p < n}
            gone = sorted(lp for lp in self.page_of[b] if lp * 16 >= n)
            for lp in gone:
                self._let_go(b, self.page_of[b][lp])
            self.free = [self.page_of[b].pop(lp) for lp in gone] + self.free
            self.n[b] = n

    def fork(self, srcs, dsts, ms):
        if len(set(dsts)) != len(dsts) or set(srcs) & set(dsts):
            raise ValueError()
        fresh = 0
        for a, b, m in zip(srcs, dsts, ms):
            if self.n[b] != 0 or m > self.n[a] or self.match(a, m, self.W - 1) != m:
                raise ValueError()
            first_own = max(0, m - self.W + 1) // 16
            last = (m + 15) // 16
            if last > self.maxp:
                raise NoSpace()
            fresh += last - first_own
        if fresh > len(self.free):
            raise NoSpace()
        out = ([], [])
        for a, b, m in zip(srcs, dsts, ms):
            win = max(0, m - self.W + 1)
            for lp in range((m + 15) // 16):
                if (lp + 1) * 16 <= win:          # wholly below the window: shared
                    pg = self.page_of[a][lp]
                    self.holders[pg].add(b)
                else:
                    pg = self.free.pop(0)
                    self.holders[pg] = {b}
                self.page_of[b][lp] = pg
            self.alive[b] = set(range(win, m))
            self.n[b] = m
            out[0].append(16 * (win // 16))
            out[1].append(win)
        return out

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
            elif p.refs[p.pages[b][pos // 16]] == 1:
                assert m[fs] == -1   # (a shared page may carry another holder's entries)
        if b in just_evicted and L > 0:
            # every position the next query can see (its W-1 predecessors) is resident
            for pos in range(max(0, L - p.W + 1), L):
                assert m[p.full_slot(b, pos)] >= 0
    # map injective on resident tokens
    assert len(res_slots) == len(set(res_slots))
    # Full pages are conserved; a page's count is the number of sequences holding it
    used = {q for x in p.pages for q in x}
    assert len(used) + len(p.free) == p.num_full_pages
    assert len(used | set(p.free)) == p.num_full_pages
    holders = {}
    for x in p.pages:
        for q in x:
            holders[q] = holders.get(q, 0) + 1
    assert holders == p.refs
    # on a shared page at most one holder has resident positions, so every
    # map entry has one owner
    for q, n in p.refs.items():
        if n > 1:
            owners = [b for b in range(p.max_seqs) if q in p.pages[b] and any(
                p.pages[b][pos // 16] == q for pos in p.resident(b))]
            assert len(owners) <= 1


@pytest.mark.parametrize("seed", range(16))
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
        elif r < 0.98:
            # fork a window-safe prefix of one sequence into an empty one
            empty = [i for i in range(S) if a.length[i] == 0]
            src = rnd.randrange(S)
            dsts = [i for i in empty if i != src]
            if not dsts or a.length[src] == 0:
                continue
            dst = rnd.choice(dsts)
            want = rnd.randint(1, a.length[src])
            m = rnd.choice([a.window_safe_len(src, want, W - 1), want])
            if m == 0:
                continue
            try:
                exp = b.fork([src], [dst], [m])
            except (ValueError, NoSpace) as e:
                before = _state(a)
                with pytest.raises(type(e)):
                    a.fork([src], [dst], [m])
                assert _state(a) == before
                continue
            assert a.fork([src], [dst], [m]) == exp
        else:
            a.release(ids)
            b.release(ids)
        assert a.map_table() == b.map_table()
        assert a.free_pages() == b.free
        _check_invariants(a, just_evicted)
        for i in ids:
            m, tail = rnd.randint(0, a.length[i] + 3), rnd.choice([0, 1, W - 1, W, W + 2])
            assert a.window_safe_len(i, m, tail) == b.match(i, m, tail)


def _fork_sequence(seed, stats):
    """Seeded operations with forks about a quarter of the time: short
    windows and roomy page budgets, so forks share pages and forks of forks
    share further."""
    rnd = random.Random(1000 + seed)
    W = rnd.choice([1, 2, 5, 16, 20, 33])
    C = 16 * rnd.randint(max(1, -(-W // 16)), max(1, -(-W // 16)) + 2)
    S = rnd.randint(3, 6)
    maxp = rnd.randint(6, 16)
    npages = rnd.randint(S * maxp // 2, S * maxp)
    free_order = list(range(npages))
    rnd.shuffle(free_order)
    ring = list(range(S * C // 16))
    rnd.shuffle(ring)
    a = PoolSim(W, C, S, maxp, npages, free_order, ring)
    b = DictPool(W, C, S, maxp, npages, free_order, ring)
    for step in range(150):
        r = rnd.random()
        just_evicted = set()
        if r < 0.25:
            src = rnd.randrange(S)
            empty = [i for i in range(S) if a.length[i] == 0 and i != src]
            if not empty or a.length[src] == 0:
                continue
            dst = rnd.choice(empty)
            want = rnd.randint(1, a.length[src])
            m = rnd.choice([a.window_safe_len(src, want, W - 1)] * 3 + [want])
            if m == 0:
                continue
            try:
                exp = b.fork([src], [dst], [m])
            except (ValueError, NoSpace) as e:
                before = _state(a)
                with pytest.raises(type(e)):
                    a.fork([src], [dst], [m])
                assert _state(a) == before
                continue
            was_shared = a.refs.get(a.pages[src][0], 0) > 1 if a.pages[src] else False
            assert a.fork([src], [dst], [m]) == exp
            stats["forks"] += 1
            stats["shared"] += exp[0][0] > 0
            stats["chained"] += was_shared and exp[0][0] > 0
        elif r < 0.5:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            ns = [rnd.choice([0, 1, 3, 16, 30]) for _ in ids]
            try:
                exp = b.alloc(ids, ns)
            except NoSpace:
                with pytest.raises(NoSpace):
                    a.alloc(ids, ns)
                continue
            assert a.alloc(ids, ns) == exp
        elif r < 0.7:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            assert a.evict(ids) == b.evict(ids)
            just_evicted = set(ids)
        elif r < 0.8:
            ids = rnd.sample(range(S), rnd.randint(1, S))
            ns = [rnd.randint(0, 2 * W + 40) for _ in ids]
            try:
                exp = b.alloc(ids, ns, importing=True)
            except NoSpace:
                with pytest.raises(NoSpace):
                    a.import_context(ids, ns)
                continue
            assert a.import_context(ids, ns) == exp
            just_evicted = {i for i, n in zip(ids, ns) if n > 0}
        elif r < 0.9:
            ids = rnd.sample(range(S), 1)
            lens = [max(0, a.length[ids[0]] - rnd.choice([1, 2, 17, 40, 100]))]
            try:
                b.truncate(ids, lens)
            except ValueError:
                before = _state(a)
                with pytest.raises(ValueError):
                    a.truncate(ids, lens)
                assert _state(a) == before
                continue
            a.truncate(ids, lens)
        else:
            ids = rnd.sample(range(S), rnd.randint(1, 2))
            a.release(ids)
            b.release(ids)
        assert a.map_table() == b.map_table()
        assert a.free_pages() == b.free
        _check_invariants(a, just_evicted)
        for i in range(S):
            m, tail = rnd.randint(0, a.length[i] + 3), rnd.choice([0, 1, W - 1, W])
            assert a.window_safe_len(i, m, tail) == b.match(i, m, tail)


def test_random_forks_against_second_simulator():
    stats = {"forks": 0, "shared": 0, "chained": 0}
    for seed in range(24):
        _fork_sequence(seed, stats)
    # the sequences exercised what they are for
    assert stats["forks"] >= 100 and stats["shared"] >= 30 and stats["chained"] >= 3, stats


@pytest.mark.parametrize("seed", range(8))
def test_cut_into_shared_page_refused(seed):
    """A source that was never evicted is forked; cutting it to a length the
    window rule allows but that reaches a shared page is refused (a later
    append would overwrite the fork's K/V), in both simulators, with nothing
    changed; a cut that keeps the shared pages whole is allowed."""
    rnd = random.Random(2000 + seed)
    W = rnd.choice([1, 2, 3, 5, 9])
    C = 16 * rnd.randint(3, 5)
    free_order = list(range(24))
    rnd.shuffle(free_order)
    a = PoolSim(W, C, 2, 8, 24, free_order, list(range(2 * C // 16)))
    b = DictPool(W, C, 2, 8, 24, free_order, list(range(2 * C // 16)))
    L = rnd.randint(W + 16, C)
    assert a.alloc([0], [L]) == b.alloc([0], [L])
    m = rnd.randint(W + 15, L)
    assert a.fork([0], [1], [m]) == b.fork([0], [1], [m])
    sh = a.shared_pages(0)
    assert sh == (m - W + 1) // 16 >= 1
    n = rnd.randrange(W - 1, 16 * sh)
    before = _state(a)
    with pytest.raises(ValueError):
        b.truncate([0], [n])
    with pytest.raises(ValueError):
        a.truncate([0], [n])
    assert _state(a) == before
    n = rnd.randint(16 * sh, L)
    a.truncate([0], [n])
    b.truncate([0], [n])
    assert a.map_table() == b.map_table() and a.free_pages() == b.free
    _check_invariants(a, set())


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
