"""Dual KV pool bookkeeping as a plain Python simulator (integers, exact).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (MiMo-V2.5 inference page, section 2.1 "KVCache Dual
Pool"):

* Two physical pools: the Full pool grows with the sequence, O(N); the SWA
  pool is sized by the window only, O(W), and is evicted on its own.
* One logical sequence view: the Full index is authoritative and a map from
  Full slots to SWA slots is kept beside it.
* On admission both capacities are checked together, so neither pool is
  over-committed because only one was looked at.
* "SWA-aware prefix cache tree", point 2: each finished prefill chunk, each
  finished request and decode progress release the SWA entries that have left
  the window, so SWA occupancy stays at window (or chunk) scale.

The vLLM MI355X post (section 3, "Which bytes move?") addresses KV through
16-token pages and a per-sequence page table; that is the Full pool layout.

Readings taken where the pages leave a step open:

* Page size P = 16.  A sequence's position ``pos`` lives in Full slot
  ``fpt[b][pos // P] * P + pos % P``.  A new Full page is taken from the
  head of a FIFO free list when the first position of that page is
  allocated; sequences are served in the order listed, positions ascending.
* The SWA pool of a sequence is a ring of C slots made of C/P pages fixed at
  creation: position ``pos`` lives in SWA slot
  ``rpt[b][(pos mod C) // P] * P + (pos mod C) % P``.
* Eviction after a sequence reaches length L releases every resident
  position <= L - W, so exactly the last min(L, W-1) positions stay resident
  -- what the next query (which sees W keys counting itself) needs.
* Admission of n new tokens for sequence b needs resident_b + n <= C in the
  ring and enough free Full pages for all listed sequences together; on
  failure nothing changes.
* ``import_context`` appends n positions whose K/V the caller writes
  directly (restoring a cached context): every position gets a Full slot,
  only the positions left inside the window get SWA slots, and positions that
  leave the window are evicted at once.  Only the in-window SWA part moves,
  as section 2.1 "Data Transfer" asks for transfers.
* ``release`` ends a request: its Full pages go back to the tail of the free
  list in logical-page order and its remaining SWA entries are dropped.
* ``truncate`` drops a sequence's newest positions, e.g. draft tokens that a
  multi-token (MTP) verification step rejected (section 5.2 of the page runs
  three MTP layers, so a step appends up to four tokens).  The window of the
  new length must still be resident, so it runs before the step's eviction.
  Dropped positions lose their SWA entry; Full pages that no longer hold a
  position go back to the head of the free list, lowest logical page first,
  so the next allocation takes them again.
* ``window_safe_len`` is the prefix-match rule of "SWA-aware prefix cache
  tree", point 1: a match of m tokens is usable only as far as the last
  ``tail`` tokens before its end still hold valid SWA slots (map >= 0); the
  match is cut back to the longest such length, the rest is a miss.  The
  page asks for W tail tokens.  The next query at position m' attends to
  [m' - W + 1, m'], so this library's attention needs W - 1 of them, which
  is also what eviction keeps; the caller chooses ``tail``.  A position of
  a sequence holds an SWA entry of that sequence only from its first
  resident position on (a page shared with another sequence may carry the
  other one's entries).
* ``fork`` reuses a matched prefix for another request (point 3 of the same
  part: a prefix node keeps a Full segment index and an SWA segment map, so
  the Full part stays shareable whatever happens to the SWA part).  An
  empty sequence dst takes the first m positions of src, m window-safe for
  src with tail W - 1.  The Full pages wholly below dst's window start
  max(0, m - W + 1) are shared (a reference count per page); the pages from
  the one holding that start to the one holding m - 1 are fresh (taken from
  the free-list head, logical order), and the window positions get dst's
  ring slots.  Every map entry so keeps one owner: shared positions are
  outside dst's window for good, and its window sits on its own pages.  The
  caller copies the K/V of [16 * first fresh page, m) (Full layers) and of
  the window (SWA layers) from src to dst.  Not enough free pages: NoSpace,
  nothing changed.  A sequence's pages are freed when the last sequence
  holding them releases them; truncating into a shared page (which a later
  append would overwrite under the other holder) is refused.
* -1 marks "no slot" in every table.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Sequence, Tuple

PAGE = 16


class NoSpace(Exception):
    """The joint Full/SWA capacity check failed; the pool is unchanged."""


class PoolSim:
    def __init__(self, window: int, ring_slots: int, max_seqs: int,
                 max_pages_per_seq: int, num_full_pages: int,
                 free_order: Sequence[int], ring_pages: Sequence[int],
                 page_size: int = PAGE):
        if page_size != PAGE:
            raise ValueError("page size must be 16")
        if window < 1:
            raise ValueError("window must be >= 1")
        if ring_slots % PAGE != 0 or ring_slots < window:
            raise ValueError("ring slots must be a multiple of 16 and >= window")
        if max_seqs < 1 or max_pages_per_seq < 1 or num_full_pages < 1:
            raise ValueError("sizes must be positive")
        if sorted(int(x) for x in free_order) != list(range(num_full_pages)):
            raise ValueError("free order must be a permutation of the Full pages")
        rp = ring_slots // PAGE
        if sorted(int(x) for x in ring_pages) != list(range(max_seqs * rp)):
            raise ValueError("ring pages must be a permutation of the ring pool pages")
        self.W = int(window)
        self.C = int(ring_slots)
        self.max_seqs = int(max_seqs)
        self.max_pages = int(max_pages_per_seq)
        self.num_full_pages = int(num_full_pages)
        self.free = deque(int(x) for x in free_order)
        self.ring = [[int(x) for x in ring_pages[b * rp:(b + 1) * rp]]
                     for b in range(max_seqs)]
        self.length = [0] * max_seqs      # tokens stored for the sequence
        self.res_start = [0] * max_seqs   # first position still in the SWA pool
        self.pages: List[List[int]] = [[] for _ in range(max_seqs)]
        self.map: Dict[int, int] = {}     # Full slot -> SWA slot, resident only
        self.refs: Dict[int, int] = {}    # Full page -> sequences holding it

    # -- slot formulas --------------------------------------------------
    def full_slot(self, b: int, pos: int) -> int:
        return self.pages[b][pos // PAGE] * PAGE + pos % PAGE

    def swa_slot(self, b: int, pos: int) -> int:
        r = pos % self.C
        return self.ring[b][r // PAGE] * PAGE + r % PAGE

    # -- helpers ----------------------------------------------------------
    def _check_ids(self, seq_ids, counts=None):
        ids = [int(b) for b in seq_ids]
        if len(set(ids)) != len(ids):
            raise ValueError("a sequence may be listed once per call")
        for b in ids:
            if not 0 <= b < self.max_seqs:
                raise ValueError("sequence id out of range")
        if counts is not None:
            if len(counts) != len(ids):
                raise ValueError("one count per sequence")
            for n in counts:
                if int(n) < 0:
                    raise ValueError("negative token count")
        return ids

    @staticmethod
    def _pages_for(length: int) -> int:
        return -(-length // PAGE)

    def _pages_needed(self, ids, counts) -> int:
        total = 0
        for b, n in zip(ids, counts):
            L = self.length[b]
            need = self._pages_for(L + int(n))
            if need > self.max_pages:
                raise NoSpace("sequence would exceed its page-table row")
            total += need - self._pages_for(L)
        return total

    # -- operations -----------------------------------------------------
    def alloc(self, seq_ids, n_new) -> Tuple[List[int], List[int]]:
        """Give Full and SWA slots to n_new[i] new positions of seq_ids[i]."""
        ids = self._check_ids(seq_ids, n_new)
        counts = [int(n) for n in n_new]
        if self._pages_needed(ids, counts) > len(self.free):
            raise NoSpace("Full pool exhausted")
        for b, n in zip(ids, counts):
            if (self.length[b] - self.res_start[b]) + n > self.C:
                raise NoSpace("SWA ring exhausted")
        full_out, swa_out = [], []
        for b, n in zip(ids, counts):
            L = self.length[b]
            for pos in range(L, L + n):
                if pos % PAGE == 0:
                    self._take_page(b)
                fs, ss = self.full_slot(b, pos), self.swa_slot(b, pos)
                self.map[fs] = ss
                full_out.append(fs)
                swa_out.append(ss)
            self.length[b] = L + n
        return full_out, swa_out

    def evict(self, seq_ids) -> Tuple[List[int], List[int]]:
        """Release every resident position that has left the window.

        Returns the Full slots whose SWA entry was released (ascending
        position per sequence, sequences in the order listed) and the count
        per sequence.
        """
        ids = self._check_ids(seq_ids)
        out, counts = [], []
        for b in ids:
            keep_from = max(0, self.length[b] - self.W + 1)
            n = 0
            for pos in range(self.res_start[b], keep_from):
                fs = self.full_slot(b, pos)
                del self.map[fs]
                out.append(fs)
                n += 1
            self.res_start[b] = max(self.res_start[b], keep_from)
            counts.append(n)
        return out, counts

    def import_context(self, seq_ids, n_new) -> Tuple[List[int], List[int]]:
        """Append positions whose K/V the caller stores directly.

        Full slots for every new position; SWA slots (else -1) only for
        positions inside the window of the new length.  Resident positions
        that leave the window are dropped as ``evict`` would.
        """
        ids = self._check_ids(seq_ids, n_new)
        counts = [int(n) for n in n_new]
        if self._pages_needed(ids, counts) > len(self.free):
            raise NoSpace("Full pool exhausted")
        full_out, swa_out = [], []
        for b, n in zip(ids, counts):
            L = self.length[b]
            new_len = L + n
            keep_from = max(0, new_len - self.W + 1)
            for pos in range(self.res_start[b], min(keep_from, L)):
                del self.map[self.full_slot(b, pos)]
            self.res_start[b] = max(self.res_start[b], keep_from)
            for pos in range(L, new_len):
                if pos % PAGE == 0:
                    self._take_page(b)
                fs = self.full_slot(b, pos)
                full_out.append(fs)
                if pos >= keep_from:
                    ss = self.swa_slot(b, pos)
                    self.map[fs] = ss
                    swa_out.append(ss)
                else:
                    swa_out.append(-1)
            self.length[b] = new_len
        return full_out, swa_out

    def _take_page(self, b: int) -> None:
        pg = self.free.popleft()
        self.refs[pg] = 1
        self.pages[b].append(pg)

    def _drop_page(self, pg: int) -> bool:
        """One holder lets go of a page; True when it is free again."""
        self.refs[pg] -= 1
        if self.refs[pg] == 0:
            del self.refs[pg]
            return True
        return False

    def shared_pages(self, b: int) -> int:
        """Leading pages of b that another sequence also holds."""
        n = 0
        while n < len(self.pages[b]) and self.refs[self.pages[b][n]] > 1:
            n += 1
        return n

    def release(self, seq_ids) -> None:
        """End the listed requests: drop their SWA entries and their hold on
        their Full pages; pages no other sequence holds go back to the tail
        of the free list in logical-page order."""
        ids = self._check_ids(seq_ids)
        for b in ids:
            for pos in range(self.res_start[b], self.length[b]):
                del self.map[self.full_slot(b, pos)]
            self.free.extend(pg for pg in self.pages[b] if self._drop_page(pg))
            self.pages[b] = []
            self.length[b] = 0
            self.res_start[b] = 0

    def truncate(self, seq_ids, new_lens) -> None:
        """Cut sequence seq_ids[i] back to new_lens[i] positions."""
        ids = self._check_ids(seq_ids)
        lens = [int(x) for x in new_lens]
        if len(lens) != len(ids):
            raise ValueError("one new length per sequence")
        for b, n in zip(ids, lens):
            if not 0 <= n <= self.length[b]:
                raise ValueError("new length outside [0, current length]")
            if self.res_start[b] > max(0, n - self.W + 1):
                raise ValueError("the window of the new length was already evicted")
            if n < self.length[b] and n < PAGE * self.shared_pages(b):
                raise ValueError("the cut reaches a page another sequence holds")
        for b, n in zip(ids, lens):
            for pos in range(n, self.length[b]):
                del self.map[self.full_slot(b, pos)]
            keep = self._pages_for(n)
            freed = self.pages[b][keep:]
            for pg in freed:
                self._drop_page(pg)
            self.pages[b] = self.pages[b][:keep]
            self.free.extendleft(reversed(freed))
            self.length[b] = n

    def fork(self, src_ids, dst_ids, lens) -> Tuple[List[int], List[int]]:
        """Give each empty dst_ids[i] the first lens[i] positions of
        src_ids[i] (see the module docstring).  Returns, per fork, the first
        position whose Full-layer K/V the caller copies and the first
        position whose SWA-layer K/V it copies (both up to lens[i])."""
        dsts = self._check_ids(dst_ids, lens)
        srcs = [int(b) for b in src_ids]
        ms = [int(m) for m in lens]
        if len(srcs) != len(dsts):
            raise ValueError("one source per fork")
        for a, b, m in zip(srcs, dsts, ms):
            if not 0 <= a < self.max_seqs or a in dsts:
                raise ValueError("source out of range or also a destination")
            if self.length[b] != 0:
                raise ValueError("a fork's destination must be empty")
            if m > self.length[a]:
                raise ValueError("fork longer than its source")
            if self.window_safe_len(a, m, self.W - 1) != m:
                raise ValueError("fork length is not window-safe for its source")
        need = 0
        for a, b, m in zip(srcs, dsts, ms):
            own = max(0, m - self.W + 1) // PAGE
            if self._pages_for(m) > self.max_pages:
                raise NoSpace("fork would exceed its page-table row")
            need += self._pages_for(m) - own
        if need > len(self.free):
            raise NoSpace("Full pool exhausted")
        full_from, swa_from = [], []
        for a, b, m in zip(srcs, dsts, ms):
            start = max(0, m - self.W + 1)
            own = start // PAGE
            for pg in self.pages[a][:own]:
                self.refs[pg] += 1
                self.pages[b].append(pg)
            for _ in range(own, self._pages_for(m)):
                self._take_page(b)
            for pos in range(start, m):
                self.map[self.full_slot(b, pos)] = self.swa_slot(b, pos)
            self.length[b] = m
            self.res_start[b] = start
            full_from.append(PAGE * own)
            swa_from.append(start)
        return full_from, swa_from

    def window_safe_len(self, b: int, m: int, tail: int) -> int:
        """Longest m' <= min(m, length) whose last min(m', tail) positions all
        have an SWA entry (0 if none)."""
        if not 0 <= b < self.max_seqs:
            raise ValueError("sequence id out of range")
        if m < 0 or tail < 0:
            raise ValueError("negative length")
        for k in range(min(m, self.length[b]), 0, -1):
            if all(pos >= self.res_start[b] and self.full_slot(b, pos) in self.map
                   for pos in range(max(0, k - tail), k)):
                return k
        return 0

    # -- table views (what the device tables must hold) ---------------------
    def seq_len_table(self) -> List[int]:
        return list(self.length)

    def fpt_table(self) -> List[List[int]]:
        return [p + [-1] * (self.max_pages - len(p)) for p in self.pages]

    def rpt_table(self) -> List[List[int]]:
        return [list(r) for r in self.ring]

    def map_table(self) -> List[int]:
        t = [-1] * (self.num_full_pages * PAGE)
        for fs, ss in self.map.items():
            t[fs] = ss
        return t

    def resident(self, b: int) -> range:
        return range(self.res_start[b], self.length[b])

    def free_pages(self) -> List[int]:
        return list(self.free)
