"""C ABI checks that need no GPU: the library loads and exports every
declared symbol; the host pool bookkeeping is bit-exact against the oracle
simulator; argument validation rejects bad calls before any launch."""
import copy
import ctypes as C
import json
import os
import random
import re

import numpy as np
import pytest

import hybrid_sliding_window_hswa_amd as H
from hybrid_sliding_window_hswa_amd import _capi
from oracle.pool import NoSpace, PoolSim

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def test_header_symbols_are_exported():
    hdr = open(os.path.join(ROOT, "include", "hswa.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"\b(hswa_[a-z_]+)\s*\(", hdr))
    assert names == set(_capi.EXPORTED)
    lib = _capi.load()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert H.hswa_version() >= 100
    lib = _capi.load()
    assert lib.hswa_status_string(-2) == b"HSWA_E_NOSPC"
    assert lib.hswa_status_string(0) == b"HSWA_OK"


def _host_pool(W, C_, S, maxp, npages, free, ring):
    return H.hswa_pool_create(W, C_, S, maxp, npages, free, ring)


def _tables(p):
    t = H.hswa_pool_read_tables(p)
    return t["seq_len"].tolist(), t["fpt"].tolist(), t["map"].tolist(), t["free"].tolist()


def test_golden_fixtures_through_the_abi():
    data = json.load(open(os.path.join(GOLDEN, "pool_small.json")))
    for sc in data["scenarios"]:
        c = sc["create"]
        p = _host_pool(c["window"], c["ring_slots"], c["max_seqs"], c["max_pages_per_seq"],
                       c["num_full_pages"], c["free_order"], c["ring_pages"])
        for op in sc["ops"]:
            if op["op"] in ("alloc", "import"):
                fn = H.hswa_pool_alloc if op["op"] == "alloc" else H.hswa_pool_import
                if op.get("nospace"):
                    before = _tables(p)
                    with pytest.raises(H.NoSpace):
                        fn(p, op["seq_ids"], op["n"])
                    assert _tables(p) == before
                else:
                    full, swa = fn(p, op["seq_ids"], op["n"])
                    assert full.tolist() == op["full"] and swa.tolist() == op["swa"]
            elif op["op"] == "evict":
                ev, cnt = H.hswa_pool_evict(p, op["seq_ids"])
                assert ev.tolist() == op["evicted"] and cnt.tolist() == op["counts"]
            elif op["op"] == "truncate":
                if op.get("invalid"):
                    before = _tables(p)
                    with pytest.raises(H.HswaError) as e:
                        H.hswa_pool_truncate(p, op["seq_ids"], op["new_len"])
                    assert e.value.status == H.HSWA_E_INVAL
                    assert _tables(p) == before
                else:
                    H.hswa_pool_truncate(p, op["seq_ids"], op["new_len"])
            elif op["op"] == "release":
                H.hswa_pool_release(p, op["seq_ids"])
            elif op["op"] == "fork":
                ff, sf = H.hswa_pool_fork(p, op["src"], op["dst"], op["m"])
                assert ff.tolist() == op["full_from"] and sf.tolist() == op["swa_from"], op
            elif op["op"] == "match":
                got = H.hswa_pool_match_len(p, [op["seq"]], [op["m"]], op["tail"])
                assert got.tolist() == [op["expect"]], op
            else:
                raise AssertionError(f"unknown fixture op {op['op']}")
        seq_len, fpt, mp, free = _tables(p)
        f = sc["final"]
        assert seq_len == f["seq_len"] and fpt == f["fpt"] and free == f["free"]
        assert {str(i): s for i, s in enumerate(mp) if s >= 0} == f["map_nonneg"]


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_bit_exact_vs_oracle(seed):
    rnd = random.Random(1000 + seed)
    W = rnd.choice([1, 3, 16, 64, 128])
    C_ = 16 * rnd.randint(-(-W // 16), -(-W // 16) + 4)
    S = rnd.randint(1, 6)
    maxp = rnd.randint(2, 20)
    npages = rnd.randint(4, S * maxp)
    free = list(range(npages))
    rnd.shuffle(free)
    ring = list(range(S * C_ // 16))
    rnd.shuffle(ring)
    p = _host_pool(W, C_, S, maxp, npages, free, ring)
    sim = PoolSim(W, C_, S, maxp, npages, free, ring)
    for _ in range(150):
        ids = rnd.sample(range(S), rnd.randint(1, S))
        r = rnd.random()
        if rnd.random() < 0.15:
            # a chunk-step boundary: evict one set, then alloc another, as
            # one operation; on failure neither part may change anything
            ev_ids = rnd.sample(range(S), rnd.randint(0, S))
            n = [rnd.choice([0, 1, 2, 7, 16, rnd.randint(0, 2 * C_)]) for _ in ids]
            snap = copy.deepcopy(sim)
            try:
                e_ev = sim.evict(ev_ids)
                e_al = sim.alloc(ids, n)
            except NoSpace:
                sim = snap
                before = _tables(p)
                with pytest.raises(H.NoSpace):
                    H.hswa_pool_evict_alloc(p, ev_ids, ids, n)
                assert _tables(p) == before
                continue
            ev, cnt, full, swa = H.hswa_pool_evict_alloc(p, ev_ids, ids, n)
            assert ev.tolist() == e_ev[0] and cnt.tolist() == e_ev[1]
            assert full.tolist() == e_al[0] and swa.tolist() == e_al[1]
        elif r < 0.45 or r >= 0.8 and r < 0.9:
            imp = r >= 0.8
            n = [rnd.choice([0, 1, 2, 7, 16, rnd.randint(0, 2 * C_)]) for _ in ids]
            fn_sim = sim.import_context if imp else sim.alloc
            fn = H.hswa_pool_import if imp else H.hswa_pool_alloc
            try:
                exp = fn_sim(ids, n)
            except NoSpace:
                before = _tables(p)
                with pytest.raises(H.NoSpace):
                    fn(p, ids, n)
                assert _tables(p) == before
                continue
            full, swa = fn(p, ids, n)
            assert full.tolist() == exp[0] and swa.tolist() == exp[1]
        elif r < 0.8:
            exp = sim.evict(ids)
            ev, cnt = H.hswa_pool_evict(p, ids)
            assert ev.tolist() == exp[0] and cnt.tolist() == exp[1]
        elif r < 0.93:
            # fork a (mostly window-safe) prefix into empty sequences
            empty = [i for i in range(S) if sim.length[i] == 0]
            full_seqs = [i for i in range(S) if sim.length[i] > 0]
            if not empty or not full_seqs:
                continue
            dst = rnd.sample(empty, rnd.randint(1, len(empty)))
            src = [rnd.choice(full_seqs) for _ in dst]
            want = [rnd.randint(0, sim.length[a]) for a in src]
            m = [rnd.choice([sim.window_safe_len(a, w, W - 1)] * 3 + [w])
                 for a, w in zip(src, want)]
            try:
                exp = sim.fork(src, dst, m)
            except (ValueError, NoSpace) as err:
                before = _tables(p)
                with pytest.raises(H.NoSpace if isinstance(err, NoSpace) else H.HswaError) as e:
                    H.hswa_pool_fork(p, src, dst, m)
                if not isinstance(err, NoSpace):
                    assert e.value.status == H.HSWA_E_INVAL
                assert _tables(p) == before
                continue
            ff, sf = H.hswa_pool_fork(p, src, dst, m)
            assert ff.tolist() == exp[0] and sf.tolist() == exp[1]
        elif r < 0.96:
            lens = [max(0, sim.length[i] - rnd.choice([0, 1, 2, 3, 17, W + 1])) for i in ids]
            try:
                sim.truncate(ids, lens)
            except ValueError:
                before = _tables(p)
                with pytest.raises(H.HswaError) as e:
                    H.hswa_pool_truncate(p, ids, lens)
                assert e.value.status == H.HSWA_E_INVAL
                assert _tables(p) == before
                continue
            H.hswa_pool_truncate(p, ids, lens)
        else:
            sim.release(ids)
            H.hswa_pool_release(p, ids)
        mids = list(range(S))
        want = [rnd.randint(0, sim.length[i] + 5) for i in mids]
        tail = rnd.choice([0, 1, W - 1, W, 2 * W])
        assert H.hswa_pool_match_len(p, mids, want, tail).tolist() == \
            [sim.window_safe_len(i, m, tail) for i, m in zip(mids, want)]
        seq_len, fpt, mp, fr = _tables(p)
        assert seq_len == sim.seq_len_table()
        assert fpt == sim.fpt_table()
        assert mp == sim.map_table()
        assert fr == sim.free_pages()


def test_evict_alloc_validation():
    """The alloc's ring check counts the eviction that comes first; a failed
    check changes nothing (not even the eviction); each list rejects repeats
    but a sequence may be in both."""
    p = _host_pool(8, 16, 2, 8, 16, list(range(16)), [0, 1])
    sim = PoolSim(8, 16, 2, 8, 16, list(range(16)), [0, 1])
    H.hswa_pool_alloc(p, [0, 1], [16, 5])
    sim.alloc([0, 1], [16, 5])
    # alone, 9 more positions overflow sequence 0's ring (16 resident + 9 > 16)
    before = _tables(p)
    with pytest.raises(H.NoSpace):
        H.hswa_pool_alloc(p, [0], [9])
    # after the eviction 7 stay resident: 7 + 10 > 16 still fails, and the
    # eviction is not applied either
    with pytest.raises(H.NoSpace):
        H.hswa_pool_evict_alloc(p, [0, 1], [0], [10])
    assert _tables(p) == before
    for bad in (([0, 0], [1], [1]), ([0], [1, 1], [1, 1]), ([2], [0], [1]), ([0], [0], [-1])):
        with pytest.raises(H.HswaError) as e:
            H.hswa_pool_evict_alloc(p, *bad)
        assert e.value.status == H.HSWA_E_INVAL
        assert _tables(p) == before
    with pytest.raises(H.HswaError):
        H.hswa_pool_evict_alloc(p, [0], [0], [9], capacity=3)   # evicted_out too small
    assert _tables(p) == before
    # 7 + 9 = 16 fits once the eviction comes first
    ev, cnt, full, swa = H.hswa_pool_evict_alloc(p, [0, 1], [0], [9])
    e_ev = sim.evict([0, 1])
    e_al = sim.alloc([0], [9])
    assert ev.tolist() == e_ev[0] and cnt.tolist() == e_ev[1] == [9, 0]
    assert full.tolist() == e_al[0] and swa.tolist() == e_al[1]
    seq_len, fpt, mp, fr = _tables(p)
    assert (seq_len, fpt, mp, fr) == (sim.seq_len_table(), sim.fpt_table(), sim.map_table(),
                                      sim.free_pages())


def test_pool_create_rejects_bad_descriptions():
    with pytest.raises(H.HswaError):
        _host_pool(0, 16, 1, 4, 4, [0, 1, 2, 3], [0])
    with pytest.raises(H.HswaError):
        _host_pool(32, 16, 1, 4, 4, [0, 1, 2, 3], [0])          # ring < window
    with pytest.raises(H.HswaError):
        _host_pool(8, 24, 1, 4, 4, [0, 1, 2, 3], [0])           # ring % 16
    with pytest.raises(H.HswaError):
        _host_pool(8, 16, 1, 4, 4, [0, 1, 1, 3], [0])           # free order
    with pytest.raises(H.HswaError):
        _host_pool(8, 32, 1, 4, 4, [0, 1, 2, 3], [0, 0])        # ring pages


def test_pool_op_validation():
    p = _host_pool(8, 16, 2, 4, 8, list(range(8)), [0, 1])
    with pytest.raises(H.HswaError) as e:
        H.hswa_pool_alloc(p, [0, 0], [1, 1])
    assert e.value.status == H.HSWA_E_INVAL
    with pytest.raises(H.HswaError):
        H.hswa_pool_alloc(p, [2], [1])
    with pytest.raises(H.HswaError):
        H.hswa_pool_alloc(p, [0], [-1])
    with pytest.raises(H.NoSpace):
        H.hswa_pool_alloc(p, [0], [17])
    H.hswa_pool_alloc(p, [0], [16])
    # evicted_out too small: error and nothing changes
    before = _tables(p)
    with pytest.raises(H.HswaError):
        H.hswa_pool_evict(p, [0], capacity=3)
    assert _tables(p) == before
    ev, cnt = H.hswa_pool_evict(p, [0])
    assert cnt.tolist() == [9] and len(ev) == 9


def _args(**kw):
    a = _capi.AttnArgs()
    a.kind = kw.get("kind", 1)
    a.window = kw.get("window", 16)
    a.num_q_heads = kw.get("hq", 8)
    a.num_kv_heads = kw.get("hkv", 2)
    a.head_dim = kw.get("d", 64)
    a.num_seqs = kw.get("n", 1)
    a.total_q = kw.get("total_q", 1)
    a.max_q_len = kw.get("max_q_len", 1)
    a.max_seq_len = kw.get("max_seq_len", 100)
    fake = 1 << 20  # never dereferenced: every case below fails validation
    a.seq_ids = a.cu_q = a.q = a.k_cache = a.v_cache = a.out = fake
    a.pool.seq_len = a.pool.fpt = a.pool.rpt = a.pool.map = fake
    a.pool.max_seqs, a.pool.max_pages_per_seq = 4, 4
    a.pool.ring_slots, a.pool.window = kw.get("ring", 32), kw.get("pool_window", 16)
    for k, v in kw.items():
        if hasattr(a, k):
            setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=96), H.HSWA_E_INVAL),
    (dict(hq=12, hkv=8), H.HSWA_E_INVAL),
    (dict(hq=32, hkv=2), H.HSWA_E_UNSUPPORTED),
    (dict(hq=2048, hkv=2048), H.HSWA_E_INVAL),  # above the KV head cap
    (dict(kind=5), H.HSWA_E_INVAL),
    (dict(window=32), H.HSWA_E_INVAL),        # above the pool window
    (dict(window=0), H.HSWA_E_INVAL),
    (dict(ring=24), H.HSWA_E_INVAL),
    (dict(q=(1 << 20) + 4), H.HSWA_E_INVAL),  # misaligned
    (dict(cu_q=None), H.HSWA_E_INVAL),
])
def test_prefill_validation(bad, code):
    a = _args(**bad)
    rc = _capi.load().hswa_prefill_chunk(C.byref(a), None)
    assert rc == code
    assert H.hswa_last_error() != ""


def test_decode_validation_and_workspace():
    lib = _capi.load()
    a = _args(total_q=2, n=1)
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    # Full layer with a long context needs a workspace; too small is rejected
    a = _args(kind=0, n=4, total_q=4, hq=64, hkv=8, d=128, max_seq_len=100000)
    need = lib.hswa_decode_workspace_bytes(C.byref(a))
    assert need > 0
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    # SWA layers never need one
    a = _args(kind=1, n=4, total_q=4)
    assert lib.hswa_decode_workspace_bytes(C.byref(a)) == 0


def test_multi_row_decode_validation_and_workspace():
    lib = _capi.load()
    # more than four rows per sequence is outside what is built
    a = _args(n=2, total_q=10, max_q_len=5)
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_UNSUPPORTED
    # rows must fit num_seqs * max_q_len; max_q_len >= 1
    a = _args(n=2, total_q=9, max_q_len=4)
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    a = _args(n=2, total_q=2, max_q_len=0)
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    # the split-K workspace holds one partial state per (row, head, split),
    # then (256-byte aligned) the work queues: 8 counters of a 128-byte line,
    # the unit count and a list of up to num_seqs * splits units.  Here 4
    # sequences x 8 KV heads aim at 2,048 work items with pieces of at least
    # 1,024 keys: 63 splits of 1,600 keys for 100,000.
    one = _args(kind=0, n=4, total_q=4, hq=64, hkv=8, d=128, max_seq_len=100000)
    four = _args(kind=0, n=4, total_q=16, max_q_len=4, hq=64, hkv=8, d=128,
                 max_seq_len=100000)
    b1 = lib.hswa_decode_workspace_bytes(C.byref(one))
    b4 = lib.hswa_decode_workspace_bytes(C.byref(four))

    def ws(rows, seqs=4, splits=63):
        partial = rows * 64 * splits * (128 + 2) * 4
        return -(-partial // 256) * 256 + (8 * 32 + 32 + seqs * splits) * 4

    assert b1 == ws(4) and b4 == ws(16)
    assert H.hswa_decode_workspace_bytes(0, 128, 4, 64, 8, 128, 100000, total_q=16) == b4
    assert H.hswa_decode_workspace_bytes(0, 128, 4, 64, 8, 128, 100000) == b1


def test_truncate_validation():
    p = _host_pool(8, 32, 2, 4, 8, list(range(8)), [0, 1, 2, 3])
    H.hswa_pool_alloc(p, [0, 1], [20, 3])
    H.hswa_pool_evict(p, [0, 1])          # seq 0 keeps positions 13..19
    before = _tables(p)
    for ids, lens in (([0], [21]), ([0], [-1]), ([0], [19]), ([0, 1], [20, 4]),
                      ([0, 0], [20, 20]), ([2], [0])):
        with pytest.raises(H.HswaError) as e:
            H.hswa_pool_truncate(p, ids, lens)
        assert e.value.status == H.HSWA_E_INVAL
        assert _tables(p) == before
    page1 = before[1][1][0]                    # sequence 1's only Full page
    H.hswa_pool_truncate(p, [0, 1], [20, 0])   # 20: no change; 0: page freed
    seq_len, fpt, mp, free = _tables(p)
    assert seq_len == [20, 0]
    assert fpt[1] == [-1] * 4
    assert free[0] == page1 and len(free) == len(before[3]) + 1


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_capi, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_capi, "_lib", None)
    with pytest.raises(ImportError):
        _capi.load()


def test_match_len_after_eviction_and_validation():
    W = 128
    p = _host_pool(W, 256, 2, 64, 128, list(range(128)), list(range(32)))
    H.hswa_pool_import(p, [0, 1], [1000, 50])   # a restored context: the tail resident
    H.hswa_pool_evict(p, [0, 1])
    # eviction keeps W - 1 positions: the whole sequence is window safe for the
    # next query, not under the page's stricter count of W
    assert H.hswa_pool_match_len(p, [0, 1], [1000, 50]).tolist() == [1000, 50]
    assert H.hswa_pool_match_len(p, [0, 1], [1000, 50], W).tolist() == [0, 50]
    assert H.hswa_pool_match_len(p, [0], [999]).tolist() == [0]
    for ids, want, tail in (([2], [1], 3), ([0], [-1], 3), ([0], [1], -1)):
        with pytest.raises(H.HswaError) as e:
            H.hswa_pool_match_len(p, ids, want, tail)
        assert e.value.status == H.HSWA_E_INVAL


def test_fp8_argument_validation():
    lib = _capi.load()
    a = _args(kv_dtype=2)
    assert lib.hswa_prefill_chunk(C.byref(a), None) == H.HSWA_E_INVAL
    a = _args(kv_dtype=H.HSWA_KV_FP8)                     # scales missing
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    a = _args(kv_dtype=H.HSWA_KV_FP8, k_scale=1 << 20, v_scale=(1 << 20) + 4)  # misaligned
    assert lib.hswa_decode(C.byref(a), None, 0, None) == H.HSWA_E_INVAL
    a = _args(kv_dtype=H.HSWA_KV_FP8, v_scale=1 << 20)     # prefill: K scales missing
    assert lib.hswa_prefill_chunk(C.byref(a), None) == H.HSWA_E_INVAL


def test_append_without_rows_is_a_noop():
    """An append with no rows returns OK without needing k_new / v_new (no
    kernel is launched); with rows, missing k_new / v_new is E_INVAL."""
    lib = _capi.load()
    a = _args(total_q=0, n=1, k_new=None, v_new=None)
    assert lib.hswa_append_kv(C.byref(a), None) == H.HSWA_OK
    a = _args(total_q=0, n=0, k_new=None, v_new=None)
    assert lib.hswa_append_kv(C.byref(a), None) == H.HSWA_OK
    a = _args(total_q=3, n=2, max_q_len=2, k_new=None, v_new=None)
    assert lib.hswa_append_kv(C.byref(a), None) == H.HSWA_E_INVAL


def test_fork_validation():
    """Forks are checked before anything changes: a destination that is not
    empty or is also a source, a length past the source or not window-safe
    (E_INVAL); too few free pages for all forks together (E_NOSPC)."""
    W, C_ = 8, 32
    p = _host_pool(W, C_, 5, 8, 12, list(range(12)), list(range(10)))
    H.hswa_pool_alloc(p, [0, 1], [30, 5])          # pages: 2 + 1, free 9
    H.hswa_pool_evict(p, [0, 1])                   # sequence 0 keeps 23..29
    before = _tables(p)
    bad = [([0], [1], [10]),        # destination not empty
           ([0], [0], [10]),        # destination is its own source
           ([0, 2], [2, 3], [5, 1]),  # a destination is also a source
           ([0], [2], [31]),        # longer than the source
           ([0], [2], [20]),        # position 13 left the SWA pool: not window-safe
           ([5], [2], [1])]         # source out of range
    for src, dst, m in bad:
        with pytest.raises(H.HswaError) as e:
            H.hswa_pool_fork(p, src, dst, m)
        assert e.value.status == H.HSWA_E_INVAL, (src, dst, m)
        assert _tables(p) == before
    # a 30-position fork shares page 0 and needs one fresh page (positions
    # 16-31 hold its window 23..29); two need two, and one is free
    H.hswa_pool_import(p, [4], [128])              # 8 pages: free 1
    before = _tables(p)
    with pytest.raises(H.NoSpace):
        H.hswa_pool_fork(p, [0, 0], [2, 3], [30, 30])
    assert _tables(p) == before
    H.hswa_pool_release(p, [4])
    ff, sf = H.hswa_pool_fork(p, [0, 0], [2, 3], [30, 30])
    assert ff.tolist() == [16, 16] and sf.tolist() == [23, 23]
    t = H.hswa_pool_read_tables(p)
    assert t["fpt"][2][0] == t["fpt"][3][0] == t["fpt"][0][0]
    assert len({t["fpt"][b][1] for b in (0, 2, 3)}) == 3
    # the shared page outlives its first holder
    H.hswa_pool_release(p, [0, 2])
    assert t["fpt"][0][0] not in H.hswa_pool_read_tables(p)["free"].tolist()
    H.hswa_pool_release(p, [3])
    assert t["fpt"][0][0] in H.hswa_pool_read_tables(p)["free"].tolist()


def test_kv_copy_validation():
    from hybrid_sliding_window_hswa_amd import _capi
    lib = _capi.load()
    a = _capi.KvCopyArgs()
    a.kind, a.num_kv_heads, a.head_dim, a.num_seqs, a.max_tok = 1, 2, 128, 1, 16
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_E_INVAL   # no pool view
    a.head_dim = 96
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_E_INVAL
    a.head_dim, a.num_seqs = 128, 0
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_OK         # nothing to copy
    assert lib.hswa_kv_copy(None, None) == H.HSWA_E_INVAL


def _fake_view(a):
    fake = 1 << 20  # never dereferenced: every case below fails validation
    a.pool.seq_len = a.pool.fpt = a.pool.rpt = a.pool.map = fake
    a.pool.max_seqs, a.pool.max_pages_per_seq = 4, 4
    a.pool.ring_slots, a.pool.window = 32, 16
    return fake


def test_fp8_copy_and_transfer_validation():
    """FP8 pages need their scale arrays (copy: K and V page scales;
    transfer: those and the buffers' scales), the page scales aligned to 16
    bytes like every device buffer, the buffer scales to 4, and kv_dtype
    must name a format; each is E_INVAL before any launch."""
    from hybrid_sliding_window_hswa_amd import _capi
    lib = _capi.load()
    a = _capi.KvCopyArgs()
    a.kind, a.num_kv_heads, a.head_dim, a.num_seqs, a.max_tok = 1, 2, 128, 1, 16
    fake = _fake_view(a)
    a.src_ids = a.dst_ids = a.first_pos = a.end_pos = a.k_cache = a.v_cache = fake
    a.kv_dtype = 7
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_E_INVAL
    assert "kv_dtype" in H.hswa_last_error()
    a.kv_dtype, a.k_scale = H.HSWA_KV_FP8, fake
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_E_INVAL     # V scales missing
    assert "scale" in H.hswa_last_error()
    a.v_scale = fake + 2
    assert lib.hswa_kv_copy(C.byref(a), None) == H.HSWA_E_INVAL     # misaligned
    assert "aligned" in H.hswa_last_error()

    x = _capi.XferArgs()
    x.kind, x.num_kv_heads, x.head_dim, x.num_seqs = 1, 2, 128, 1
    x.total_tok, x.max_tok = 16, 16
    fake = _fake_view(x)
    x.seq_ids = x.cu_tok = x.k_cache = x.v_cache = x.buf_k = x.buf_v = fake
    x.kv_dtype = -1
    assert lib.hswa_kv_offload(C.byref(x), None) == H.HSWA_E_INVAL
    assert "kv_dtype" in H.hswa_last_error()
    x.kv_dtype, x.k_scale, x.v_scale = H.HSWA_KV_FP8, fake, fake
    for fn in (lib.hswa_kv_offload, lib.hswa_kv_restore):
        assert fn(C.byref(x), None) == H.HSWA_E_INVAL               # buffer scales missing
        assert "buf_k_scale" in H.hswa_last_error()
    x.buf_k_scale, x.buf_v_scale = fake, fake + 1
    assert lib.hswa_kv_restore(C.byref(x), None) == H.HSWA_E_INVAL  # misaligned
    assert "aligned" in H.hswa_last_error()
    x.buf_v_scale, x.k_scale = fake + 4, fake + 4   # buffer scales need 4, page scales 16
    assert lib.hswa_kv_offload(C.byref(x), None) == H.HSWA_E_INVAL
    assert "16-byte" in H.hswa_last_error()


@pytest.mark.parametrize("seqs,hkv,max_len,splits", [
    (256, 8, 32769, 2),     # the mixed decode: two pieces of 16,448 keys
    (64, 8, 262145, 13),    # long contexts: pieces of at most 20,480 keys
    (256, 1, 32769, 8),     # one KV head: more pieces for parallelism
    (1, 8, 32769, 33),      # one sequence: pieces of 1,024 keys (the floor)
    (4, 8, 1000, 1),        # short contexts: no split
])
def test_decode_split_plan(seqs, hkv, max_len, splits):
    """Full-layer decode plans about 2,048 (sequence, KV head, piece) work
    items with pieces of 1,024 to about 20K keys; the workspace holds one
    partial state per (row, head, piece) and the work list."""
    b = H.hswa_decode_workspace_bytes(0, 128, seqs, 8 * hkv, hkv, 128, max_len)
    if splits == 1:
        assert b == 0
        return
    partial = seqs * 8 * hkv * splits * (128 + 2) * 4
    assert b == -(-partial // 256) * 256 + (8 * 32 + 32 + seqs * splits) * 4
