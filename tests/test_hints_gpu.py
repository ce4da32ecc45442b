"""GPU checks of the caller-hint and ring-aliasing guards.

- Full decode sizes its split-K grid from the caller's max_seq_len.  A hint
  below a sequence's length (e.g. the pre-append length) must still cover
  every key: the result equals the oracle's.
- Prefill sizes its grid from max_q_len.  Rows past a hint that is too small
  are not computed; they come back as NaN with valid length -1, and every
  row inside the grid is still exact.
- A SWA ring of C slots holds at most positions [L - C, L).  A restore whose
  range reaches below L - C must not write the aliased slots of newer,
  live positions, and an SWA transfer of more than C positions per sequence
  is refused.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA

from harness import TOL, Setup, dev, make_seqs, oracle_rows
from test_transfer_gpu import Layers, _bits, _contexts

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hint_delta", [-1, -2047])
def test_decode_max_seq_len_hint_below_length(gpu, hint_delta):
    """Contexts of 4,096 and 2,048 tokens plus one appended token.  The hint
    4,096 (the pre-append length) plans 4 splits of 1,024 keys, one short of
    the 4,097 keys of the first sequence; hint 2,050 plans 3."""
    hq, hkv, d, W = 64, 8, 128, 128
    ctxs = [4096, 2048]
    B = len(ctxs)
    seqs = make_seqs([c + 1 for c in ctxs], hq, hkv, d, seed=131)
    maxp = max(ctxs) // 16 + 2
    st = Setup(H.FULL, W, W, B, maxp, B * maxp + 4, hkv, d, seed=131)
    ids = list(range(B))
    H.hswa_pool_import(st.pool, ids, ctxs)
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(ctxs)]), dtype=torch.int32, device=dev())
    kf = torch.cat([s.k[:c] for s, c in zip(seqs, ctxs)]).to(dev())
    vf = torch.cat([s.v[:c] for s, c in zip(seqs, ctxs)]).to(dev())
    H.hswa_append_kv(H.FULL, kf, vf, sid, st.view, st.kc, st.vc, cu, max(ctxs))
    H.hswa_pool_alloc(st.pool, ids, [1] * B)
    pos = list(ctxs)
    q = torch.stack([s.q[p] for s, p in zip(seqs, pos)]).to(dev())
    kn = torch.stack([s.k[p] for s, p in zip(seqs, pos)]).to(dev())
    vn = torch.stack([s.v[p] for s, p in zip(seqs, pos)]).to(dev())
    hint = max(ctxs) + 1 + hint_delta
    nb = H.hswa_decode_workspace_bytes(H.FULL, W, B, hq, hkv, d, hint)
    ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
    out = torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=dev())
    vl = torch.full((B,), -7, dtype=torch.int32, device=dev())
    H.hswa_decode(H.FULL, W, q, kn, vn, sid, hint, st.view, st.kc, st.vc, out, ws, vl)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    for b in range(B):
        exp = oracle_rows(seqs[b], [pos[b]], H.FULL, W)[0]
        err = float(np.max(np.abs(got[b] - exp)))
        assert err < TOL, f"sequence {b}: {err:.3e}"
    assert vl.cpu().tolist() == [p + 1 for p in pos]


@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_prefill_max_q_len_hint_below_rows(gpu, kind):
    """100 rows with the hint 40: the grid holds two 32-row blocks (hq 8,
    hkv 2), so rows 64..99 are NaN with valid length -1; rows 0..63 match
    the oracle."""
    hq, hkv, d, W, n = 8, 2, 128, 16, 100
    seqs = make_seqs([n], hq, hkv, d, seed=133)
    st = Setup(kind, W, W + n + 12, 1, n // 16 + 2, n // 16 + 4, hkv, d, seed=133)
    H.hswa_pool_alloc(st.pool, [0], [n])
    s = seqs[0]
    cu = torch.tensor([0, n], dtype=torch.int32, device=dev())
    sid = torch.zeros(1, dtype=torch.int32, device=dev())
    out = torch.zeros((n, hq, d), dtype=torch.float32, device=dev())
    vl = torch.zeros((n,), dtype=torch.int32, device=dev())
    H.hswa_prefill_chunk(kind, W, s.q.to(dev()), s.k.to(dev()), s.v.to(dev()), sid, cu, 40,
                         st.view, st.kc, st.vc, out, vl)
    torch.cuda.synchronize()
    got, vlen = out.cpu().double().numpy(), vl.cpu().numpy()
    exp = oracle_rows(s, list(range(64)), kind, W)
    assert float(np.max(np.abs(got[:64] - exp))) < TOL
    assert vlen[:64].tolist() == [OA.valid_length(p, kind, W) for p in range(64)]
    assert np.all(np.isnan(got[64:]))
    assert np.all(vlen[64:] == -1)


def test_swa_restore_below_ring_start_leaves_live_slots(gpu):
    """A 300-token sequence with W = 128 and a 128-slot ring: restoring
    positions [100, 228) writes only [172, 228) (position 172 is the oldest
    the ring can hold); positions 228..299, whose slots positions 100..171
    alias, keep their bits."""
    hkv, d, W, L = 2, 64, 128, 300
    k, v = _contexts([L], hkv, d, 137)
    lay = Layers([L], hkv, d, W, 137, 1)
    lay.fill(k, v)
    (bk0, bv0), cnt = lay.move(H.SWA, True)
    assert cnt == [W - 1]                     # positions 173 .. 299
    first = torch.tensor([100], dtype=torch.int32, device=dev())
    cu = torch.tensor([0, 128], dtype=torch.int32, device=dev())
    zk = torch.zeros((128, hkv, d), dtype=torch.bfloat16, device=dev())
    zv = torch.zeros((128, hkv, d), dtype=torch.float16, device=dev())
    H.hswa_kv_restore(H.SWA, lay.sid, cu, 128, 128, lay.view, lay.sk, lay.sv, zk, zv,
                      first_pos=first)
    (bk1, bv1), _ = lay.move(H.SWA, True)
    k0, v0, k1, v1 = _bits(bk0), _bits(bv0), _bits(bk1), _bits(bv1)
    # buffer row r is position 173 + r: rows of 173..227 were restored to 0,
    # rows of 228..299 are untouched
    n_new = 228 - 173
    assert np.all(k1[:n_new] == 0) and np.all(v1[:n_new] == 0)
    assert np.array_equal(k1[n_new:cnt[0]], k0[n_new:cnt[0]])
    assert np.array_equal(v1[n_new:cnt[0]], v0[n_new:cnt[0]])
    # more positions per sequence than the ring holds is refused
    with pytest.raises(H.HswaError) as e:
        H.hswa_kv_restore(H.SWA, lay.sid, torch.tensor([0, 129], dtype=torch.int32,
                                                       device=dev()),
                          129, 129, lay.view, lay.sk, lay.sv,
                          torch.zeros((129, hkv, d), dtype=torch.bfloat16, device=dev()),
                          torch.zeros((129, hkv, d), dtype=torch.float16, device=dev()),
                          first_pos=first)
    assert e.value.status == H.HSWA_E_INVAL
