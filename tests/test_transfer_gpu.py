"""GPU parity of the window-masked tier transfer (MiMo-V2.5 inference page,
sec. 2.1: "Data Transfer" goes by the SWA mask; layer-by-layer pulling).

* Offload: the packed buffer holds, bit for bit, what the oracle's host image
  says (SWA layers: the window [L-W+1, L); Full layers: every position), for
  pinned host and device buffers, ragged lengths and permuted pages.
* Restore into a second pool with other page orders: the restored slots hold
  the same bits as the source, every other slot keeps its sentinel, and decode
  over the restored pool equals decode over the source bit for bit (and the
  oracle within 4e-3).
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle import transfer as OT

from harness import TOL, dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Layers:
    """A pool with one Full and one SWA layer, contexts restored by import +
    append (Full: every position, SWA: the window tail)."""

    def __init__(self, lens, hkv, d, W, seed, perm_seed, fill=float("nan")):
        B = len(lens)
        self.B, self.W, self.hkv, self.d = B, W, hkv, d
        self.C = 16 * (-(-W // 16))
        self.maxp = max(lens) // 16 + 2
        self.npages = B * self.maxp + 7
        free = synth.permutation(self.npages, perm_seed, 1)
        ring = synth.permutation(B * self.C // 16, perm_seed, 2)
        self.pool = H.hswa_pool_create(W, self.C, B, self.maxp, self.npages, free, ring,
                                       device=dev())
        self.view = H.hswa_pool_get_view(self.pool)
        self.fk, self.fv = H.kv_cache_alloc(self.npages, hkv, d, dev(), fill)
        self.sk, self.sv = H.kv_cache_alloc(B * self.C // 16, hkv, d, dev(), fill)
        self.ids = list(range(B))
        self.sid = torch.tensor(self.ids, dtype=torch.int32, device=dev())
        H.hswa_pool_import(self.pool, self.ids, lens)
        self.lens = list(lens)

    def caches(self, kind):
        return (self.fk, self.fv) if kind == H.FULL else (self.sk, self.sv)

    def fill(self, k, v):
        """Append the contexts k[b], v[b] ([L, Hkv, d] bf16, cpu)."""
        for kind in (H.FULL, H.SWA):
            cnt = H.hswa_pool_window_counts(self.pool, kind, self.ids).tolist()
            live = [b for b in self.ids if cnt[b] > 0]
            if not live:
                continue
            cu = torch.tensor(np.concatenate([[0], np.cumsum([cnt[b] for b in live])]),
                              dtype=torch.int32, device=dev())
            kc, vc = self.caches(kind)
            kk = torch.cat([k[b][self.lens[b] - cnt[b]:] for b in live]).to(dev())
            vv = torch.cat([v[b][self.lens[b] - cnt[b]:] for b in live]).to(dev())
            H.hswa_append_kv(kind, kk, vv, torch.tensor(live, dtype=torch.int32, device=dev()),
                             self.view, kc, vc, cu, max(cnt))

    def move(self, kind, to_host, bufs=None, pinned=True, explicit=False):
        cnt = H.hswa_pool_window_counts(self.pool, kind, self.ids).tolist()
        T = sum(cnt)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(cnt)]), dtype=torch.int32, device=dev())
        first = None
        if explicit:   # the same positions named explicitly
            first = torch.tensor([L - c for L, c in zip(self.lens, cnt)], dtype=torch.int32,
                                 device=dev())
        if bufs is None:
            shape = (max(T, 1), self.hkv, self.d)
            if pinned:
                bufs = (torch.empty(shape, dtype=torch.bfloat16, pin_memory=True),
                        torch.empty(shape, dtype=torch.float16, pin_memory=True))
            else:
                bufs = (torch.empty(shape, dtype=torch.bfloat16, device=dev()),
                        torch.empty(shape, dtype=torch.float16, device=dev()))
        kc, vc = self.caches(kind)
        fn = H.hswa_kv_offload if to_host else H.hswa_kv_restore
        fn(kind, self.sid, cu, T, max(max(cnt), 1), self.view, kc, vc, bufs[0], bufs[1],
           first_pos=first)
        torch.cuda.synchronize()
        return bufs, cnt

    def slots(self, kind):
        """Physical slot of every transferred position, in buffer order."""
        t = H.hswa_pool_read_tables(self.pool)
        out = []
        for b in self.ids:
            for pos in OT.transfer_positions(kind, self.lens[b], self.W):
                if kind == H.FULL:
                    out.append(int(t["fpt"][b][pos // 16]) * 16 + pos % 16)
                else:
                    r = pos % self.C
                    ring = self.pool.tables["rpt"].cpu().view(self.B, self.C // 16)
                    out.append(int(ring[b][r // 16]) * 16 + r % 16)
        return out


def _contexts(lens, hkv, d, seed):
    k = [synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_K) for b, L in enumerate(lens)]
    v = [synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_V) for b, L in enumerate(lens)]
    return k, v


@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("d,hkv", [(128, 8), (64, 2), (128, 12)])
def test_offload_matches_oracle_image(gpu, pinned, d, hkv):
    lens = [700, 1, 0, 127, 128, 129, 37, 2050]
    W = 128
    k, v = _contexts(lens, hkv, d, 21)
    src = Layers(lens, hkv, d, W, 21, 3)
    src.fill(k, v)
    for kind in (H.FULL, H.SWA):
        (bk, bv), cnt = src.move(kind, True, pinned=pinned)
        assert cnt == OT.transfer_counts(kind, lens, W)
        ek, ev = OT.host_image(kind, W, [(_bits(k[b]), _bits(v[b])) for b in src.ids])
        T = sum(cnt)
        assert np.array_equal(_bits(bk)[:T].reshape(-1), ek.reshape(-1)), kind
        assert np.array_equal(_bits(bv)[:T].reshape(-1), ev.reshape(-1)), kind


def test_round_trip_into_other_pages(gpu):
    lens = [1500, 90, 3, 128, 4100]
    hq, hkv, d, W = 64, 8, 128, 128
    k, v = _contexts(lens, hkv, d, 31)
    src = Layers(lens, hkv, d, W, 31, 1)
    src.fill(k, v)
    dst = Layers(lens, hkv, d, W, 31, 2, fill=7.0)   # other page orders, sentinel 7
    for kind in (H.FULL, H.SWA):
        bufs, _ = src.move(kind, True)
        dst.move(kind, False, bufs=bufs, explicit=True)
        kc_s, vc_s = src.caches(kind)
        kc_d, vc_d = dst.caches(kind)
        ss, sd = src.slots(kind), dst.slots(kind)
        ks, vs = kc_s.cpu(), vc_s.cpu()
        kd, vd = kc_d.cpu(), vc_d.cpu()
        # restored slots: same bits as the source's slots of the same positions
        for a, b in zip(ss, sd):
            assert torch.equal(kd[b // 16, :, b % 16].view(torch.int16),
                               ks[a // 16, :, a % 16].view(torch.int16))
            assert torch.equal(vd[b // 16, :, :, b % 16].view(torch.int16),
                               vs[a // 16, :, :, a % 16].view(torch.int16))
        # every other slot keeps the sentinel
        keep = torch.ones(kd.shape[0] * 16, dtype=torch.bool)
        keep[torch.as_tensor(sd, dtype=torch.long)] = False
        kk = kd.permute(0, 2, 1, 3).reshape(-1, hkv * d)[keep]
        vv = vd.permute(0, 3, 1, 2).reshape(-1, hkv * d)[keep]
        assert torch.all(kk == 7.0) and torch.all(vv == 7.0)
    # decode one new token over both pools: identical outputs, oracle-close
    q = synth.bf16_normal((len(lens), hq, d), 31, 5, 0, synth.ROLE_Q)
    kn = synth.bf16_normal((len(lens), hkv, d), 31, 5, 0, synth.ROLE_K)
    vn = synth.bf16_normal((len(lens), hkv, d), 31, 5, 0, synth.ROLE_V)
    outs = []
    for L in (src, dst):
        H.hswa_pool_alloc(L.pool, L.ids, [1] * len(lens))
        res = []
        for kind in (H.FULL, H.SWA):
            kc, vc = L.caches(kind)
            maxlen = max(lens) + 1
            nb = H.hswa_decode_workspace_bytes(kind, W, len(lens), hq, hkv, d, maxlen)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            out = torch.empty((len(lens), hq, d), dtype=torch.float32, device=dev())
            H.hswa_decode(kind, W, q.to(dev()), kn.to(dev()), vn.to(dev()), L.sid, maxlen,
                          L.view, kc, vc, out, ws)
            res.append(out.cpu())
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    for kind, got in zip((OA.FULL, OA.SWA), outs[1]):
        for b, L in enumerate(lens):
            kk = synth.to_f64(torch.cat([k[b], kn[b:b + 1]]))
            vv = synth.to_f64(torch.cat([v[b], vn[b:b + 1]]))
            exp = OA.attend(synth.to_f64(q[b:b + 1]), [L], kk, vv, kind, W)
            err = float(np.max(np.abs(got[b:b + 1].double().numpy() - exp)))
            assert err < TOL, (kind, b, err)


def test_transfer_rejects_pageable_host_memory(gpu):
    lens = [40]
    src = Layers(lens, 2, 64, 16, 41, 1)
    cu = torch.tensor([0, 15], dtype=torch.int32, device=dev())
    bk = torch.empty((15, 2, 64), dtype=torch.bfloat16)          # pageable, not pinned
    bv = torch.empty((15, 2, 64), dtype=torch.float16)
    with pytest.raises(H.HswaError) as e:
        H.hswa_kv_offload(H.SWA, src.sid, cu, 15, 15, src.view, src.sk, src.sv, bk, bv)
    assert e.value.status == H.HSWA_E_INVAL


def test_explicit_positions_ignore_later_growth(gpu):
    """With first_pos the moved range stays put while seq_len grows (an alloc
    on another stream): offload after an alloc returns the pre-alloc window."""
    lens = [300, 50]
    hkv, d, W = 2, 64, 32
    k, v = _contexts(lens, hkv, d, 51)
    src = Layers(lens, hkv, d, W, 51, 1)
    src.fill(k, v)
    (bk0, bv0), cnt = src.move(H.SWA, True, explicit=True)
    H.hswa_pool_alloc(src.pool, src.ids, [1, 1])   # seq_len grows by one
    T = sum(cnt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(cnt)]), dtype=torch.int32, device=dev())
    first = torch.tensor([L - c for L, c in zip(lens, cnt)], dtype=torch.int32, device=dev())
    bk = torch.empty(bk0.shape, dtype=bk0.dtype, pin_memory=True)   # empty_like drops pinning
    bv = torch.empty(bv0.shape, dtype=bv0.dtype, pin_memory=True)
    H.hswa_kv_offload(H.SWA, src.sid, cu, T, max(cnt), src.view, src.sk, src.sv, bk, bv,
                      first_pos=first)
    torch.cuda.synchronize()
    assert torch.equal(bk[:T].view(torch.int16), bk0[:T].view(torch.int16))
    assert torch.equal(bv[:T].view(torch.int16), bv0[:T].view(torch.int16))


@pytest.mark.parametrize("case", range(12))
def test_offload_random_configuration(gpu, case):
    """Seeded random shapes: KV heads 1-12, d, window 1-200 (rings down to
    one page), 1-6 sequences of 0-3,000 tokens, pinned or device buffers;
    the packed image of both layer kinds equals the oracle's bit for bit."""
    import random
    rnd = random.Random(9500 + case)
    hkv, d = rnd.choice([1, 2, 3, 8, 12]), rnd.choice([64, 128])
    W = rnd.choice([1, 2, 5, 33, 128, 200])
    lens = [rnd.randint(0, 3000) for _ in range(rnd.randint(1, 6))]
    pinned = rnd.random() < 0.5
    print(f"case {case}: hkv {hkv} d {d} W {W} lens {lens} pinned {pinned}", flush=True)
    k, v = _contexts(lens, hkv, d, 800 + case)
    src = Layers(lens, hkv, d, W, 800 + case, 4)
    src.fill(k, v)
    for kind in (H.FULL, H.SWA):
        (bk, bv), cnt = src.move(kind, True, pinned=pinned)
        assert cnt == OT.transfer_counts(kind, lens, W)
        ek, ev = OT.host_image(kind, W, [(_bits(k[b]), _bits(v[b])) for b in src.ids])
        T = sum(cnt)
        assert np.array_equal(_bits(bk)[:T].reshape(-1), ek.reshape(-1)), kind
        assert np.array_equal(_bits(bv)[:T].reshape(-1), ev.reshape(-1)), kind
