"""GPU parity of FP8 pages through the window-masked tier transfer and the
page-to-page copy (Baidu Day0 hybrid-attention article, Layered
quantization, point 2: FP8 KV per token and head; MiMo-V2.5 inference page,
sec. 2.1: "KVCache Dual Pool", Data Transfer by the SWA mask, and
"SWA-aware prefix cache tree", point 3: the window moves with a reused
prefix).

* Offload: the code and scale buffers hold, bit for bit, the oracle's FP8
  host image of the same inputs (SWA layers: the window [L-W+1, L); Full
  layers: every position), for pinned host and device buffers, ragged
  lengths and permuted pages.
* Restore into a second pool with other page orders: the restored slots
  hold the source's codes and scales bit for bit, every other byte keeps its
  sentinel, and FP8 decode over the restored pool equals decode over the
  source bit for bit (and the oracle on the dequantized rows within 4e-3).
* Copy, FP8 and BF16 pages: for pairs with ragged ranges (partial tiles at
  both ends, a whole tile, ranges cut by either sequence's length or ring,
  a pair with equal ids), the destination slots of the copied positions
  hold the source's bits and every other byte of the layer is unchanged.
* Seeded random configurations of both (KV heads 1-12, d 64 and 128,
  windows 1-200, rings from one page up).
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle import fp8 as F8
from oracle import transfer as OT

from harness import TOL, dev
from test_fp8_decode_gpu import Fp8Pool

pytestmark = pytest.mark.gpu


def _contexts(lens, hkv, d, seed):
    k = [synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_K) for b, L in enumerate(lens)]
    v = [synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_V) for b, L in enumerate(lens)]
    return k, v


def _move(P, kind, lens, to_host, bufs=None, pinned=True, explicit=False):
    cnt = H.hswa_pool_window_counts(P.pool, kind, P.ids).tolist()
    T = sum(cnt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(cnt)]), dtype=torch.int32, device=dev())
    first = None
    if explicit:
        first = torch.tensor([L - c for L, c in zip(lens, cnt)], dtype=torch.int32, device=dev())
    if bufs is None:
        def mk(shape, dt):
            if pinned:
                return torch.empty(shape, dtype=dt, pin_memory=True)
            return torch.empty(shape, dtype=dt, device=dev())
        rows = max(T, 1)
        bufs = (mk((rows, P.hkv, P.d), torch.uint8), mk((rows, P.hkv, P.d), torch.uint8),
                mk((rows, P.hkv), torch.float32), mk((rows, P.hkv), torch.float32))
    kc, vc, ks, vs = P.bufs(kind)
    fn = H.hswa_kv_offload if to_host else H.hswa_kv_restore
    fn(kind, P.sid, cu, T, max(max(cnt), 1), P.view, kc, vc, bufs[0], bufs[1], first_pos=first,
       k_scale=ks, v_scale=vs, buf_k_scale=bufs[2], buf_v_scale=bufs[3])
    torch.cuda.synchronize()
    return bufs, cnt


def _u32(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("d,hkv", [(128, 8), (64, 2), (128, 12)])
def test_fp8_offload_matches_oracle_image(gpu, pinned, d, hkv):
    lens = [700, 1, 0, 127, 128, 129, 37, 2050]
    W = 128
    k, v = _contexts(lens, hkv, d, 23)
    P = Fp8Pool(lens, hkv, d, W, 5)
    P.append_context(k, v, lens)
    for kind in (H.FULL, H.SWA):
        bufs, cnt = _move(P, kind, lens, True, pinned=pinned)
        assert cnt == OT.transfer_counts(kind, lens, W)
        ck, cv, sk, sv = OT.host_image_fp8(kind, W, [(k[b].float().numpy(), v[b].float().numpy())
                                                     for b in P.ids])
        T = sum(cnt)
        assert np.array_equal(bufs[0][:T].cpu().numpy(), ck), kind
        assert np.array_equal(bufs[1][:T].cpu().numpy(), cv), kind
        assert np.array_equal(_u32(bufs[2][:T]), sk.view(np.uint32)), kind
        assert np.array_equal(_u32(bufs[3][:T]), sv.view(np.uint32)), kind


def _round_trip(src, dst, lens, W, pinned=True):
    """Offload every layer kind of src and restore it into dst (its own page
    orders): dst's restored slots hold src's codes and scales bit for bit,
    every other byte of dst keeps what it held."""
    sentinel = {kind: [t.cpu() for t in dst.bufs(kind)] for kind in (H.FULL, H.SWA)}
    for kind in (H.FULL, H.SWA):
        bufs, _ = _move(src, kind, lens, True, pinned=pinned)
        _move(dst, kind, lens, False, bufs=bufs, explicit=True)
        s_all = [t.cpu() for t in src.bufs(kind)]
        d_all = [t.cpu() for t in dst.bufs(kind)]
        want = sentinel[kind]
        for b, L in enumerate(lens):
            for pos in OT.transfer_positions(kind, L, W):
                a, c = src.slot(kind, b, pos), dst.slot(kind, b, pos)
                for i in range(4):
                    if i == 1:      # V codes: a column of the page
                        want[i][c // 16, :, :, c % 16] = s_all[i][a // 16, :, :, a % 16]
                    else:           # K codes, K and V scales: a row
                        want[i][c // 16, :, c % 16] = s_all[i][a // 16, :, a % 16]
        for i in range(4):
            g, w = d_all[i].numpy(), want[i].numpy()
            if g.dtype == np.float32:
                g, w = g.view(np.uint32), w.view(np.uint32)
            assert np.array_equal(g, w), (kind, i)


def test_fp8_round_trip_into_other_pages(gpu):
    lens = [1500, 90, 3, 128, 4100]
    hq, hkv, d, W = 64, 8, 128, 128
    k, v = _contexts(lens, hkv, d, 33)
    src = Fp8Pool(lens, hkv, d, W, 11)
    src.append_context(k, v, lens)
    dst = Fp8Pool(lens, hkv, d, W, 12)        # other page orders; codes 0x7F, NaN scales
    _round_trip(src, dst, lens, W)
    # decode one new token over both pools: identical outputs, oracle-close
    B = len(lens)
    q = synth.bf16_normal((B, hq, d), 33, 5, 0, synth.ROLE_Q)
    kn = synth.bf16_normal((B, hkv, d), 33, 5, 0, synth.ROLE_K)
    vn = synth.bf16_normal((B, hkv, d), 33, 5, 0, synth.ROLE_V)
    outs = []
    for P in (src, dst):
        H.hswa_pool_alloc(P.pool, P.ids, [1] * B)
        res = []
        for kind in (H.FULL, H.SWA):
            kc, vc, ks, vs = P.bufs(kind)
            maxlen = max(lens) + 1
            nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen)
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            out = torch.empty((B, hq, d), dtype=torch.float32, device=dev())
            H.hswa_decode(kind, W, q.to(dev()), kn.to(dev()), vn.to(dev()), P.sid, maxlen,
                          P.view, kc, vc, out, ws, k_scale=ks, v_scale=vs)
            res.append(out.cpu())
        outs.append(res)
    for a, b in zip(*outs):
        assert torch.equal(a, b)

    def deq(x):
        codes, scale = F8.quantize_rows(x.float().numpy())
        return F8.dequantize_rows(codes, scale)

    for kind, got in zip((OA.FULL, OA.SWA), outs[1]):
        for b, L in enumerate(lens):
            kk = deq(torch.cat([k[b], kn[b:b + 1]]))
            vv = deq(torch.cat([v[b], vn[b:b + 1]]))
            exp = OA.attend(synth.to_f64(q[b:b + 1]), [L], kk, vv, kind, W)
            err = float(np.max(np.abs(got[b:b + 1].double().numpy() - exp)))
            assert err < TOL, (kind, b, err)


@pytest.mark.parametrize("case", range(10))
def test_fp8_transfer_random_configuration(gpu, case):
    """Seeded random shapes: KV heads 1-12, d, window 1-200 (rings down to
    one page), 1-6 sequences of 0-2,000 tokens, pinned or device buffers.
    The packed image of both layer kinds equals the oracle's bit for bit,
    and restoring it into a pool with other page orders puts back the same
    bits and nothing else."""
    import random
    rnd = random.Random(9700 + case)
    hkv, d = rnd.choice([1, 2, 3, 8, 12]), rnd.choice([64, 128])
    W = rnd.choice([1, 2, 5, 16, 33, 128, 200])
    lens = [rnd.randint(0, 2000) for _ in range(rnd.randint(1, 6))]
    pinned = rnd.random() < 0.5
    print(f"case {case}: hkv {hkv} d {d} W {W} lens {lens} pinned {pinned}", flush=True)
    k, v = _contexts(lens, hkv, d, 830 + case)
    src = Fp8Pool(lens, hkv, d, W, 40 + case)
    src.append_context(k, v, lens)
    for kind in (H.FULL, H.SWA):
        bufs, cnt = _move(src, kind, lens, True, pinned=pinned)
        assert cnt == OT.transfer_counts(kind, lens, W)
        ck, cv, sk, sv = OT.host_image_fp8(kind, W, [(k[b].float().numpy(), v[b].float().numpy())
                                                     for b in src.ids])
        T = sum(cnt)
        assert np.array_equal(bufs[0][:T].cpu().numpy().reshape(-1), ck.reshape(-1)), kind
        assert np.array_equal(bufs[1][:T].cpu().numpy().reshape(-1), cv.reshape(-1)), kind
        assert np.array_equal(_u32(bufs[2][:T]).reshape(-1), sk.view(np.uint32).reshape(-1))
        assert np.array_equal(_u32(bufs[3][:T]).reshape(-1), sv.view(np.uint32).reshape(-1))
    _round_trip(src, Fp8Pool(lens, hkv, d, W, 60 + case), lens, W, pinned)


def test_fp8_transfer_rejects_missing_buffer_scales(gpu):
    lens = [40]
    P = Fp8Pool(lens, 2, 64, 16, 41)
    cu = torch.tensor([0, 15], dtype=torch.int32, device=dev())
    kc, vc, ks, vs = P.bufs(H.SWA)
    bk = torch.empty((15, 2, 64), dtype=torch.uint8, device=dev())
    bv = torch.empty((15, 2, 64), dtype=torch.uint8, device=dev())
    with pytest.raises(ValueError):
        H.hswa_kv_offload(H.SWA, P.sid, cu, 15, 15, P.view, kc, vc, bk, bv, k_scale=ks,
                          v_scale=vs)


class CopyPool:
    """One pool, a Full and a SWA layer of either page format, every
    sequence's context imported and its window appended."""

    def __init__(self, lens, hkv, d, W, C, seed, fp8):
        S = len(lens)
        self.S, self.C, self.fp8 = S, C, fp8
        self.maxp = max(lens) // 16 + 2
        npages = S * self.maxp + 3
        free = synth.permutation(npages, seed, 1)
        ring = synth.permutation(S * C // 16, seed, 2)
        self.pool = H.hswa_pool_create(W, C, S, self.maxp, npages, free, ring, device=dev())
        self.view = H.hswa_pool_get_view(self.pool)
        if fp8:
            self.layers = {H.FULL: H.kv_cache_alloc_fp8(npages, hkv, d, dev(), 0x7F),
                           H.SWA: H.kv_cache_alloc_fp8(S * C // 16, hkv, d, dev(), 0x7F)}
        else:
            self.layers = {H.FULL: H.kv_cache_alloc(npages, hkv, d, dev(), float("nan")),
                           H.SWA: H.kv_cache_alloc(S * C // 16, hkv, d, dev(), float("nan"))}
        ids = list(range(S))
        H.hswa_pool_import(self.pool, ids, lens)
        k, v = _contexts(lens, hkv, d, seed)
        for kind, bufs in self.layers.items():
            cnt = H.hswa_pool_window_counts(self.pool, kind, ids).tolist()
            live = [b for b in ids if cnt[b] > 0]
            if not live:                 # W = 1: no SWA layer rows to append
                continue
            cu = torch.tensor(np.concatenate([[0], np.cumsum([cnt[b] for b in live])]),
                              dtype=torch.int32, device=dev())
            sc = dict(k_scale=bufs[2], v_scale=bufs[3]) if fp8 else {}
            H.hswa_append_kv(kind, torch.cat([k[b][lens[b] - cnt[b]:] for b in live]).to(dev()),
                             torch.cat([v[b][lens[b] - cnt[b]:] for b in live]).to(dev()),
                             torch.tensor(live, dtype=torch.int32, device=dev()), self.view,
                             bufs[0], bufs[1], cu, max(cnt), **sc)
        torch.cuda.synchronize()
        self.fpt = H.hswa_pool_read_tables(self.pool)["fpt"]
        self.rpt = self.pool.tables["rpt"].cpu().view(S, C // 16)

    def slot(self, kind, b, pos):
        if kind == H.FULL:
            return int(self.fpt[b][pos // 16]) * 16 + pos % 16
        r = pos % self.C
        return int(self.rpt[b][r // 16]) * 16 + r % 16


def _bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int32) if t.dtype == torch.float32 else (
        t if t.dtype == torch.uint8 else t.view(torch.int16))


@pytest.mark.parametrize("fp8", [True, False], ids=["fp8", "bf16"])
@pytest.mark.parametrize("d,hkv", [(128, 4), (64, 3)])
def test_copy_moves_exactly_the_listed_positions(gpu, fp8, d, hkv):
    W, C = 48, 64
    lens = [300, 77, 45, 260, 100, 45, 20]
    # (source, destination, first, end)
    pairs = [(0, 3, 37, 290), (1, 4, 0, 500), (2, 5, 16, 32), (6, 6, 0, 20)]
    _check_copy(lens, pairs, hkv, d, W, C, 70 + d + hkv, fp8)


@pytest.mark.parametrize("case", range(10))
def test_copy_random_configuration(gpu, case):
    """Seeded random copies: FP8 or BF16 pages, KV heads 1-8, d, windows
    1-200 with rings of the window or up to three pages more, 2-4 disjoint
    pairs whose destination is about as long as the source, with ranges
    from 0, from the window start, from inside the ring or anywhere, to
    the shared end, past it, or a few positions on (some empty)."""
    import random
    rnd = random.Random(9900 + case)
    fp8 = case % 2 == 0
    hkv, d = rnd.choice([1, 2, 3, 8]), rnd.choice([64, 128])
    W = rnd.choice([1, 2, 5, 16, 33, 128, 200])
    C = 16 * (-(-W // 16) + rnd.choice([0, 0, 1, 3]))
    n = rnd.randint(2, 4)
    src = [rnd.randint(1, 700) for _ in range(n)]
    dst = [max(1, L + rnd.choice([-20, 0, 0, 5, 100])) for L in src]
    lens = src + dst
    pairs = []
    for i in range(n):
        m = min(src[i], dst[i])
        first = rnd.choice([0, max(0, m - W + 1), max(0, m - rnd.randint(1, C)),
                            rnd.randint(0, m)])
        end = rnd.choice([m, m + 50, first + rnd.choice([0, 1, 15, 16, 17])])
        pairs.append((i, n + i, first, end))
    print(f"case {case}: fp8 {fp8} hkv {hkv} d {d} W {W} C {C} lens {lens} pairs {pairs}",
          flush=True)
    _check_copy(lens, pairs, hkv, d, W, C, 90 + case, fp8)


def _check_copy(lens, pairs, hkv, d, W, C, seed, fp8):
    P = CopyPool(lens, hkv, d, W, C, seed, fp8)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=dev())
    for kind, bufs in P.layers.items():
        before = [t.cpu().clone() for t in bufs]
        want = [t.clone() for t in before]
        for a, b, first, end in pairs:
            if a == b:
                continue
            p1 = min(end, lens[a], lens[b])
            p0 = first
            if kind == H.SWA:
                p0 = max(p0, lens[a] - C, lens[b] - C)
            p0 = max(p0, 0)
            for pos in range(p0, p1):
                s, t = P.slot(kind, a, pos), P.slot(kind, b, pos)
                for i, x in enumerate(want):
                    if i == 1:
                        x[t // 16, :, :, t % 16] = before[i][s // 16, :, :, s % 16]
                    else:
                        x[t // 16, :, t % 16] = before[i][s // 16, :, s % 16]
        cols = list(zip(*pairs))
        max_tok = C if kind == H.SWA else max(1, max(e - f for _, _, f, e in pairs))
        sc = dict(k_scale=bufs[2], v_scale=bufs[3]) if fp8 else {}
        H.hswa_kv_copy(kind, i32(cols[0]), i32(cols[1]), i32(cols[2]), i32(cols[3]), max_tok,
                       P.view, bufs[0], bufs[1], **sc)
        torch.cuda.synchronize()
        for i, (g, w) in enumerate(zip(bufs, want)):
            assert torch.equal(_bits(g), _bits(w)), (kind, i)
