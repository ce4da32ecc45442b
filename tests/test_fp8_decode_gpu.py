"""GPU parity of FP8 KV pages (Baidu Day0 hybrid-attention article, Layered
quantization, point 2: FP8 KV per token, head and 128-element tile).

* The quantizing append writes, bit for bit, the e4m3 codes and fp32 scales
  of the oracle's quantizer (K token-major, V dim-major, scales per page,
  head and token), for Full pages and SWA rings, ragged lengths and partial
  page tiles.
* Decode over FP8 pages (plain and multi-row, split-K, GQA 1..8) matches the
  fp64 oracle evaluated on the dequantized K/V within 4e-3.  Slots nobody
  wrote hold NaN codes (0x7F) and NaN scales, so a stray read shows up.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA
from oracle import fp8 as F8

from harness import TOL, dev

pytestmark = pytest.mark.gpu


def _f32(t):
    return t.float().cpu().numpy()


def _deq(x):
    """Oracle codes, scales and fp64 dequantized values of bf16 rows [..., d]."""
    codes, scale = F8.quantize_rows(_f32(x))
    return codes, scale, F8.dequantize_rows(codes, scale)


class Fp8Pool:
    def __init__(self, lens, hkv, d, W, seed, C=None, extra_steps=8):
        B = len(lens)
        self.B, self.W, self.hkv, self.d = B, W, hkv, d
        self.C = C or 16 * (-(-W // 16))
        self.maxp = (max(lens) + extra_steps * 4) // 16 + 2
        self.npages = B * self.maxp + 5
        free = synth.permutation(self.npages, seed, 1)
        ring = synth.permutation(B * self.C // 16, seed, 2)
        self.pool = H.hswa_pool_create(W, self.C, B, self.maxp, self.npages, free, ring,
                                       device=dev())
        self.view = H.hswa_pool_get_view(self.pool)
        self.full = H.kv_cache_alloc_fp8(self.npages, hkv, d, dev(), 0x7F)
        self.swa = H.kv_cache_alloc_fp8(B * self.C // 16, hkv, d, dev(), 0x7F)
        self.ids = list(range(B))
        self.sid = torch.tensor(self.ids, dtype=torch.int32, device=dev())
        H.hswa_pool_import(self.pool, self.ids, lens)

    def bufs(self, kind):
        return self.full if kind == H.FULL else self.swa

    def append_context(self, k, v, lens):
        for kind in (H.FULL, H.SWA):
            cnt = H.hswa_pool_window_counts(self.pool, kind, self.ids).tolist()
            live = [b for b in self.ids if cnt[b] > 0]
            if not live:
                continue
            cu = torch.tensor(np.concatenate([[0], np.cumsum([cnt[b] for b in live])]),
                              dtype=torch.int32, device=dev())
            kc, vc, ks, vs = self.bufs(kind)
            H.hswa_append_kv(kind,
                             torch.cat([k[b][lens[b] - cnt[b]:lens[b]] for b in live]).to(dev()),
                             torch.cat([v[b][lens[b] - cnt[b]:lens[b]] for b in live]).to(dev()),
                             torch.tensor(live, dtype=torch.int32, device=dev()), self.view,
                             kc, vc, cu, max(cnt), k_scale=ks, v_scale=vs)

    def slot(self, kind, b, pos):
        if kind == H.FULL:
            t = H.hswa_pool_read_tables(self.pool)
            return int(t["fpt"][b][pos // 16]) * 16 + pos % 16
        ring = self.pool.tables["rpt"].cpu().view(self.B, self.C // 16)
        r = pos % self.C
        return int(ring[b][r // 16]) * 16 + r % 16


@pytest.mark.parametrize("d,hkv", [(128, 8), (64, 2)])
def test_quantizing_append_matches_oracle(gpu, d, hkv):
    lens = [700, 1, 17, 128, 130, 33]
    W = 128
    k = [synth.bf16_normal((L, hkv, d), 5, 0, b, synth.ROLE_K) for b, L in enumerate(lens)]
    v = [synth.bf16_normal((L, hkv, d), 5, 0, b, synth.ROLE_V) for b, L in enumerate(lens)]
    # a few rows scaled far down and one all-zero row: subnormal codes, zero scale
    k[0][3] *= 1e-4
    v[2][5] = 0
    _check_quantizing_append(lens, hkv, d, W, 5, k, v)


@pytest.mark.parametrize("case", range(8))
def test_quantizing_append_random_configuration(gpu, case):
    """Seeded random shapes: KV heads 1-12, d, window 1-200 (rings down to
    one page), 1-6 sequences of 1-1,500 tokens (partial page tiles)."""
    import random
    rnd = random.Random(9900 + case)
    hkv, d = rnd.choice([1, 2, 3, 8, 12]), rnd.choice([64, 128])
    W = rnd.choice([1, 2, 5, 33, 128, 200])
    lens = [rnd.randint(1, 1500) for _ in range(rnd.randint(1, 6))]
    print(f"case {case}: hkv {hkv} d {d} W {W} lens {lens}", flush=True)
    k = [synth.bf16_normal((L, hkv, d), 60 + case, 0, b, synth.ROLE_K) for b, L in enumerate(lens)]
    v = [synth.bf16_normal((L, hkv, d), 60 + case, 0, b, synth.ROLE_V) for b, L in enumerate(lens)]
    _check_quantizing_append(lens, hkv, d, W, 60 + case, k, v)


def _check_quantizing_append(lens, hkv, d, W, seed, k, v):
    """Codes and scales of every stored position equal the oracle
    quantizer's, bit for bit, in both the Full pages and the SWA ring."""
    P = Fp8Pool(lens, hkv, d, W, seed)
    P.append_context(k, v, lens)
    torch.cuda.synchronize()
    for kind in (H.FULL, H.SWA):
        kc, vc, ks, vs = (t.cpu() for t in P.bufs(kind))
        for b, L in enumerate(lens):
            lo = 0 if kind == H.FULL else max(0, L - W + 1)
            kcode, kscale, _ = _deq(k[b][lo:L])
            vcode, vscale, _ = _deq(v[b][lo:L])
            for j, pos in enumerate(range(lo, L)):
                s = P.slot(kind, b, pos)
                pg, off = s // 16, s % 16
                assert np.array_equal(kc[pg, :, off, :].numpy(), kcode[j]), (kind, b, pos)
                assert np.array_equal(vc[pg, :, :, off].numpy(), vcode[j]), (kind, b, pos)
                assert np.array_equal(ks[pg, :, off].numpy().view(np.uint32),
                                      kscale[j].view(np.uint32)), (kind, b, pos)
                assert np.array_equal(vs[pg, :, off].numpy().view(np.uint32),
                                      vscale[j].view(np.uint32)), (kind, b, pos)


def _fp8_decode_scenario(ctxs, steps, hq, hkv, d, W, seed, max_rows=1):
    B = len(ctxs)
    C = 16 * max(-(-(W - 1 + max_rows) // 16), -(-W // 16))
    P = Fp8Pool(ctxs, hkv, d, W, seed, C=C, extra_steps=steps)
    k = [synth.bf16_normal((c + steps * max_rows, hkv, d), seed, 0, b, synth.ROLE_K)
         for b, c in enumerate(ctxs)]
    v = [synth.bf16_normal((c + steps * max_rows, hkv, d), seed, 0, b, synth.ROLE_V)
         for b, c in enumerate(ctxs)]
    P.append_context(k, v, ctxs)
    lens = list(ctxs)
    worst = 0.0
    for t in range(steps):
        n = [1] * B if max_rows == 1 else synth.uniform_ints(B, 1, max_rows, seed, t, 0)
        H.hswa_pool_alloc(P.pool, P.ids, n)
        rows = [(b, lens[b], lens[b] + n[b]) for b in P.ids]
        q = synth.bf16_normal((sum(n), hq, d), seed, 100 + t, 0, synth.ROLE_Q)
        kn = torch.cat([k[b][a:e] for b, a, e in rows])
        vn = torch.cat([v[b][a:e] for b, a, e in rows])
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        maxlen = max(e for _, _, e in rows)
        for kind in (H.FULL, H.SWA):
            kc, vc, ks, vs = P.bufs(kind)
            out = torch.full((sum(n), hq, d), float("nan"), dtype=torch.float32, device=dev())
            vl = torch.full((sum(n),), -1, dtype=torch.int32, device=dev())
            nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen, total_q=sum(n))
            ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
            kw = dict(cu_q=cu, max_q_len=max(n)) if max_rows > 1 else {}
            H.hswa_decode(kind, W, q.to(dev()), kn.to(dev()), vn.to(dev()), P.sid, maxlen,
                          P.view, kc, vc, out, ws, vl, k_scale=ks, v_scale=vs, **kw)
            got = out.cpu().double().numpy()
            o = 0
            for b, a, e in rows:
                _, _, kd = _deq(k[b][:e])
                _, _, vd = _deq(v[b][:e])
                exp = OA.attend(synth.to_f64(q[o:o + e - a]), range(a, e), kd, vd, kind, W)
                assert np.all(np.isfinite(got[o:o + e - a])), (t, kind, b)
                err = float(np.max(np.abs(got[o:o + e - a] - exp)))
                worst = max(worst, err)
                assert err < TOL, f"step {t} kind {kind} seq {b}: {err:.3e}"
                o += e - a
            assert vl.cpu().tolist() == [OA.valid_length(p, kind, W)
                                         for b, a, e in rows for p in range(a, e)]
        H.hswa_pool_evict(P.pool, P.ids)
        lens = [e for _, _, e in rows]
    return worst


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_fp8_decode_gqa(gpu, g):
    hkv = 2 if g < 8 else 8
    _fp8_decode_scenario([900, 1, 130, 2500, 127], 3, g * hkv, hkv, 128, 128, 40 + g)


def test_fp8_decode_long_split(gpu):
    _fp8_decode_scenario([20000, 6000, 50], 2, 64, 8, 128, 128, 51)


def test_fp8_decode_d64(gpu):
    _fp8_decode_scenario([1500, 90, 700], 3, 8, 2, 64, 128, 52)


def test_fp8_multi_row_decode(gpu):
    _fp8_decode_scenario([3000, 40, 129, 9000], 3, 64, 8, 128, 128, 53, max_rows=4)


@pytest.mark.parametrize("g,rows", [(2, 4), (4, 2), (1, 4), (8, 1)])
def test_fp8_head_pairs_multi_row(gpu, g, rows):
    """Full layers with split-K and an even KV head count decode both heads
    of a pair in one workgroup; these shapes (G x rows <= 8) cover every
    column layout of that path, with ragged rows and contexts that cross
    splits."""
    _fp8_decode_scenario([5000, 40, 2100, 1, 3333], 2, g * 4, 4, 128, 128, 70 + g,
                         max_rows=rows)


@pytest.mark.parametrize("kind,hint", [(H.FULL, 2), (H.FULL, 4096), (H.SWA, 2)])
def test_decode_reads_every_e4m3_code_exactly(gpu, kind, hint):
    """Every finite e4m3 code, through the decode path, comes back as its
    exact value.  One stored key's V codes are all 254 finite codes (two KV
    heads x 128 dims) with V scale 1; its K codes are 448 and Q is all ones,
    so its score exceeds the new token's (K = 0) by thousands and its weight
    is 1 while the new token's is 0.  The output is then that key's V, code
    by code, bit for bit (the fp16 weight 2^8 and the final 2^-8 are exact).
    The Full layer with a length hint of 4,096 takes split-K over both KV
    heads at once, with the combine."""
    hkv, d, W = 2, 128, 128
    P = Fp8Pool([1], hkv, d, W, 61)
    codes = np.arange(256, dtype=np.uint8).reshape(hkv, d)
    codes[(codes & 0x7F) == 0x7F] &= 0x80     # the two NaN codes -> +-0
    kc, vc, ks, vs = P.bufs(kind)
    s = P.slot(kind, 0, 0)
    pg, off = s // 16, s % 16
    kc[pg, :, off, :] = 0x7E
    vc[pg, :, :, off] = torch.as_tensor(codes, device=dev())
    ks[pg, :, off] = 1.0
    vs[pg, :, off] = 1.0
    H.hswa_pool_alloc(P.pool, [0], [1])
    q = torch.ones((1, hkv, d), dtype=torch.bfloat16, device=dev())
    zero = torch.zeros((1, hkv, d), dtype=torch.bfloat16, device=dev())
    out = torch.full((1, hkv, d), float("nan"), dtype=torch.float32, device=dev())
    nb = H.hswa_decode_workspace_bytes(kind, W, 1, hkv, hkv, d, hint)
    assert (nb > 0) == (hint > 2)
    ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
    H.hswa_decode(kind, W, q, zero, zero, P.sid, hint, P.view, kc, vc, out, ws,
                  k_scale=ks, v_scale=vs)
    want = F8.E4M3_TABLE[codes].astype(np.float32)
    got = out.cpu().numpy()[0]
    assert np.array_equal(got.view(np.uint32) & 0x7FFFFFFF, want.view(np.uint32) & 0x7FFFFFFF) \
        and np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("case", range(16))
def test_fp8_decode_random_configuration(gpu, case):
    """Seeded random shapes: contexts 1-3,000 tokens, GQA group, KV heads
    1-3, d, window 1-200 (rings down to one page), 1-4 rows per sequence."""
    import random
    rnd = random.Random(9100 + case)
    g, hkv = rnd.choice([1, 2, 4, 8]), rnd.choice([1, 2, 3])
    d, W = rnd.choice([64, 128]), rnd.choice([1, 2, 5, 33, 128, 200])
    ctxs = [rnd.randint(1, 3000) for _ in range(rnd.randint(1, 5))]
    steps, rows = rnd.randint(1, 3), rnd.choice([1, 2, 3, 4])
    print(f"case {case}: g {g} hkv {hkv} d {d} W {W} ctxs {ctxs} steps {steps} rows {rows}",
          flush=True)
    _fp8_decode_scenario(ctxs, steps, g * hkv, hkv, d, W, 300 + case, max_rows=rows)
