"""GPU checks of fp16 attention outputs (out_dtype = HSWA_OUT_F16).

The kernels compute exactly as for fp32 outputs and round once at the
store, so an fp16 output must equal the fp32 output of the same call rounded
to nearest-even, bit for bit, and stay within 4e-3 of the fp64 oracle.
Covered: SWA and Full chunked prefill (ragged tails, d 64 and 128), plain,
multi-row and split-K decode, FP8 pages.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA

from harness import TOL, Setup, chunked_prefill, dev, make_seqs, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", [H.SWA, H.FULL])
def test_prefill_f16_out(gpu, kind, d):
    hq, hkv, W, chunk = 16, 2, 128, 192
    lens = [450, 77, 1]
    seqs = make_seqs(lens, hq, hkv, d, 90 + d)
    maxp = max(lens) // 16 + 2
    res = {}
    for dt in (torch.float32, torch.float16):
        st = Setup(kind, W, W + chunk, len(lens), maxp, len(lens) * maxp + 3, hkv, d, 9)
        res[dt], vl, _ = chunked_prefill(st, seqs, chunk, hq, out_dtype=dt)
    for b, s in enumerate(seqs):
        a32, a16 = res[torch.float32][b], res[torch.float16][b]
        assert torch.equal(a16.view(torch.int16), a32.half().view(torch.int16)), b
        exp = oracle_rows(s, list(range(lens[b])), kind, W)
        err = float(np.max(np.abs(a16.double().numpy() - exp)))
        assert err < TOL, (b, err)


def _decode_pair(kind, rows, fp8):
    hq, hkv, d, W = 64, 8, 128, 128
    ctxs = [9000, 300, 17, 2500]
    B = len(ctxs)
    C = 16 * (-(-(W - 1 + rows) // 16))
    maxp = (max(ctxs) + rows) // 16 + 2
    npages = B * maxp + 4
    pool = H.hswa_pool_create(W, C, B, maxp, npages, synth.permutation(npages, 3, 1),
                              synth.permutation(B * C // 16, 3, 2), device=dev())
    view = H.hswa_pool_get_view(pool)
    n_pages = npages if kind == H.FULL else B * C // 16
    if fp8:
        kc, vc, ks, vs = H.kv_cache_alloc_fp8(n_pages, hkv, d, dev(), 0x7F)
    else:
        (kc, vc), ks, vs = H.kv_cache_alloc(n_pages, hkv, d, dev(), float("nan")), None, None
    ids = list(range(B))
    sid = torch.tensor(ids, dtype=torch.int32, device=dev())
    H.hswa_pool_import(pool, ids, ctxs)
    cnt = H.hswa_pool_window_counts(pool, kind, ids).tolist()
    k = [synth.bf16_normal((c + rows, hkv, d), 4, 0, b, synth.ROLE_K) for b, c in enumerate(ctxs)]
    v = [synth.bf16_normal((c + rows, hkv, d), 4, 0, b, synth.ROLE_V) for b, c in enumerate(ctxs)]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(cnt)]), dtype=torch.int32, device=dev())
    H.hswa_append_kv(kind, torch.cat([k[b][c - n:c] for b, (c, n) in enumerate(zip(ctxs, cnt))]).to(dev()),
                     torch.cat([v[b][c - n:c] for b, (c, n) in enumerate(zip(ctxs, cnt))]).to(dev()),
                     sid, view, kc, vc, cu, max(cnt), k_scale=ks, v_scale=vs)
    H.hswa_pool_alloc(pool, ids, [rows] * B)
    T = rows * B
    q = synth.bf16_normal((T, hq, d), 4, 1, 0, synth.ROLE_Q).to(dev())
    kn = torch.cat([k[b][c:c + rows] for b, c in enumerate(ctxs)]).to(dev())
    vn = torch.cat([v[b][c:c + rows] for b, c in enumerate(ctxs)]).to(dev())
    maxlen = max(ctxs) + rows
    nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen, total_q=T)
    ws = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
    kw = dict(cu_q=torch.arange(0, T + 1, rows, dtype=torch.int32, device=dev()),
              max_q_len=rows) if rows > 1 else {}
    outs = {}
    for i, dt in enumerate((torch.float32, torch.float16)):
        out = torch.full((T, hq, d), float("nan"), dtype=dt, device=dev())
        # the first call appends the new rows, the second reads them
        H.hswa_decode(kind, W, q, kn if i == 0 else None, vn if i == 0 else None, sid, maxlen,
                      view, kc, vc, out, ws, k_scale=ks, v_scale=vs, **kw)
        outs[dt] = out.cpu()
    assert torch.equal(outs[torch.float16].view(torch.int16),
                       outs[torch.float32].half().view(torch.int16))
    if not fp8:
        for b, c in enumerate(ctxs):
            pos = list(range(c, c + rows))
            qq = synth.to_f64(q[b * rows:(b + 1) * rows])
            exp = OA.attend(qq, pos, synth.to_f64(k[b]), synth.to_f64(v[b]), kind, W)
            got = outs[torch.float16][b * rows:(b + 1) * rows].double().numpy()
            assert float(np.max(np.abs(got - exp))) < TOL


@pytest.mark.parametrize("kind", [H.FULL, H.SWA])
@pytest.mark.parametrize("rows", [1, 4])
@pytest.mark.parametrize("fp8", [False, True])
def test_decode_f16_out(gpu, kind, rows, fp8):
    _decode_pair(kind, rows, fp8)
