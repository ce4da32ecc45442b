"""Decode calls captured in a HIP graph and replayed.

A serving loop can capture its launch-bound decode calls once and replay
them every step.  The decode path allocates nothing inside the call and
records no memset: the split-K work queue's counters are cleared by the
queue pre-pass kernel's own stores, and hswa_decode_noalloc keeps its state
in the library's device scratch.  Here a Full layer (split-K over the work
queue, then the combine) and a SWA layer, on bf16 and FP8 pages, with a
caller workspace or none, are captured once; each of several replays, with
eager decode calls and synchronizations between them, must equal the eager
result bit for bit.  Each call appends the step's new key (the same rows
every time, so the pages end up unchanged) and attends.
"""
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H
import synth

from harness import dev
from test_fp8_transfer_gpu import CopyPool

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_decode_replays_from_a_hip_graph(gpu, fp8, noalloc):
    hq, hkv, d, W = 64, 8, 128, 128
    ctxs = [5000, 40, 2100, 777, 3000]
    B = len(ctxs)
    P = CopyPool(ctxs, hkv, d, W, 16 * (-(-W // 16)), 177, fp8)
    sid = torch.arange(B, dtype=torch.int32, device=dev())
    # one decode step: the new position's slots, then each call appends its
    # key (the same rows every time) and attends
    H.hswa_pool_alloc(P.pool, list(range(B)), [1] * B)
    q = synth.bf16_normal((B, hq, d), 178, 0, 0, synth.ROLE_Q).to(dev())
    kn = synth.bf16_normal((B, hkv, d), 178, 0, 0, synth.ROLE_K).to(dev())
    vn = synth.bf16_normal((B, hkv, d), 178, 0, 0, synth.ROLE_V).to(dev())
    maxlen = max(ctxs) + 1
    ws = {}
    for kind in (H.FULL, H.SWA):
        nb = H.hswa_decode_workspace_bytes(kind, W, B, hq, hkv, d, maxlen)
        ws[kind] = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev())
    assert ws[H.FULL].numel() > 1, "the Full call should take split-K"

    def decode(kind, out):
        bufs = P.layers[kind]
        sc = dict(k_scale=bufs[2], v_scale=bufs[3]) if fp8 else {}
        if noalloc:
            H.hswa_decode_noalloc(kind, W, q, kn, vn, sid, maxlen, P.view, bufs[0], bufs[1],
                                  out, **sc)
        else:
            H.hswa_decode(kind, W, q, kn, vn, sid, maxlen, P.view, bufs[0], bufs[1], out,
                          ws[kind], **sc)

    def fresh():
        return {kind: torch.full((B, hq, d), float("nan"), dtype=torch.float32, device=dev())
                for kind in (H.FULL, H.SWA)}

    want = fresh()
    for kind in (H.FULL, H.SWA):
        decode(kind, want[kind])
    torch.cuda.synchronize()
    assert all(bool(torch.all(torch.isfinite(w))) for w in want.values())

    got = fresh()
    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream
        for kind in (H.FULL, H.SWA):
            decode(kind, got[kind])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for kind in (H.FULL, H.SWA):
            decode(kind, got[kind])
    for replay in range(3):
        for kind in (H.FULL, H.SWA):
            got[kind].fill_(float("nan"))
        other = fresh()                  # eager calls between replays
        for kind in (H.FULL, H.SWA):
            decode(kind, other[kind])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for kind in (H.FULL, H.SWA):
            assert torch.equal(got[kind], want[kind]), (replay, kind)
            assert torch.equal(other[kind], want[kind]), (replay, kind)
    del g
