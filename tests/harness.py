"""Drives the library through its C ABI on scenarios shaped like the
workloads, and evaluates the oracle on the same seeded inputs.

The GPU side receives inputs drawn by ``synth``; the oracle receives the very
same numbers as contiguous per-sequence arrays.  Nothing the GPU computes is
ever fed to the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

import hybrid_sliding_window_hswa_amd as H
import synth
from oracle import attention as OA

TOL = 4e-3  # max-abs error allowed against the fp64 oracle for bf16 inputs


def dev():
    return torch.device("cuda:0")


@dataclasses.dataclass
class SeqData:
    q: torch.Tensor  # [L, Hq, d] bf16 (cpu)
    k: torch.Tensor  # [L, Hkv, d] bf16 (cpu)
    v: torch.Tensor


def make_seqs(lengths, hq, hkv, d, seed, layer=0) -> List[SeqData]:
    out = []
    for b, L in enumerate(lengths):
        out.append(SeqData(
            synth.bf16_normal((L, hq, d), seed, layer, b, synth.ROLE_Q),
            synth.bf16_normal((L, hkv, d), seed, layer, b, synth.ROLE_K),
            synth.bf16_normal((L, hkv, d), seed, layer, b, synth.ROLE_V)))
    return out


def oracle_rows(s: SeqData, positions, kind, window, scale=None, fp8=False):
    """The oracle's rows at `positions`; fp8: over the values FP8 pages hold
    for the sequence's K/V (each row quantized, code times scale)."""
    q = synth.to_f64(s.q[positions])
    if fp8:
        from oracle import fp8 as F8
        k, v = (F8.dequantize_rows(*F8.quantize_rows(x.float().numpy())) for x in (s.k, s.v))
    else:
        k, v = synth.to_f64(s.k), synth.to_f64(s.v)
    return OA.attend(q, positions, k, v, kind, window, scale)


class Setup:
    """A pool with device tables plus one layer's K/V buffers."""

    def __init__(self, kind, window, ring_slots, max_seqs, max_pages, num_full_pages, hkv, d,
                 seed, poison=True, fp8=False):
        self.kind, self.W, self.C = kind, window, ring_slots
        self.hkv, self.d = hkv, d
        free = synth.permutation(num_full_pages, seed, 1)
        ring = synth.permutation(max_seqs * ring_slots // 16, seed, 2)
        self.pool = H.hswa_pool_create(window, ring_slots, max_seqs, max_pages, num_full_pages,
                                       free, ring, device=dev())
        self.view = H.hswa_pool_get_view(self.pool)
        npages = num_full_pages if kind == H.FULL else max_seqs * ring_slots // 16
        self.fp8 = fp8
        if fp8:   # codes 0x7F (NaN) and NaN scales, or zeros
            self.kc, self.vc, self.ks, self.vs = H.kv_cache_alloc_fp8(
                npages, hkv, d, dev(), 0x7F if poison else 0)
            if not poison:
                self.ks.zero_()
                self.vs.zero_()
        else:
            self.kc, self.vc = H.kv_cache_alloc(npages, hkv, d, dev(),
                                                float("nan") if poison else 0.0)
            self.ks = self.vs = None
        self.ring_pages = ring.reshape(max_seqs, ring_slots // 16)

    def scales(self):
        """Keyword arguments naming the FP8 scale arrays (none for BF16)."""
        return dict(k_scale=self.ks, v_scale=self.vs) if self.fp8 else {}

    def poison_ring_positions(self, b, positions):
        """NaN into the ring slots of positions that just left the window."""
        if self.kind != H.SWA or len(positions) == 0:
            return
        r = np.asarray(positions) % self.C
        pages = torch.as_tensor(self.ring_pages[b][r // 16].astype(np.int64), device=dev())
        offs = torch.as_tensor((r % 16).astype(np.int64), device=dev())
        if self.fp8:
            self.kc[pages, :, offs, :] = 0x7F
            self.vc[pages, :, :, offs] = 0x7F
            self.ks[pages, :, offs] = float("nan")
            self.vs[pages, :, offs] = float("nan")
        else:
            self.kc[pages, :, offs, :] = float("nan")
            self.vc[pages, :, :, offs] = float("nan")


def chunked_prefill(setup: Setup, seqs: List[SeqData], chunk: int, hq: int,
                    scale: float = 0.0, seq_ids=None, poison_evicted=True,
                    out_dtype=torch.float32):
    """Prefills every sequence in chunks; returns per-sequence fp32 outputs
    [L, Hq, d] (cpu), valid lengths and the host-side slot logs."""
    d = setup.d
    B = len(seqs)
    ids = list(range(B)) if seq_ids is None else list(seq_ids)
    lens = [s.q.shape[0] for s in seqs]
    outs = [torch.empty((L, hq, d), dtype=out_dtype) for L in lens]
    vlens = [torch.empty(L, dtype=torch.int32) for L in lens]
    log = {"alloc": [], "evict": []}
    done = [0] * B
    while True:
        act = [b for b in range(B) if done[b] < lens[b]]
        if not act:
            break
        n = [min(chunk, lens[b] - done[b]) for b in act]
        full, swa = H.hswa_pool_alloc(setup.pool, [ids[b] for b in act], n)
        log["alloc"].append((full, swa))
        rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
        q = torch.cat([seqs[b].q[a:e] for b, a, e in rows]).to(dev())
        kn = torch.cat([seqs[b].k[a:e] for b, a, e in rows]).to(dev())
        vn = torch.cat([seqs[b].v[a:e] for b, a, e in rows]).to(dev())
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev())
        sid = torch.tensor([ids[b] for b in act], dtype=torch.int32, device=dev())
        out = torch.full((q.shape[0], hq, d), float("nan"), dtype=out_dtype, device=dev())
        vl = torch.full((q.shape[0],), -7, dtype=torch.int32, device=dev())
        H.hswa_prefill_chunk(setup.kind, setup.W, q, kn, vn, sid, cu, max(n), setup.view,
                             setup.kc, setup.vc, out, vl, scale, **setup.scales())
        ev, cnt = H.hswa_pool_evict(setup.pool, [ids[b] for b in act])
        log["evict"].append((ev, cnt))
        torch.cuda.synchronize()
        out_c, vl_c = out.cpu(), vl.cpu()
        o = 0
        for (b, a, e), c in zip(rows, cnt):
            outs[b][a:e] = out_c[o:o + e - a]
            vlens[b][a:e] = vl_c[o:o + e - a]
            o += e - a
            if poison_evicted and c > 0:
                first = e - setup.W + 1 - c  # evicted positions end at e - W
                setup.poison_ring_positions(ids[b], list(range(first, first + c)))
        for b, k in zip(act, n):
            done[b] += k
    return outs, vlens, log
