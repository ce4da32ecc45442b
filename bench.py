"""Benchmark of the Hybrid SWA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workloads (all inputs seeded synthetic N(0,1) values rounded to bf16,
resident in HBM before the timed region starts):

  swa_chunked_prefill (default)
      SWA-only chunked prefill: 8 sequences with lengths uniform in
      [2048, 16384], chunk 2048, 64 query / 8 KV heads, head_dim 128, W = 128,
      a ring of W + chunk slots per sequence in 16-token pages placed by a
      seeded random permutation.  One step = the whole chunked prefill of the
      batch: for every chunk, pool alloc (joint capacity check + device table
      update), KV append, SWA attention, out-of-window eviction; then release.
      `value` = prefill tokens/s.  The same run measures the other four
      configurations and embeds each, with its own roofline and oracle
      baseline: the mixed decode under "decode", the single-chunk run under
      "single_chunk", the 70-layer stack under "hybrid_stack" and the
      long-context decode under "long_decode" (--headline-only skips the
      last three).
  mixed_decode
      256 sequences, contexts uniform in [4096, 32768], one Full layer (paged
      Full pool, 16-token pages in random order) and one SWA layer (ring of
      W = 128 slots); one step = alloc one token per sequence, append + attend
      both layers, evict.  `value` = algorithmic HBM GB/s.
  hybrid_stack
      70 attention-only layers (6 SWA then 1 Full, repeated), one 65536-token
      sequence prefilled in 4096-token chunks, and the same with all 70 layers
      Full.  `value` = stack tokens/s; the Full-layer kernel is MFMA-bound.
  long_decode
      64 sequences, contexts uniform in [131072, 262144], 14 layers (6 SWA then
      1 Full, twice), SWA ring of W + 256 slots.  `value` = HBM GB/s.
  mixed_decode_fp8
      The mixed decode over FP8 pages (e4m3 codes with an fp32 scale per
      token and head, quantized by the append): half the K/V bytes per key.
      `value` = algorithmic HBM GB/s of the FP8 bytes.
  swa_chunked_prefill_fp8
      swa_chunked_prefill over FP8 pages: the appends quantize each chunk,
      the attention reads codes and scales.  `value` = tokens/s.
  mtp_decode
      Multi-token decode: the mixed decode's 256 sequences with one token
      plus three draft tokens per step (rows of a sequence share every K/V
      byte read); the step keeps a seeded accepted prefix (truncate) before
      evicting.  `value` = algorithmic HBM GB/s.
  mtp_decode_fp8
      mtp_decode over FP8 pages (32 (row, head) columns per KV head: the
      two-tile kernel).  `value` = algorithmic HBM GB/s of the FP8 bytes.
  tier_transfer
      Window-masked offload and restore of a 14-layer hybrid stack's KV
      (16 sequences, contexts 4096-32768) through pinned host memory: SWA
      layers move only their W-1-token windows.  `value` = restore GB/s over
      PCIe; also offload GB/s and restore + first decode step, serial versus
      pulled layer by layer on a second stream.
  tier_transfer_fp8
      tier_transfer over FP8 pages: the buffers hold code bytes and the fp32
      scale of each (token, head), 2 * Hkv * (d + 4) bytes per token instead
      of 4 * Hkv * d.  `value` = restore GB/s of those bytes.
  tp8_share
      One GPU's share of an 8-way KV-head split: the default run's prefill
      and mixed decode with 8 query heads and 1 KV head (the same lengths,
      chunk, W and contexts).  `value` = prefill tokens/s of the share; the
      decode under "decode".
  swa_single_chunk
      One SWA layer, one 1024-token sequence (8 query / 2 KV heads, head_dim
      64) prefilled in one chunk, then 16 decode steps.  `value` = tok/s.

The dominant kernel's duration is measured with HIP events recorded on the
stream it is launched on; `roofline.achieved` = algorithmic bytes (or flops)
per launch / that duration.  `roofline.traffic` is the measured HBM bytes
per launch from rocprofv3 counters (profiles/traffic.json), given only when
they were taken on the current kernel source, else null.

`cpu_baseline` is the oracle (fp64 NumPy, untuned, one thread) timed on a
bounded sample of the same workload, with the host's core count and NumPy's
default BLAS thread count recorded beside it.  `dtype` names the MFMA input
types; `precision` spells out the type of every stage.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
PCIE_PEAK_GBS = 63.0           # PCIe 5.0 x16, one direction: 32 GT/s * 16 lanes * 128/130 / 8
MFMA_BF16_PEAK_TFS = 2516.6    # 256 CU * 2.4 GHz * 4096 flop/clk (dense)
PEAKS = {"hbm": (HBM_PEAK_GBS, "GB/s"), "mfma": (MFMA_BF16_PEAK_TFS, "TFLOP/s"),
         "pcie": (PCIE_PEAK_GBS, "GB/s")}
METRIC = "Hybrid-SWA attn prefill tok/s + decode HBM GB/s (% of MI355X peak)"
ODT = {"f32": "fp32", "f16": "fp16"}

CSRC = os.path.join(ROOT, "hybrid_sliding_window_hswa_amd", "csrc")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def KV_TOKEN_BYTES(hkv, d):
    return 2 * hkv * d * 2  # K (bf16) and V (fp16) of one token


# headers every kernel source includes: a change to them changes the kernels
KERNEL_HEADERS = ("device.h", "internal.h", "index.h")


def _code_only(text):
    """C++ source without its comments, whitespace runs collapsed: a change
    to comments or layout does not change the kernels (the sources hold no
    string literal with comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(fname):
    """SHA-256 over the code of a kernel source followed by the shared
    device headers (comments and layout excluded)."""
    h = hashlib.sha256()
    for name in (fname,) + KERNEL_HEADERS:
        with open(os.path.join(CSRC, name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(key, fname):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256") != source_sha(fname):
        return None
    return t.get("hbm_bytes_per_launch")


def measured_mfma_ops(key, fname):
    """MFMA ops (units of 512 flops, bf16 plus fp16) per launch from the
    committed counter summary, if it was taken on the current source of the
    kernel; else None."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)["mfma_ops"][key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256") != source_sha(fname):
        return None
    return t.get("mops_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------


class Ctx:
    """Holds torch, the binding and a stream for the run."""

    def __init__(self):
        import torch
        import hybrid_sliding_window_hswa_amd as H
        self.torch = torch
        self.H = H
        self.lib = H.library()
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        self.sptr = C.c_void_p(self.stream.cuda_stream)

    def i32(self, x):
        return self.torch.tensor(np.asarray(x, dtype=np.int32), device=self.dev)


def _arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def _attn_args(cx, kind, window, hq, hkv, d, seq_ids, cu_q, total_q, max_q_len, max_seq_len,
               view, q, k_new, v_new, kc, vc, out):
    from hybrid_sliding_window_hswa_amd import _capi
    a = _capi.AttnArgs()
    a.kind, a.window = kind, window
    a.num_q_heads, a.num_kv_heads, a.head_dim = hq, hkv, d
    a.scale = 0.0
    a.num_seqs = seq_ids.shape[0]
    a.seq_ids = seq_ids.data_ptr()
    a.cu_q = cu_q.data_ptr() if cu_q is not None else None
    a.total_q, a.max_q_len, a.max_seq_len = total_q, max_q_len, max_seq_len
    a.q = q.data_ptr() if q is not None else None
    a.k_new = k_new.data_ptr() if k_new is not None else None
    a.v_new = v_new.data_ptr() if v_new is not None else None
    a.pool = view
    a.k_cache, a.v_cache = kc.data_ptr(), vc.data_ptr()
    a.out = out.data_ptr() if out is not None else None
    # the output type must match the buffer: the kernels write 4 or 2 bytes
    # per element as out_dtype says
    if out is not None:
        if out.dtype == cx.torch.float16:
            a.out_dtype = 1
        elif out.dtype == cx.torch.float32:
            a.out_dtype = 0
        else:
            raise ValueError(f"output buffer must be float32 or float16, not {out.dtype}")
    a.vlen_out = None
    return a


def _check(cx, rc):
    if rc != 0:
        raise RuntimeError(f"hswa call failed ({rc}): {cx.H.hswa_last_error()}")


# ---------------------------------------------------------------------------
# SWA / Full chunked prefill over a batch of sequences


class ChunkedPrefill:
    """Precomputes every chunk step's batch; run() replays the whole chunked
    prefill of the batch through every layer via the C ABI.  `pattern` lists
    the layers ('S' SWA, 'F' Full), each with K/V buffers of its own; all
    layers see the same synthetic Q/K/V (an attention-only stack)."""

    def __init__(self, cx, lens, chunk, hq, hkv, d, W, seed, pattern="S", ring=None,
                 out="f32", one_stream=False, combine_pool_ops=True, fp8=False):
        torch, H = cx.torch, cx.H
        import synth
        self.cx = cx
        self.combine_pool_ops = combine_pool_ops
        self.fp8 = fp8
        self.obytes = 2 if out == "f16" else 4
        self.lens, self.chunk, self.hq, self.hkv, self.d, self.W = lens, chunk, hq, hkv, d, W
        B = len(lens)
        self.B = B
        C_ = ring or W + chunk
        C_ = -(-C_ // 16) * 16
        maxp = max(lens) // 16 + 2
        nfull = B * maxp + 16
        free = synth.permutation(nfull, seed, 1)
        ringp = synth.permutation(B * C_ // 16, seed, 2)
        self.pool = H.hswa_pool_create(W, C_, B, maxp, nfull, free, ringp, device=cx.dev)
        self.view = H.hswa_pool_get_view(self.pool)
        self.layers = []
        self.scales = []  # FP8 pages: (k_scale, v_scale) per layer
        for kind in pattern:
            npages = nfull if kind == "F" else B * C_ // 16
            if fp8:
                kc, vc, ks, vs = H.kv_cache_alloc_fp8(npages, hkv, d, cx.dev, 0)
                self.scales.append((ks, vs))
            else:
                kc, vc = H.kv_cache_alloc(npages, hkv, d, cx.dev, 0.0)
            self.layers.append((H.FULL if kind == "F" else H.SWA, kc, vc))
        # inputs per sequence, generated on the device
        self.q, self.k, self.v = [], [], []
        for b, L in enumerate(lens):
            self.q.append(synth.bf16_normal((L, hq, d), seed, 0, b, synth.ROLE_Q, device=cx.dev))
            self.k.append(synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_K, device=cx.dev))
            self.v.append(synth.bf16_normal((L, hkv, d), seed, 0, b, synth.ROLE_V, device=cx.dev))
        # chunk steps
        self.steps = []
        done = [0] * B
        max_rows = 0
        while True:
            act = [b for b in range(B) if done[b] < lens[b]]
            if not act:
                break
            n = [min(chunk, lens[b] - done[b]) for b in act]
            rows = [(b, done[b], done[b] + k) for b, k in zip(act, n)]
            cat = (lambda xs: xs[0]) if len(rows) == 1 else torch.cat
            st = {
                "ids": _arr(act), "n": _arr(n), "nseq": len(act), "max_n": max(n),
                "sid": cx.i32(act),
                "cu": cx.i32(np.concatenate([[0], np.cumsum(n)])),
                "qpos": cx.i32([done[b] for b in act]),
                "q": cat([self.q[b][a:e] for b, a, e in rows]),
                "k": cat([self.k[b][a:e] for b, a, e in rows]),
                "v": cat([self.v[b][a:e] for b, a, e in rows]),
                "rows": rows,
            }
            max_rows = max(max_rows, st["q"].shape[0])
            self.steps.append(st)
            for b, k in zip(act, n):
                done[b] += k
        self.out = torch.empty((max_rows, hq, d), device=cx.dev,
                               dtype=torch.float16 if out == "f16" else torch.float32)
        self.all_ids = _arr(list(range(B)))
        # An all-SWA stack passes each sequence's first row position (q_pos):
        # its appends and attention then read no pool table that alloc,
        # evict or release write, and those pool calls go to a second stream
        # (default priority) beside the attention, with no waits between the
        # streams.  Full layers read the Full page table that alloc writes,
        # so a stack with Full layers keeps one stream.
        self.side = None
        if "F" not in pattern and not one_stream:
            self.side_stream = torch.cuda.Stream()
            self.side = C.c_void_p(self.side_stream.cuda_stream)
        for st in self.steps:
            T = st["q"].shape[0]
            st["args"] = []
            for li, (kind, kc, vc) in enumerate(self.layers):
                app = _attn_args(cx, kind, W, hkv, hkv, d, st["sid"], st["cu"], T, st["max_n"],
                                 0, self.view, None, st["k"], st["v"], kc, vc, None)
                att = _attn_args(cx, kind, W, hq, hkv, d, st["sid"], st["cu"], T, st["max_n"],
                                 0, self.view, st["q"], None, None, kc, vc, self.out)
                if fp8:
                    ks, vs = self.scales[li]
                    for a in (app, att):
                        a.kv_dtype = H.HSWA_KV_FP8
                        a.k_scale, a.v_scale = ks.data_ptr(), vs.data_ptr()
                if "F" not in pattern:
                    app.q_pos = att.q_pos = st["qpos"].data_ptr()
                st["args"].append((app, att))
        self.tokens = sum(lens)

    def run(self, events=None):
        lib, cx = self.cx.lib, self.cx
        h = self.pool.handle
        ps = self.side or cx.sptr  # stream of the pool calls
        prev = None  # the previous chunk step's sequences, evicted at this step's start
        for st in self.steps:
            ids, idp = st["ids"]
            n, np_ = st["n"]
            if prev is None:
                _check(cx, lib.hswa_pool_alloc(h, st["nseq"], idp, np_, None, None, ps))
            elif self.combine_pool_ops:
                # the previous step's eviction and this step's alloc: one
                # table-update launch
                _check(cx, lib.hswa_pool_evict_alloc(h, prev[0], prev[1], None, 0, None,
                                                     st["nseq"], idp, np_, None, None, ps))
            else:
                _check(cx, lib.hswa_pool_evict(h, prev[0], prev[1], None, 0, None, ps))
                _check(cx, lib.hswa_pool_alloc(h, st["nseq"], idp, np_, None, None, ps))
            for app, att in st["args"]:
                _check(cx, lib.hswa_append_kv(C.byref(app), cx.sptr))
                if events is not None:
                    e0, e1 = cx.torch.cuda.Event(enable_timing=True), cx.torch.cuda.Event(
                        enable_timing=True)
                    e0.record(cx.stream)
                _check(cx, lib.hswa_prefill_chunk(C.byref(att), cx.sptr))
                if events is not None:
                    e1.record(cx.stream)
                    events.append((att.kind, st, e0, e1))
            prev = (st["nseq"], idp)
        if prev is not None:
            _check(cx, lib.hswa_pool_evict(h, prev[0], prev[1], None, 0, None, ps))
        ids, idp = self.all_ids
        _check(cx, lib.hswa_pool_release(h, self.B, idp, ps))

    def attn_bytes(self, st, kind):
        """Algorithmic HBM bytes of one attention launch: Q read (bf16), O
        written (fp32), and the K/V of each key the chunk needs read once
        (SWA: the chunk plus its W-1 halo; Full: the whole prefix)."""
        T = st["q"].shape[0]
        # FP8 pages: one code per element plus an fp32 scale per token and
        # head, for K and for V
        kvb = 2 * self.hkv * (self.d + 4) if self.fp8 else KV_TOKEN_BYTES(self.hkv, self.d)
        if kind == self.cx.H.FULL:
            keys = sum(e for b, a, e in st["rows"])
        else:
            keys = sum((e - a) + min(self.W - 1, a) for b, a, e in st["rows"])
        return T * self.hq * self.d * (2 + self.obytes) + keys * kvb

    def attn_flops(self, st, kind):
        """4 * d * Hq flops per scored (query, key) pair."""
        pairs = 0
        for b, a, e in st["rows"]:
            if kind == self.cx.H.SWA:
                pairs += _pairs_swa(e, self.W) - _pairs_swa(a, self.W)
            else:
                pairs += e * (e + 1) // 2 - a * (a + 1) // 2
        return 4 * self.d * self.hq * pairs


def _pairs_swa(n, W):
    return n * (n + 1) // 2 if n <= W else n * W - W * (W - 1) // 2


# ---------------------------------------------------------------------------
# Decode over Full + SWA layers


class Decode:
    """Decode steps over a layer pattern ("F" Full, "S" SWA).  rows = 1 is a
    plain decode step; rows > 1 verifies one token plus rows-1 drafts per
    sequence (multi-token decode), then keeps a seeded accepted prefix
    (hswa_pool_truncate) before the eviction."""

    def __init__(self, cx, ctxs, pattern, hq, hkv, d, W, ring, seed, steps_total, rows=1,
                 fill=True, fp8=False, out="f32"):
        torch, H = cx.torch, cx.H
        import synth
        self.cx, self.hq, self.hkv, self.d, self.W = cx, hq, hkv, d, W
        B = len(ctxs)
        self.B = B
        self.rows = rows
        self.fp8 = fp8
        self.obytes = 2 if out == "f16" else 4
        self.seed = seed
        self.ctx0 = list(ctxs)
        maxlen = max(ctxs) + steps_total * rows + 1
        maxp = maxlen // 16 + 2
        nfull = (int(sum(c // 16 + 2 for c in ctxs) * 1.1) + B * (steps_total * rows // 16 + 2)
                 + 64)
        free = synth.permutation(nfull, seed, 1)
        ringp = synth.permutation(B * ring // 16, seed, 2)
        self.pool = H.hswa_pool_create(W, ring, B, maxp, nfull, free, ringp, device=cx.dev)
        self.view = H.hswa_pool_get_view(self.pool)
        ids = list(range(B))
        self.ids = _arr(ids)
        self.sid = cx.i32(ids)
        H.hswa_pool_import(self.pool, ids, ctxs, want_slots=False)
        self.layers = []
        self.scales = []
        for li, kind in enumerate(pattern):
            npg = nfull if kind == "F" else B * ring // 16
            if fp8:
                kc, vc, ks, vs = H.kv_cache_alloc_fp8(npg, hkv, d, cx.dev)
            else:
                (kc, vc), ks, vs = H.kv_cache_alloc(npg, hkv, d, cx.dev), None, None
            # restore the context: generated per sequence on the device and
            # appended (Full: every position, SWA: the last W-1)
            for b, c in (enumerate(ctxs) if fill else ()):
                n = c if kind == "F" else min(c, W - 1)
                kk = synth.bf16_normal((n, hkv, d), seed, li, b, synth.ROLE_K, device=cx.dev)
                vv = synth.bf16_normal((n, hkv, d), seed, li, b, synth.ROLE_V, device=cx.dev)
                H.hswa_append_kv(H.FULL if kind == "F" else H.SWA, kk, vv, cx.i32([b]), self.view,
                                 kc, vc, cx.i32([0, n]), n, k_scale=ks, v_scale=vs)
                del kk, vv
            self.layers.append((H.FULL if kind == "F" else H.SWA, kc, vc))
            self.scales.append((ks, vs))
            if fill and sum(ctxs) > (1 << 22):
                torch.cuda.synchronize()
                log(f"decode setup: layer {li + 1} of {len(pattern)} restored")
        torch.cuda.synchronize()
        # per-step inputs (rows new tokens per sequence per layer)
        T = B * rows
        g = lambda shape, *s: synth.bf16_normal(shape, seed, 900, *s, device=cx.dev)
        self.q = [g((T, hq, d), li, synth.ROLE_Q) for li in range(len(pattern))]
        self.kn = [g((T, hkv, d), li, synth.ROLE_K) for li in range(len(pattern))]
        self.vn = [g((T, hkv, d), li, synth.ROLE_V) for li in range(len(pattern))]
        self.out = torch.empty((T, hq, d), device=cx.dev,
                               dtype=torch.float16 if out == "f16" else torch.float32)
        self.max_seq_len = maxlen
        self.cu = cx.i32(np.arange(0, T + 1, rows)) if rows > 1 else None
        nb = max(H.hswa_decode_workspace_bytes(H.FULL, W, B, hq, hkv, d, maxlen, total_q=T), 16)
        self.ws = torch.empty(nb // 4 + 4, dtype=torch.float32, device=cx.dev)
        self.nbytes_ws = self.ws.numel() * 4
        self.args = []
        for li, (kind, kc, vc) in enumerate(self.layers):
            a = _attn_args(cx, kind, W, hq, hkv, d, self.sid, self.cu, T, rows, maxlen,
                           self.view, self.q[li], self.kn[li], self.vn[li], kc, vc, self.out)
            if fp8:
                a.kv_dtype = H.HSWA_KV_FP8
                a.k_scale = self.scales[li][0].data_ptr()
                a.v_scale = self.scales[li][1].data_ptr()
            self.args.append(a)
        self.lens = list(ctxs)
        self.pattern = pattern
        self.nrows = _arr([rows] * B)
        self.step_no = 0
        self.step_bytes = []     # algorithmic bytes of every step run
        self.accepted = []       # tokens kept by every step

    def step(self, events=None):
        lib, cx, H = self.cx.lib, self.cx, self.cx.H
        h = self.pool.handle
        ids, idp = self.ids
        _, np_ = self.nrows
        _check(cx, lib.hswa_pool_alloc(h, self.B, idp, np_, None, None, cx.sptr))
        self.lens = [x + self.rows for x in self.lens]
        for a in self.args:
            if events is not None:
                e0, e1 = cx.torch.cuda.Event(enable_timing=True), cx.torch.cuda.Event(
                    enable_timing=True)
                e0.record(cx.stream)
            _check(cx, lib.hswa_decode(C.byref(a), C.c_void_p(self.ws.data_ptr()),
                                       self.nbytes_ws, cx.sptr))
            if events is not None:
                e1.record(cx.stream)
                events.append((a.kind, list(self.lens), e0, e1))
        self.step_bytes.append(sum(self.layer_bytes(a.kind, self.lens) for a in self.args))
        if self.rows > 1:
            import synth
            acc = synth.uniform_ints(self.B, 1, self.rows, self.seed, 700, self.step_no)
            self.lens = [x - self.rows + k for x, k in zip(self.lens, acc)]
            keep, kp = _arr(self.lens)
            _check(cx, lib.hswa_pool_truncate(h, self.B, idp, kp, cx.sptr))
            self.accepted.append(sum(acc))
        else:
            self.accepted.append(self.B)
        self.step_no += 1
        _check(cx, lib.hswa_pool_evict(h, self.B, idp, None, 0, None, cx.sptr))

    def layer_bytes(self, kind, lens):
        """Algorithmic HBM bytes of one decode layer call at lengths `lens`
        (after the step's rows were allocated): the K/V of every key some row
        attends to, read once for all rows of the sequence (Full: L keys; SWA:
        the first row's window through the last row, min(L, W - 1 + rows)),
        Q read, O written (fp32 or fp16), and the rows' K/V read and written by the
        append."""
        kvb = KV_TOKEN_BYTES(self.hkv, self.d)
        # FP8 pages: one byte per K/V element plus an fp32 scale per token,
        # head and tensor; the append reads bf16 rows and writes FP8 ones
        kvs = 2 * self.hkv * (self.d + 4) if self.fp8 else kvb
        r = self.rows
        keys = sum(L if kind == self.cx.H.FULL else min(L, self.W - 1 + r) for L in lens)
        T = len(lens) * r
        return keys * kvs + T * (self.hq * self.d * (2 + self.obytes) + kvb + kvs)


# ---------------------------------------------------------------------------
# CPU baseline (the oracle, untuned)


def host_info():
    """Host cores this process may use and the BLAS thread count NumPy would
    use by default (the oracle is timed on one thread)."""
    info = {"host_cores": len(os.sched_getaffinity(0)), "blas_threads_default": None}
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
        info["blas_threads_default"] = max(n) if n else None
    except Exception:
        pass
    return info


def _one_thread():
    """Context that holds NumPy's BLAS to one thread (a no-op without
    threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def _baseline(value, unit, sample, dt):
    return {"value": round(value, 2), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{sample}; fp64 NumPy on 1 thread, {dt:.1f} s", **host_info()}


def cpu_baseline_prefill(cx, cp: ChunkedPrefill, budget_s: float, seed=7):
    """The oracle (fp64 NumPy, one thread) on a bounded sample of the same
    prefill: query rows drawn uniformly from the batch, each with all heads
    and its full window of keys.  Inputs are copied to the host first; only
    the oracle is timed."""
    import synth
    from oracle import attention as OA
    rng = np.random.default_rng(seed)
    W = cp.W

    def draw(k):
        out = []
        for _ in range(k):
            b = int(rng.integers(cp.B))
            pos = int(rng.integers(cp.lens[b]))
            lo = max(0, pos - W + 1)
            out.append((pos - lo, synth.to_f64(cp.q[b][pos:pos + 1]),
                        synth.to_f64(cp.k[b][lo:pos + 1]), synth.to_f64(cp.v[b][lo:pos + 1])))
        return out

    def run(sample):
        t0 = time.perf_counter()
        for rel, q, k, v in sample:
            OA.attend(q, [rel], k, v, OA.SWA, W)
        return time.perf_counter() - t0

    with _one_thread():
        per_row = run(draw(32)) / 32
        n = max(64, int(budget_s / max(per_row, 1e-6)))
        sample = draw(n)
        dt = run(sample)
    return _baseline(n / dt, "tok/s", f"{n} query rows (each with all {cp.hq} heads and its "
                     f"{W}-key window) drawn uniformly from the {cp.B} sequences", dt)


def cpu_baseline_single_chunk(cx, cp: ChunkedPrefill, dc_ctx, budget_s: float):
    """The oracle on the whole single-chunk workload: every prefill row of the
    sequence, then one row per decode step over its restored window, repeated
    until about budget_s of CPU time; tok/s over prefill plus decode rows."""
    import synth
    from oracle import attention as OA
    W, L = cp.W, cp.lens[0]
    q, k, v = (synth.to_f64(t) for t in (cp.q[0], cp.k[0], cp.v[0]))
    dq, dk, dv = dc_ctx  # decode rows [n, Hq, d] and their windows [n, W, Hkv, d]
    passes, dt = 0, 0.0
    with _one_thread():
        while passes < 1 or dt < budget_s:
            t0 = time.perf_counter()
            OA.attend(q, range(L), k, v, OA.SWA, W)
            for i in range(dq.shape[0]):
                OA.attend(dq[i:i + 1], [dk.shape[1] - 1], dk[i], dv[i], OA.SWA, W)
            dt += time.perf_counter() - t0
            passes += 1
    rows = L + dq.shape[0]
    return _baseline(rows * passes / dt, "tok/s",
                     f"the whole workload ({L} prefill rows + {dq.shape[0]} decode rows, all "
                     f"heads) x {passes} passes", dt)


def cpu_baseline_decode(cx, dc, sample_seqs, sample_layers, budget_s: float):
    """The oracle on sampled (sequence, layer) decode calls of the same
    workload: the first step's query row of each sampled sequence against its
    restored context plus the step's new key.  GB/s-equivalent = the calls'
    algorithmic bytes (as the GPU line counts them) / oracle time; every
    sampled sequence runs all sampled layers, in order, until the budget is
    spent (at least one sequence)."""
    import synth
    from oracle import attention as OA
    torch, H = cx.torch, cx.H
    W, hkv, d = dc.W, dc.hkv, dc.d
    done_bytes, dt, nseq, ncall = 0, 0.0, 0, 0
    for b in sample_seqs:
        ctx = dc.ctx0[b]
        for li in sample_layers:
            kind = dc.layers[li][0]
            n = ctx if kind == H.FULL else min(ctx, W - 1)
            kk = synth.bf16_normal((n, hkv, d), dc.seed, li, b, synth.ROLE_K, device=cx.dev)
            vv = synth.bf16_normal((n, hkv, d), dc.seed, li, b, synth.ROLE_V, device=cx.dev)
            k = synth.to_f64(torch.cat([kk, dc.kn[li][b:b + 1]]))
            v = synth.to_f64(torch.cat([vv, dc.vn[li][b:b + 1]]))
            q = synth.to_f64(dc.q[li][b:b + 1])
            del kk, vv
            with _one_thread():
                t0 = time.perf_counter()
                OA.attend(q, [n], k, v, kind, W)
                dt += time.perf_counter() - t0
            del k, v
            done_bytes += dc.layer_bytes(kind, [ctx + 1])
            ncall += 1
        nseq += 1
        if dt >= budget_s:
            break
    kinds = "".join("F" if dc.layers[li][0] == H.FULL else "S" for li in sample_layers)
    return _baseline(done_bytes / dt / 1e9, "GB/s",
                     f"{nseq} sequences (the shortest and longest context first, then seeded "
                     f"ones) x layers {kinds}: {ncall} calls of one query row with all heads",
                     dt)


def cpu_baseline_stack(cx, cp: ChunkedPrefill, pattern: str, budget_s: float, seed=13):
    """The oracle on sampled query rows of the 70-layer stack (every layer
    sees the same Q/K/V): Full rows at the chunk edges and seeded positions,
    SWA rows at seeded positions.  Time per scored pair is measured for each
    kind and scaled by the stack's pair counts, giving tok/s-equivalent of
    the hybrid stack and of the all-Full variant."""
    import synth
    from oracle import attention as OA
    N, W, chunk = cp.lens[0], cp.W, cp.chunk
    k, v = synth.to_f64(cp.k[0]), synth.to_f64(cp.v[0])
    rng = np.random.default_rng(seed)
    edges = [p for a in range(0, N, chunk) for p in (a, a + chunk - 1)]
    full_pos = [edges[0], edges[-1]] + [int(x) for x in rng.integers(0, N, 64)] + edges[1:-1]
    swa_pos = [int(x) for x in rng.integers(W, N, 4096)]
    res = {}
    with _one_thread():
        for kind, plist in ((OA.FULL, full_pos), (OA.SWA, swa_pos)):
            t, keys, rows = 0.0, 0, 0
            for pos in plist:
                q = synth.to_f64(cp.q[0][pos:pos + 1])
                t0 = time.perf_counter()
                OA.attend(q, [pos], k, v, kind, W)
                t += time.perf_counter() - t0
                keys += OA.valid_length(pos, kind, W)
                rows += 1
                if t >= budget_s / 2 and rows >= 4:
                    break
            res[kind] = (t, keys, rows)
    s_full = N * (N + 1) // 2
    s_swa = _pairs_swa(N, W)
    t_full = res[OA.FULL][0] / res[OA.FULL][1] * s_full    # one Full layer, all rows
    t_swa = res[OA.SWA][0] / res[OA.SWA][1] * s_swa
    nf, ns = pattern.count("F"), pattern.count("S")
    stack = nf * t_full + ns * t_swa
    out = _baseline(N / stack, "tok/s",
                    f"{res[OA.FULL][2]} Full rows (chunk edges and seeded positions) and "
                    f"{res[OA.SWA][2]} SWA rows, all heads; time per scored pair scaled by the "
                    f"stack's pair counts ({nf} Full + {ns} SWA layers)",
                    res[OA.FULL][0] + res[OA.SWA][0])
    out["all_full_value"] = round(N / (len(pattern) * t_full), 4)
    return out


# ---------------------------------------------------------------------------


def timed(cx, fn, steps, warmup):
    torch = cx.torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def roofline(bound, achieved, traffic=None):
    peak, unit = PEAKS[bound]
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def kernel_stats(cp, ev, kind):
    """Average duration, algorithmic GB/s and TFLOP/s of the attention
    launches of one layer kind, from the events recorded around them."""
    sel = [(st, e0.elapsed_time(e1) / 1e3) for k, st, e0, e1 in ev if k == kind]
    if not sel:
        return None
    t = sum(x for _, x in sel)
    return {"avg_us": t / len(sel) * 1e6,
            "gbs": sum(cp.attn_bytes(st, kind) for st, _ in sel) / t / 1e9,
            "tflops": sum(cp.attn_flops(st, kind) for st, _ in sel) / t / 1e12,
            "launches": len(sel)}


def run_decode(cx, dc, pattern, steps, warm):
    """Times `steps` decode steps; returns the step's algorithmic GB/s, the
    tokens kept per second and per-kind call durations from events."""
    torch, H = cx.torch, cx.H
    for _ in range(warm):
        dc.step()
    torch.cuda.synchronize()
    first = len(dc.step_bytes)
    t0 = time.perf_counter()
    for _ in range(steps):
        dc.step()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    step_bytes = sum(dc.step_bytes[first:]) / steps
    tok_per_step = sum(dc.accepted[first:]) / steps
    ev = []
    for _ in range(2):
        dc.step(ev)
    torch.cuda.synchronize()
    res = {"gbs": step_bytes / sec / 1e9, "ms_per_step": sec * 1e3, "bytes_per_step": step_bytes,
           "tok_per_s": tok_per_step / sec}
    for kind, name in ((H.FULL, "full"), (H.SWA, "swa")):
        sel = [(l, e0.elapsed_time(e1) / 1e3) for k, l, e0, e1 in ev if k == kind]
        if sel:
            t = sum(x for _, x in sel)
            res[name + "_call_us"] = t / len(sel) * 1e6
            res[name + "_gbs"] = sum(dc.layer_bytes(kind, l) for l, _ in sel) / t / 1e9
    return res


# What the bf16-page path computes in: bf16 inputs and K pages, V pages in
# fp16 (converted exactly from bf16 by the append), the QK product on the
# bf16 MFMA, the PV product on the fp16 MFMA with fp16 weights, softmax and
# accumulation in fp32, fp32 output (fp16 with --out f16).
PRECISION = {"inputs": "bf16", "k_pages": "bf16", "v_pages": "fp16",
             "qk_mfma": "bf16 x bf16 -> fp32", "pv_mfma": "fp16 x fp16 -> fp32",
             "softmax": "fp32", "output": "fp32"}


def base_line(args, value, unit, ms, config, rl):
    prec = dict(PRECISION, output=ODT[getattr(args, "out", "f32")])
    return {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16/fp16",
            "precision": prec, "data": "synthetic", "config": config, "roofline": rl}


# keys of the output contract that a config embedded in the default line
# does not repeat
_CONTRACT = ("metric", "n_gpus", "warmup", "higher_is_better", "scaling", "vs_baseline", "data",
             "precision")


def embed(line):
    """A workload's line as a sub-object of the default line: its config
    keys, then its measurements (value, unit, roofline, cpu_baseline ...)."""
    cfg = line.pop("config")
    return {**cfg, **{k: v for k, v in line.items() if k not in _CONTRACT}}


def copy_calibration(cx):
    """A plain 1 GiB device-to-device copy, three times: the reference that
    scales the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a counter run."""
    torch = cx.torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device=cx.dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def copy_ceiling(cx):
    """Practical HBM ceiling measured in the same run: a plain 1 GiB
    device-to-device copy (torch's copy kernel), timed with events on the
    launch stream over 10 copies after 2 untimed ones.  GB/s counts the bytes
    read plus the bytes written.  A copy is half writes; the decode kernels
    only read, so they can exceed it."""
    torch = cx.torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=cx.dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cx.stream)
    for _ in range(10):
        b.copy_(a)
    e1.record(cx.stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / 10
    del a, b
    torch.cuda.empty_cache()
    return round(2 * n / sec / 1e9, 1)


# ---------------------------------------------------------------------------
# Workloads


def wl_swa_chunked_prefill(cx, args):
    import synth
    H = cx.H
    wl = synth.C2
    lens = synth.uniform_lengths(wl.num_seqs, wl.len_lo, wl.len_hi, wl.seed)
    cp = ChunkedPrefill(cx, lens, wl.chunk, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                        wl.window, wl.seed, out=args.out, one_stream=args.single_stream,
                        combine_pool_ops=not args.separate_pool_ops)
    cx.torch.cuda.synchronize()
    log(f"prefill: {cp.tokens} tokens in {len(cp.steps)} chunk steps")
    sec = timed(cx, cp.run, args.steps, args.warmup)
    ev = []
    for _ in range(max(1, min(args.steps, 5))):
        cp.run(ev)
    cx.torch.cuda.synchronize()
    ks = kernel_stats(cp, ev, H.SWA)
    log(f"prefill: {cp.tokens / sec:.4g} tok/s, {sec * 1e3:.3f} ms/step, kernel {ks}")
    config = {
        "workload": "swa_chunked_prefill", "num_seqs": wl.num_seqs,
        "seq_len_range": [wl.len_lo, wl.len_hi], "seq_lens": lens, "chunk": wl.chunk,
        "window": wl.window, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
        "head_dim": wl.head_dim, "page_size": 16, "ring_slots": wl.window + wl.chunk,
        "output_dtype": ODT[args.out], "seed": wl.seed,
        "pool_calls": ("launch stream" if args.single_stream else
                       "second stream, beside appends and attention (q_pos given)") +
                      ("; evict and alloc separate" if args.separate_pool_ops else
                       "; each step's evict joined to the next step's alloc"),
    }
    rl = roofline("hbm", ks["gbs"], measured_traffic("prefill_swa", "kernels_prefill.hip")
                  if args.out == "f32" else None)
    line = base_line(args, round(cp.tokens / sec, 1), "tok/s", sec * 1e3, config, rl)
    line["kernel"] = {"name": "prefill_kernel<128,SWA>", "avg_us": round(ks["avg_us"], 2),
                      "launches_timed": ks["launches"], "tflops": round(ks["tflops"], 2),
                      "mfma_frac": round(ks["tflops"] / MFMA_BF16_PEAK_TFS, 4)}
    # the kernel writes more than it reads (fp32 O): a copy, half writes, is
    # the practical ceiling next to which its GB/s is read
    cc = copy_ceiling(cx)
    line["copy_ceiling"] = {"gbs": cc, "kernel_frac": round(ks["gbs"] / cc, 4)}
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(cx, cp, args.cpu_seconds)
        log(f"cpu baseline: {line['cpu_baseline']}")
    del cp
    cx.torch.cuda.empty_cache()
    if not args.no_decode:
        d = wl_mixed_decode(cx, args)
        line["decode"] = {**d["config"], "value": d["value"], "unit": d["unit"],
                          "frac": d["step_frac_of_hbm_peak"], "ms_per_step": d["ms_per_step"],
                          "roofline": d["roofline"], "full_call_us": d["full_call_us"],
                          "swa_call_us": d["swa_call_us"], "copy_ceiling": d["copy_ceiling"],
                          "cpu_baseline": d["cpu_baseline"]}
    if not args.headline_only:
        # the other configurations of the workload statement, each with its
        # own roofline and oracle baseline
        for key, fn in (("single_chunk", wl_swa_single_chunk), ("hybrid_stack", wl_hybrid_stack),
                        ("long_decode", wl_long_decode)):
            line[key] = embed(fn(cx, args))
            cx.torch.cuda.empty_cache()
    return line


def wl_mixed_decode(cx, args):
    import synth
    wl = synth.C3
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    steps, warm = args.decode_steps, 4
    dc = Decode(cx, ctxs, "FS", wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                wl.ring_slots, wl.seed, steps + warm + 8, out=args.out)
    r = run_decode(cx, dc, "FS", steps, warm)
    log(f"decode: {r}")
    config = {"workload": "mixed_decode", "num_seqs": wl.num_seqs,
              "ctx_range": [wl.ctx_lo, wl.ctx_hi], "layers": "1 Full + 1 SWA",
              "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "window": wl.window, "ring_slots": wl.ring_slots,
              "output_dtype": ODT[args.out], "seed": wl.seed}
    rl = roofline("hbm", r["full_gbs"], measured_traffic("decode_full", "kernels_decode.hip")
                  if args.out == "f32" else None)
    line = base_line(args, round(r["gbs"], 1), "GB/s", r["ms_per_step"], config, rl)
    line["step_frac_of_hbm_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
    line["full_call_us"] = round(r["full_call_us"], 1)
    line["swa_call_us"] = round(r["swa_call_us"], 1)
    cc = copy_ceiling(cx)
    line["copy_ceiling"] = {"gbs": cc, "full_call_frac": round(r["full_gbs"] / cc, 4)}
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        seqs = _sample_seqs(ctxs, 16, wl.seed)
        line["cpu_baseline"] = cpu_baseline_decode(cx, dc, seqs, [0, 1], args.cpu_seconds)
        log(f"decode cpu baseline: {line['cpu_baseline']}")
    return line


def _sample_seqs(ctxs, n, seed):
    """The shortest- and longest-context sequences, then seeded others."""
    lo, hi = int(np.argmin(ctxs)), int(np.argmax(ctxs))
    rest = [int(b) for b in np.random.default_rng(seed + 17).permutation(len(ctxs))
            if b not in (lo, hi)]
    return ([lo, hi] + rest)[:n]


def wl_swa_chunked_prefill_fp8(cx, args):
    """The SWA chunked prefill over FP8 pages: the appends quantize each
    chunk's K/V, the attention reads codes and scales."""
    import synth
    H = cx.H
    wl = synth.C2
    lens = synth.uniform_lengths(wl.num_seqs, wl.len_lo, wl.len_hi, wl.seed)
    cp = ChunkedPrefill(cx, lens, wl.chunk, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                        wl.window, wl.seed, out=args.out, one_stream=args.single_stream,
                        combine_pool_ops=not args.separate_pool_ops, fp8=True)
    cx.torch.cuda.synchronize()
    sec = timed(cx, cp.run, args.steps, args.warmup)
    ev = []
    for _ in range(max(1, min(args.steps, 5))):
        cp.run(ev)
    cx.torch.cuda.synchronize()
    ks = kernel_stats(cp, ev, H.SWA)
    log(f"prefill fp8: {cp.tokens / sec:.4g} tok/s, {sec * 1e3:.3f} ms/step, kernel {ks}")
    config = {"workload": "swa_chunked_prefill_fp8", "num_seqs": wl.num_seqs,
              "seq_len_range": [wl.len_lo, wl.len_hi], "seq_lens": lens, "chunk": wl.chunk,
              "window": wl.window, "num_q_heads": wl.num_q_heads,
              "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
              "kv_dtype": "fp8 e4m3, fp32 scale per token and head",
              "ring_slots": wl.window + wl.chunk, "output_dtype": ODT[args.out],
              "seed": wl.seed}
    rl = roofline("hbm", ks["gbs"], measured_traffic("prefill_swa_fp8", "kernels_prefill.hip")
                  if args.out == "f32" else None)
    line = base_line(args, round(cp.tokens / sec, 1), "tok/s", sec * 1e3, config, rl)
    line["dtype"] = "fp8 K/V, bf16/fp16 MFMA"
    line["precision"] = dict(line["precision"], k_pages="e4m3 + fp32 scale per token and head",
                             v_pages="e4m3 + fp32 scale per token and head",
                             qk_mfma="bf16 (exact e4m3 codes) x bf16 -> fp32, times the K scale",
                             pv_mfma="fp16 (code x V scale, rounded) x fp16 weight -> fp32")
    line["kernel"] = {"name": "prefill_kernel<128,SWA,FP8>", "avg_us": round(ks["avg_us"], 2),
                      "launches_timed": ks["launches"], "tflops": round(ks["tflops"], 2),
                      "mfma_frac": round(ks["tflops"] / MFMA_BF16_PEAK_TFS, 4)}
    line["cpu_baseline"] = None
    return line


def wl_mixed_decode_fp8(cx, args):
    """The mixed decode over FP8 pages (e4m3 codes, fp32 scale per token and
    head): half the K/V bytes per key."""
    import synth
    wl = synth.C3
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    steps, warm = args.decode_steps, 4
    dc = Decode(cx, ctxs, "FS", wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                wl.ring_slots, wl.seed, steps + warm + 8, fp8=True, out=args.out)
    r = run_decode(cx, dc, "FS", steps, warm)
    log(f"decode fp8: {r}")
    config = {"workload": "mixed_decode_fp8", "num_seqs": wl.num_seqs,
              "ctx_range": [wl.ctx_lo, wl.ctx_hi], "layers": "1 Full + 1 SWA",
              "kv_dtype": "fp8 e4m3, fp32 scale per token and head",
              "output_dtype": ODT[args.out],
              "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "window": wl.window, "ring_slots": wl.ring_slots,
              "seed": wl.seed}
    rl = roofline("hbm", r["full_gbs"], measured_traffic("decode_full_fp8", "kernels_decode.hip")
                  if args.out == "f32" else None)
    line = base_line(args, round(r["gbs"], 1), "GB/s", r["ms_per_step"], config, rl)
    line["dtype"] = "fp8 K/V, bf16/fp16 MFMA"
    # FP8 pages: codes turn exactly into bf16 (K) and fp16 (V) operands; the
    # K scale multiplies each score, the V scale rides in the fp16 weight
    line["precision"] = dict(line["precision"], k_pages="e4m3 + fp32 scale per token and head",
                             v_pages="e4m3 + fp32 scale per token and head",
                             qk_mfma="bf16 (exact e4m3 codes) x bf16 -> fp32, times the K scale",
                             pv_mfma="fp16 (exact e4m3 codes) x fp16 (weight x V scale x 2^8) "
                                     "-> fp32")
    line["step_frac_of_hbm_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
    line["tok_per_s"] = round(r["tok_per_s"], 1)
    line["full_call_us"] = round(r["full_call_us"], 1)
    line["swa_call_us"] = round(r["swa_call_us"], 1)
    return line


def wl_mtp_decode(cx, args, fp8=False):
    """Multi-token decode: one token plus three drafts per sequence per step
    over one Full and one SWA layer, accepted prefix kept; fp8: over FP8
    pages."""
    import synth
    wl = synth.MTP
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    steps, warm = args.decode_steps, 4
    rows = wl.drafts + 1
    dc = Decode(cx, ctxs, "FS", wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                wl.ring_slots, wl.seed, steps + warm + 8, rows=rows, fp8=fp8, out=args.out)
    r = run_decode(cx, dc, "FS", steps, warm)
    log(f"mtp decode{' fp8' if fp8 else ''}: {r}")
    config = {"workload": "mtp_decode_fp8" if fp8 else "mtp_decode", "num_seqs": wl.num_seqs,
              "ctx_range": [wl.ctx_lo, wl.ctx_hi], "rows_per_seq": rows,
              "accepted_rows": [1, rows], "layers": "1 Full + 1 SWA",
              "output_dtype": ODT[args.out],
              "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
              "head_dim": wl.head_dim, "window": wl.window, "ring_slots": wl.ring_slots,
              "seed": wl.seed}
    if fp8:
        config["kv_dtype"] = "fp8 e4m3, fp32 scale per token and head"
    rl = roofline("hbm", r["full_gbs"],
                  None if fp8 else measured_traffic("decode_full_mtp", "kernels_decode.hip"))
    line = base_line(args, round(r["gbs"], 1), "GB/s", r["ms_per_step"], config, rl)
    if fp8:
        line["dtype"] = "fp8 K/V, bf16/fp16 MFMA"
        line["precision"] = dict(line["precision"], k_pages="e4m3 + fp32 scale per token and head",
                                 v_pages="e4m3 + fp32 scale per token and head")
    line["step_frac_of_hbm_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
    line["accepted_tok_per_s"] = round(r["tok_per_s"], 1)
    line["full_call_us"] = round(r["full_call_us"], 1)
    line["swa_call_us"] = round(r["swa_call_us"], 1)
    return line


def wl_tier_transfer(cx, args, fp8=False):
    """Window-masked offload/restore of a 14-layer hybrid stack through pinned
    host memory, and restore + first decode step, serial and pulled layer by
    layer on a second stream.  fp8: the pages are FP8, and the buffers hold
    code bytes and per-(token, head) fp32 scales."""
    import synth
    from hybrid_sliding_window_hswa_amd import _capi
    torch, H, lib = cx.torch, cx.H, cx.lib
    wl = synth.TIER
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    hq, hkv, d, W = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window
    B, ids = len(ctxs), list(range(len(ctxs)))
    src = Decode(cx, ctxs, wl.pattern, hq, hkv, d, W, wl.ring_slots, wl.seed, 8, fp8=fp8)
    dst = Decode(cx, ctxs, wl.pattern, hq, hkv, d, W, wl.ring_slots, wl.seed + 1, 8, fill=False,
                 fp8=fp8)
    plan = {}
    for kind in (H.FULL, H.SWA):
        cnt = [int(x) for x in H.hswa_pool_window_counts(src.pool, kind, ids)]
        plan[kind] = (cnt, cx.i32(np.concatenate([[0], np.cumsum(cnt)])),
                      cx.i32([L - c for L, c in zip(ctxs, cnt)]))
    bufs, a_off, a_res = [], [], []
    for li, (kind, kc, vc) in enumerate(src.layers):
        cnt, cu, first = plan[kind]
        T = sum(cnt)
        if fp8:
            bk = torch.empty((T, hkv, d), dtype=torch.uint8, pin_memory=True)
            bv = torch.empty((T, hkv, d), dtype=torch.uint8, pin_memory=True)
            bks = torch.empty((T, hkv), dtype=torch.float32, pin_memory=True)
            bvs = torch.empty((T, hkv), dtype=torch.float32, pin_memory=True)
        else:
            bk = torch.empty((T, hkv, d), dtype=torch.bfloat16, pin_memory=True)
            bv = torch.empty((T, hkv, d), dtype=torch.float16, pin_memory=True)
            bks = bvs = None
        bufs.append((bk, bv, bks, bvs))
        for dc, lst in ((src, a_off), (dst, a_res)):
            a = _capi.XferArgs()
            a.kind, a.num_kv_heads, a.head_dim, a.num_seqs = kind, hkv, d, B
            a.seq_ids, a.cu_tok, a.first_pos = dc.sid.data_ptr(), cu.data_ptr(), first.data_ptr()
            a.total_tok, a.max_tok = T, max(cnt)
            a.pool = dc.view
            a.k_cache, a.v_cache = dc.layers[li][1].data_ptr(), dc.layers[li][2].data_ptr()
            a.buf_k, a.buf_v = bk.data_ptr(), bv.data_ptr()
            if fp8:
                a.kv_dtype = H.HSWA_KV_FP8
                a.k_scale = dc.scales[li][0].data_ptr()
                a.v_scale = dc.scales[li][1].data_ptr()
                a.buf_k_scale, a.buf_v_scale = bks.data_ptr(), bvs.data_ptr()
            lst.append(a)
    # bytes per moved token: codes and scales of K and V for FP8 pages
    kvb = 2 * hkv * (d + 4) if fp8 else KV_TOKEN_BYTES(hkv, d)
    masked = sum(sum(plan[kind][0]) for kind, _, _ in src.layers) * kvb
    unmasked = len(src.layers) * sum(ctxs) * kvb
    swa_bytes = sum(sum(plan[kind][0]) for kind, _, _ in src.layers if kind == H.SWA) * kvb

    def offload_all():
        for a in a_off:
            _check(cx, lib.hswa_kv_offload(C.byref(a), cx.sptr))

    def restore_all(stream=None, events=None):
        for a in a_res:
            _check(cx, lib.hswa_kv_restore(C.byref(a), stream or cx.sptr))
            if events is not None:
                ev = torch.cuda.Event()
                ev.record(events[0])
                events[1].append(ev)

    steps, warm = max(args.steps // 4, 3), 1
    t_off = timed(cx, offload_all, steps, warm)
    t_res = timed(cx, restore_all, steps, warm)
    # one layer's restore, SWA and Full, for the per-kind link rate
    per_kind = {}
    for kind in (H.FULL, H.SWA):
        li = [i for i, (k, _, _) in enumerate(src.layers) if k == kind][0]
        t = timed(cx, lambda: _check(cx, lib.hswa_kv_restore(C.byref(a_res[li]), cx.sptr)),
                  steps, warm)
        per_kind[kind] = (sum(plan[kind][0]) * kvb, t)

    # restore then the first decode step: serial on one stream, or pulled
    # layer by layer on a second stream while the first computes
    ids_a, idp = dst.ids
    ctx_a = _arr(ctxs)
    copy = torch.cuda.Stream()  # default priority
    copy_ptr = C.c_void_p(copy.cuda_stream)

    def reset():
        _check(cx, lib.hswa_pool_release(dst.pool.handle, B, idp, cx.sptr))
        _check(cx, lib.hswa_pool_import(dst.pool.handle, B, idp, ctx_a[1], None, None, cx.sptr))
        dst.lens = list(ctxs)

    def serial():
        reset()
        restore_all()
        dst.step()

    def pulled():
        reset()
        ready = torch.cuda.Event()
        ready.record(cx.stream)
        copy.wait_event(ready)
        evs = []
        restore_all(copy_ptr, (copy, evs))
        h = dst.pool.handle
        _, onep = dst.nrows
        _check(cx, lib.hswa_pool_alloc(h, B, idp, onep, None, None, cx.sptr))
        dst.lens = [x + 1 for x in dst.lens]
        for a, ev in zip(dst.args, evs):
            cx.stream.wait_event(ev)
            _check(cx, lib.hswa_decode(C.byref(a), C.c_void_p(dst.ws.data_ptr()), dst.nbytes_ws,
                                       cx.sptr))
        _check(cx, lib.hswa_pool_evict(h, B, idp, None, 0, None, cx.sptr))

    t_ser = timed(cx, serial, steps, warm)
    t_pull = timed(cx, pulled, steps, warm)
    torch.cuda.synchronize()
    res_gbs = masked / t_res / 1e9
    config = {"workload": "tier_transfer_fp8" if fp8 else "tier_transfer", "num_seqs": B,
              "ctx_range": [wl.ctx_lo, wl.ctx_hi],
              "layers": len(wl.pattern), "pattern": "6 SWA then 1 Full, x2",
              "num_kv_heads": hkv, "head_dim": d, "window": W, "host_buffers": "pinned",
              "kv_dtype": "fp8 e4m3, fp32 scale per token and head" if fp8 else "bf16/fp16",
              "seed": wl.seed}
    line = base_line(args, round(res_gbs, 2), "GB/s", t_res * 1e3, config,
                     roofline("pcie", res_gbs, None))
    line["steps"] = steps
    if fp8:
        line["dtype"] = "fp8 K/V, bf16/fp16 MFMA"
        line["precision"] = dict(line["precision"],
                                 k_pages="e4m3 + fp32 scale per token and head",
                                 v_pages="e4m3 + fp32 scale per token and head",
                                 host_buffers="e4m3 codes + fp32 scales, moved verbatim")
    line["offload_gbs"] = round(masked / t_off / 1e9, 2)
    line["offload_ms"] = round(t_off * 1e3, 3)
    line["restore_full_layer_gbs"] = round(per_kind[H.FULL][0] / per_kind[H.FULL][1] / 1e9, 2)
    line["restore_swa_layer_gbs"] = round(per_kind[H.SWA][0] / per_kind[H.SWA][1] / 1e9, 2)
    line["restore_swa_layer_us"] = round(per_kind[H.SWA][1] * 1e6, 1)
    line["bytes_masked"] = masked
    line["bytes_unmasked"] = unmasked
    line["mask_fraction"] = round(masked / unmasked, 5)
    line["swa_share_of_masked_bytes"] = round(swa_bytes / masked, 5)
    line["restore_then_step_ms"] = round(t_ser * 1e3, 3)
    line["pulled_layerwise_ms"] = round(t_pull * 1e3, 3)
    return line


def wl_hybrid_stack(cx, args):
    import synth
    H = cx.H
    wl = synth.C4
    res = {}
    steps = max(1, min(args.steps, 3))
    for variant, pattern in (("hybrid", wl.pattern), ("all_full", "F" * len(wl.pattern))):
        cp = ChunkedPrefill(cx, [wl.seq_len], wl.chunk, wl.num_q_heads, wl.num_kv_heads,
                            wl.head_dim, wl.window, wl.seed, pattern=pattern)
        cx.torch.cuda.synchronize()
        n = steps if variant == "hybrid" else 1
        sec = timed(cx, cp.run, n, min(args.warmup, 1))
        ev = []
        cp.run(ev)
        cx.torch.cuda.synchronize()
        res[variant] = {"sec": sec, "full": kernel_stats(cp, ev, H.FULL),
                        "swa": kernel_stats(cp, ev, H.SWA),
                        "flops": sum(cp.attn_flops(st, kind) for st in cp.steps
                                     for kind, _, _ in cp.layers)}
        log(f"stack {variant}: {wl.seq_len / sec:.4g} tok/s, {sec:.3f} s/step, "
            f"full {res[variant]['full']}, swa {res[variant]['swa']}")
        if variant == "hybrid" and not args.no_cpu_baseline:
            res["cpu"] = cpu_baseline_stack(cx, cp, wl.pattern, args.cpu_seconds)
            log(f"stack cpu baseline: {res['cpu']}")
        del cp, ev
        cx.torch.cuda.empty_cache()
    hy, af = res["hybrid"], res["all_full"]
    fk = hy["full"]
    config = {"workload": "hybrid_stack", "layers": len(wl.pattern),
              "pattern": "6 SWA then 1 Full, x10", "seq_len": wl.seq_len, "chunk": wl.chunk,
              "window": wl.window, "num_q_heads": wl.num_q_heads,
              "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "seed": wl.seed}
    rl = roofline("mfma", fk["tflops"], measured_traffic("prefill_full", "kernels_prefill.hip"))
    line = base_line(args, round(wl.seq_len / hy["sec"], 1), "tok/s", hy["sec"] * 1e3, config,
                     rl)
    line["steps"] = steps
    line["kernel"] = {"name": "prefill_kernel<128,FULL>", "avg_us": round(fk["avg_us"], 2),
                      "launches_timed": fk["launches"], "gbs": round(fk["gbs"], 1)}
    line["swa_kernel"] = {"avg_us": round(hy["swa"]["avg_us"], 2),
                          "gbs": round(hy["swa"]["gbs"], 1)}
    line["all_full"] = {"value": round(wl.seq_len / af["sec"], 1), "unit": "tok/s",
                        "ms_per_step": round(af["sec"] * 1e3, 3),
                        "full_kernel_tflops": round(af["full"]["tflops"], 1)}
    line["time_ratio_hybrid_over_all_full"] = round(hy["sec"] / af["sec"], 5)
    line["flop_ratio_hybrid_over_all_full"] = round(hy["flops"] / af["flops"], 6)
    # the same ratio from the MFMA op counters (rocprofv3), which include the
    # masked parts of the tiles the kernels compute
    mf = measured_mfma_ops("prefill_full", "kernels_prefill.hip")
    ms = measured_mfma_ops("prefill_swa_stack", "kernels_prefill.hip")
    nf = wl.pattern.count("F")
    line["mfma_op_ratio_hybrid_over_all_full"] = (
        round((nf * mf + (len(wl.pattern) - nf) * ms) / (len(wl.pattern) * mf), 6)
        if mf and ms else None)
    line["cpu_baseline"] = res.get("cpu")
    return line


def wl_long_decode(cx, args):
    import synth
    wl = synth.C5
    ctxs = synth.uniform_lengths(wl.num_seqs, wl.ctx_lo, wl.ctx_hi, wl.seed)
    steps, warm = max(2, args.decode_steps // 2), 2
    t0 = time.perf_counter()
    dc = Decode(cx, ctxs, wl.pattern, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                wl.ring_slots, wl.seed, steps + warm + 4)
    log(f"long decode: setup {time.perf_counter() - t0:.1f} s")
    r = run_decode(cx, dc, wl.pattern, steps, warm)
    log(f"long decode: {r}")
    config = {"workload": "long_decode", "num_seqs": wl.num_seqs,
              "ctx_range": [wl.ctx_lo, wl.ctx_hi], "layers": len(wl.pattern),
              "pattern": "6 SWA then 1 Full, x2", "ring_slots": wl.ring_slots,
              "window": wl.window, "num_q_heads": wl.num_q_heads,
              "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "seed": wl.seed}
    rl = roofline("hbm", r["full_gbs"],
                  measured_traffic("decode_full_long", "kernels_decode.hip"))
    line = base_line(args, round(r["gbs"], 1), "GB/s", r["ms_per_step"], config, rl)
    line["steps"] = steps
    line["step_frac_of_hbm_peak"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
    line["full_call_us"] = round(r["full_call_us"], 1)
    line["swa_call_us"] = round(r["swa_call_us"], 1)
    cc = copy_ceiling(cx)
    line["copy_ceiling"] = {"gbs": cc, "full_call_frac": round(r["full_gbs"] / cc, 4)}
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        full = [i for i, k in enumerate(wl.pattern) if k == "F"][:2]
        swa = [i for i, k in enumerate(wl.pattern) if k == "S"][:1] + \
              [i for i, k in enumerate(wl.pattern) if k == "S" and i > full[0]][:1]
        seqs = _sample_seqs(ctxs, 4, wl.seed)
        line["cpu_baseline"] = cpu_baseline_decode(cx, dc, seqs, full + swa, args.cpu_seconds)
        log(f"long decode cpu baseline: {line['cpu_baseline']}")
    return line


def wl_swa_single_chunk(cx, args):
    import synth
    H = cx.H
    wl = synth.C1
    L = wl.prefill_len
    cp = ChunkedPrefill(cx, [L], L, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                        wl.seed)
    sec = timed(cx, cp.run, args.steps, args.warmup)
    ev = []
    cp.run(ev)
    cx.torch.cuda.synchronize()
    ks = kernel_stats(cp, ev, H.SWA)
    config = {"workload": "swa_single_chunk", "seq_len": L, "decode_steps": wl.decode_steps,
              "window": wl.window, "num_q_heads": wl.num_q_heads,
              "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "seed": wl.seed}
    line = base_line(args, round(L / sec, 1), "tok/s", sec * 1e3, config,
                     roofline("hbm", ks["gbs"],
                              measured_traffic("prefill_swa_d64", "kernels_prefill.hip")))
    line["kernel"] = {"name": "prefill_kernel<64,SWA>", "avg_us": round(ks["avg_us"], 2)}
    dc = Decode(cx, [L], "S", wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window,
                wl.window + 16, wl.seed, wl.decode_steps + 8)
    r = run_decode(cx, dc, "S", wl.decode_steps, 2)
    line["decode_step_us"] = round(r["ms_per_step"] * 1e3, 2)
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        import synth
        W, n = wl.window, wl.decode_steps
        tail = [synth.bf16_normal((W - 1, wl.num_kv_heads, wl.head_dim), wl.seed, 0, 0, role,
                                  device=cx.dev) for role in (synth.ROLE_K, synth.ROLE_V)]
        # keys of decode step t (position L + t): the restored tail, then the
        # step's new key once per earlier step (every step appends the same row)
        ks, vs = (synth.to_f64(cx.torch.cat([t] + [new[0:1]] * n)) for t, new in
                  zip(tail, (dc.kn[0], dc.vn[0])))
        dk = np.stack([ks[t:t + W] for t in range(n)])
        dv = np.stack([vs[t:t + W] for t in range(n)])
        dq = np.repeat(synth.to_f64(dc.q[0][0:1]), n, axis=0)
        line["cpu_baseline"] = cpu_baseline_single_chunk(cx, cp, (dq, dk, dv),
                                                         min(args.cpu_seconds, 2.0))
        log(f"single chunk cpu baseline: {line['cpu_baseline']}")
    return line


def wl_tp8_share(cx, args):
    """One GPU's share of an 8-way head split of the default run: the same
    SWA chunked prefill (lengths, chunk, W) and mixed decode (contexts) with
    Hq = 8 and Hkv = 1, i.e. what each of eight GPUs holds and computes when
    KV heads are divided among them (no exchange inside attention)."""
    import synth
    H = cx.H
    wl, wd = synth.C2, synth.C3
    hq, hkv = wl.num_q_heads // 8, wl.num_kv_heads // 8
    lens = synth.uniform_lengths(wl.num_seqs, wl.len_lo, wl.len_hi, wl.seed)
    cp = ChunkedPrefill(cx, lens, wl.chunk, hq, hkv, wl.head_dim, wl.window, wl.seed,
                        out=args.out)
    cx.torch.cuda.synchronize()
    sec = timed(cx, cp.run, args.steps, args.warmup)
    ev = []
    for _ in range(max(1, min(args.steps, 5))):
        cp.run(ev)
    cx.torch.cuda.synchronize()
    ks = kernel_stats(cp, ev, H.SWA)
    log(f"tp8 share prefill: {cp.tokens / sec:.4g} tok/s, {sec * 1e3:.3f} ms/step, kernel {ks}")
    config = {
        "workload": "tp8_share", "share": "1 of 8 GPUs, KV heads split 8 ways",
        "num_seqs": wl.num_seqs, "seq_len_range": [wl.len_lo, wl.len_hi], "seq_lens": lens,
        "chunk": wl.chunk, "window": wl.window, "num_q_heads": hq, "num_kv_heads": hkv,
        "head_dim": wl.head_dim, "page_size": 16, "ring_slots": wl.window + wl.chunk,
        "output_dtype": ODT[args.out], "seed": wl.seed,
    }
    line = base_line(args, round(cp.tokens / sec, 1), "tok/s", sec * 1e3, config,
                     roofline("hbm", ks["gbs"], None))
    line["kernel"] = {"name": "prefill_kernel<128,SWA>", "avg_us": round(ks["avg_us"], 2),
                      "launches_timed": ks["launches"], "tflops": round(ks["tflops"], 2)}
    if not args.no_decode:
        ctxs = synth.uniform_lengths(wd.num_seqs, wd.ctx_lo, wd.ctx_hi, wd.seed)
        steps, warm = args.decode_steps, 4
        dc = Decode(cx, ctxs, "FS", hq, hkv, wd.head_dim, wd.window, wd.ring_slots, wd.seed,
                    steps + warm + 8, out=args.out)
        r = run_decode(cx, dc, "FS", steps, warm)
        log(f"tp8 share decode: {r}")
        line["decode"] = {"num_seqs": wd.num_seqs, "ctx_range": [wd.ctx_lo, wd.ctx_hi],
                          "layers": "1 Full + 1 SWA", "num_q_heads": hq, "num_kv_heads": hkv,
                          "value": round(r["gbs"], 1), "unit": "GB/s",
                          "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                          "ms_per_step": round(r["ms_per_step"], 4),
                          "roofline": roofline("hbm", r["full_gbs"], None),
                          "full_call_us": round(r["full_call_us"], 1),
                          "swa_call_us": round(r["swa_call_us"], 1)}
    line["cpu_baseline"] = None
    return line


WORKLOADS = {
    "swa_chunked_prefill": wl_swa_chunked_prefill,
    "tp8_share": wl_tp8_share,
    "mixed_decode": wl_mixed_decode,
    "mixed_decode_fp8": wl_mixed_decode_fp8,
    "swa_chunked_prefill_fp8": wl_swa_chunked_prefill_fp8,
    "mtp_decode": wl_mtp_decode,
    "mtp_decode_fp8": lambda cx, args: wl_mtp_decode(cx, args, fp8=True),
    "tier_transfer": wl_tier_transfer,
    "tier_transfer_fp8": lambda cx, args: wl_tier_transfer(cx, args, fp8=True),
    "hybrid_stack": wl_hybrid_stack,
    "long_decode": wl_long_decode,
    "swa_single_chunk": wl_swa_single_chunk,
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # after the setup's idle time the GPU takes about 15 chunked-prefill
    # steps (~18 ms) to reach its steady clock; 30 warm-up steps cover it
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="swa_chunked_prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--decode-steps", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--single-stream", action="store_true",
                    help="chunked prefill: issue the pool calls on the launch stream, after "
                         "the attention they follow, instead of on a second stream")
    ap.add_argument("--separate-pool-ops", action="store_true",
                    help="chunked prefill: evict each step and alloc the next as two pool "
                         "calls instead of one hswa_pool_evict_alloc")
    ap.add_argument("--headline-only", action="store_true",
                    help="default workload: measure the chunked prefill and the mixed decode "
                         "only, not the single-chunk, 70-layer stack and long-context decode "
                         "configurations")
    ap.add_argument("--out", choices=sorted(ODT), default="f32",
                    help="attention output type of the prefill and decode workloads "
                         "(f32 default; f16 halves the bytes written)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy first, as the reference for the "
                         "HBM byte counters of a rocprofv3 --pmc run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    cx = Ctx()
    if args.copy_calibration:
        copy_calibration(cx)
    line = WORKLOADS[args.workload](cx, args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
