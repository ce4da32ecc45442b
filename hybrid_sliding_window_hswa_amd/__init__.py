"""Hybrid Sliding-Window Attention hot path for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libhswa.so (include/hswa.h).  The
functions keep the C names; they only marshal arguments (torch tensors ->
device pointers, Python sequences -> host int32 arrays) and turn a non-zero
status into an exception.  Every step of the path runs in the library's HIP
kernels and host C++; torch provides device memory and streams only.

Sources: "MiMo-V2.5 Series Inference Full-Link Optimization: Pushing Hybrid
SWA Efficiency to the Extreme" (sec. 1.1 layer mix and window, sec. 1.2
decode cost, sec. 2.1 KVCache Dual Pool and SWA-aware prefix cache tree)
and "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct
MI355X" (sec. 3, 16-token pages behind a page table).
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np

from . import _capi
from ._capi import (HSWA_DECODE_SCRATCH_BYTES, HSWA_E_HIP, HSWA_E_INVAL, HSWA_E_NOSPC,
                    HSWA_E_UNSUPPORTED, HSWA_KV_BF16, HSWA_KV_FP8, HSWA_LAYER_FULL,
                    HSWA_LAYER_SWA, HSWA_OK)

PAGE_SIZE = 16
DECODE_SCRATCH_BYTES = HSWA_DECODE_SCRATCH_BYTES
FULL = HSWA_LAYER_FULL
SWA = HSWA_LAYER_SWA

__all__ = [
    "HswaError", "NoSpace", "FULL", "SWA", "PAGE_SIZE",
    "hswa_pool_create", "hswa_pool_destroy", "hswa_pool_get_view", "hswa_pool_alloc",
    "hswa_pool_evict", "hswa_pool_evict_alloc", "hswa_pool_import", "hswa_pool_release", "hswa_pool_truncate",
    "hswa_pool_match_len", "hswa_pool_read_tables", "hswa_pool_fork", "hswa_kv_copy",
    "hswa_prefill_chunk", "hswa_decode", "hswa_decode_workspace_bytes", "hswa_append_kv",
    "hswa_decode_noalloc", "DECODE_SCRATCH_BYTES",
    "hswa_pool_window_counts", "hswa_kv_offload", "hswa_kv_restore",
    "hswa_last_error", "hswa_version", "kv_cache_shapes", "kv_cache_alloc",
    "kv_cache_alloc_fp8", "library",
]


class HswaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_capi.load().hswa_status_string(status).decode()}: {message}")
        self.status = status


class NoSpace(HswaError):
    """The joint Full/SWA capacity check failed; the pool is unchanged."""


def library():
    return _capi.load()


def hswa_last_error() -> str:
    return library().hswa_last_error().decode()


def hswa_version() -> int:
    return library().hswa_version()


def _check(rc: int):
    if rc != HSWA_OK:
        msg = hswa_last_error()
        if rc == HSWA_E_NOSPC:
            raise NoSpace(rc, msg)
        raise HswaError(rc, msg)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_capi.I32P)


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Pool


class Pool:
    """A pool handle plus the device tables it mirrors (kept alive here)."""

    def __init__(self, handle, tables, desc):
        self.handle = handle
        self.tables = tables  # dict of torch int32 tensors or None
        self.desc = desc

    def __del__(self):
        try:
            hswa_pool_destroy(self)
        except Exception:
            pass


def hswa_pool_create(window: int, ring_slots: int, max_seqs: int, max_pages_per_seq: int,
                     num_full_pages: int, full_free_order, ring_pages, device=None) -> Pool:
    """Creates a pool.  With ``device`` (e.g. "cuda:0") the four device
    tables are allocated there as int32 torch tensors and mirrored by the
    library; without it the pool keeps host bookkeeping only."""
    lib = library()
    free = _i32(full_free_order)
    ring = _i32(ring_pages)
    tables = None
    desc = _capi.PoolDesc()
    desc.page_size = PAGE_SIZE
    desc.window = window
    desc.ring_slots = ring_slots
    desc.max_seqs = max_seqs
    desc.max_pages_per_seq = max_pages_per_seq
    desc.num_full_pages = num_full_pages
    if free.size != num_full_pages or ring.size != max_seqs * (ring_slots // PAGE_SIZE):
        raise ValueError("full_free_order / ring_pages have the wrong length")
    desc.full_free_order = _p(free)
    desc.ring_pages = _p(ring)
    if device is not None:
        import torch
        tables = {
            "seq_len": torch.empty(max_seqs, dtype=torch.int32, device=device),
            "fpt": torch.empty(max_seqs * max_pages_per_seq, dtype=torch.int32, device=device),
            "rpt": torch.empty(ring.size, dtype=torch.int32, device=device),
            "map": torch.empty(num_full_pages * PAGE_SIZE, dtype=torch.int32, device=device),
        }
        desc.dev_seq_len = tables["seq_len"].data_ptr()
        desc.dev_fpt = tables["fpt"].data_ptr()
        desc.dev_rpt = tables["rpt"].data_ptr()
        desc.dev_map = tables["map"].data_ptr()
    h = C.c_void_p()
    _check(lib.hswa_pool_create(C.byref(desc), C.byref(h)))
    info = dict(window=window, ring_slots=ring_slots, max_seqs=max_seqs,
                max_pages_per_seq=max_pages_per_seq, num_full_pages=num_full_pages)
    return Pool(h, tables, info)


def hswa_pool_destroy(pool: Pool) -> None:
    if pool.handle is not None and pool.handle.value:
        library().hswa_pool_destroy(pool.handle)
    pool.handle = None


def hswa_pool_get_view(pool: Pool) -> _capi.PoolView:
    v = _capi.PoolView()
    _check(library().hswa_pool_get_view(pool.handle, C.byref(v)))
    return v


def hswa_pool_alloc(pool: Pool, seq_ids: Sequence[int], n_new: Sequence[int],
                    want_slots: bool = True, stream=None):
    """Returns (full_slots, swa_slots) as int32 arrays (None if not wanted)."""
    ids, n = _i32(seq_ids), _i32(n_new)
    tot = int(np.clip(n, 0, None).sum()) if n.size else 0
    full = np.empty(tot, np.int32) if want_slots else None
    swa = np.empty(tot, np.int32) if want_slots else None
    _check(library().hswa_pool_alloc(pool.handle, ids.size, _p(ids), _p(n), _p(full), _p(swa),
                                     _stream(stream)))
    return full, swa


def hswa_pool_import(pool: Pool, seq_ids: Sequence[int], n_new: Sequence[int],
                     want_slots: bool = True, stream=None):
    ids, n = _i32(seq_ids), _i32(n_new)
    tot = int(np.clip(n, 0, None).sum()) if n.size else 0
    full = np.empty(tot, np.int32) if want_slots else None
    swa = np.empty(tot, np.int32) if want_slots else None
    _check(library().hswa_pool_import(pool.handle, ids.size, _p(ids), _p(n), _p(full),
                                      _p(swa), _stream(stream)))
    return full, swa


def hswa_pool_evict(pool: Pool, seq_ids: Sequence[int], want_slots: bool = True,
                    capacity: Optional[int] = None, stream=None):
    """Returns (evicted_full_slots, counts) (None, counts if not wanted)."""
    ids = _i32(seq_ids)
    cap = capacity if capacity is not None else ids.size * pool.desc["ring_slots"]
    ev = np.empty(max(cap, 1), np.int32) if want_slots else None
    cnt = np.empty(max(ids.size, 1), np.int32)
    _check(library().hswa_pool_evict(pool.handle, ids.size, _p(ids), _p(ev), cap, _p(cnt),
                                     _stream(stream)))
    cnt = cnt[:ids.size]
    if ev is not None:
        ev = ev[:int(cnt.sum())]
    return ev, cnt


def hswa_pool_evict_alloc(pool: Pool, ev_ids: Sequence[int], al_ids: Sequence[int],
                          n_new: Sequence[int], want_slots: bool = True,
                          capacity: Optional[int] = None, stream=None):
    """hswa_pool_evict(ev_ids) then hswa_pool_alloc(al_ids, n_new) as one
    operation (one device-table update).  Returns (evicted_full_slots,
    counts, full_slots, swa_slots); the slot arrays are None if not wanted."""
    ev_i, al_i, n = _i32(ev_ids), _i32(al_ids), _i32(n_new)
    if n.size != al_i.size:
        raise ValueError("one n_new per allocated sequence")
    cap = capacity if capacity is not None else ev_i.size * pool.desc["ring_slots"]
    ev = np.empty(max(cap, 1), np.int32) if want_slots else None
    cnt = np.empty(max(ev_i.size, 1), np.int32)
    tot = int(np.clip(n, 0, None).sum()) if n.size else 0
    full = np.empty(tot, np.int32) if want_slots else None
    swa = np.empty(tot, np.int32) if want_slots else None
    _check(library().hswa_pool_evict_alloc(pool.handle, ev_i.size, _p(ev_i), _p(ev), cap,
                                           _p(cnt), al_i.size, _p(al_i), _p(n), _p(full),
                                           _p(swa), _stream(stream)))
    cnt = cnt[:ev_i.size]
    if ev is not None:
        ev = ev[:int(cnt.sum())]
    return ev, cnt, full, swa


def hswa_pool_release(pool: Pool, seq_ids: Sequence[int], stream=None) -> None:
    ids = _i32(seq_ids)
    _check(library().hswa_pool_release(pool.handle, ids.size, _p(ids), _stream(stream)))


def hswa_pool_truncate(pool: Pool, seq_ids: Sequence[int], new_len: Sequence[int],
                       stream=None) -> None:
    """Cuts each listed sequence back to new_len positions (rejected drafts of
    a multi-token step); call before the step's evict."""
    ids, n = _i32(seq_ids), _i32(new_len)
    if n.size != ids.size:
        raise ValueError("one new length per sequence")
    _check(library().hswa_pool_truncate(pool.handle, ids.size, _p(ids), _p(n), _stream(stream)))


def hswa_pool_match_len(pool: Pool, seq_ids: Sequence[int], want: Sequence[int],
                        tail: Optional[int] = None) -> np.ndarray:
    """Window-safe match lengths; ``tail`` defaults to W - 1 (what the next
    query needs)."""
    ids, w = _i32(seq_ids), _i32(want)
    if w.size != ids.size:
        raise ValueError("one length per sequence")
    t = pool.desc["window"] - 1 if tail is None else tail
    out = np.empty(max(ids.size, 1), np.int32)
    _check(library().hswa_pool_match_len(pool.handle, ids.size, _p(ids), _p(w), t, _p(out)))
    return out[:ids.size]


def hswa_pool_fork(pool: Pool, src_ids: Sequence[int], dst_ids: Sequence[int],
                   lens: Sequence[int], stream=None):
    """Empty sequences dst_ids[i] take the first lens[i] (window-safe)
    positions of src_ids[i].  Returns (full_from, swa_from): per fork, the
    first position whose K/V hswa_kv_copy must copy for FULL and for SWA
    layers."""
    src, dst, n = _i32(src_ids), _i32(dst_ids), _i32(lens)
    if not (src.size == dst.size == n.size):
        raise ValueError("one source, destination and length per fork")
    ff = np.empty(max(dst.size, 1), np.int32)
    sf = np.empty(max(dst.size, 1), np.int32)
    _check(library().hswa_pool_fork(pool.handle, dst.size, _p(src), _p(dst), _p(n), _p(ff),
                                     _p(sf), _stream(stream)))
    return ff[:dst.size], sf[:dst.size]


def hswa_pool_read_tables(pool: Pool) -> dict:
    d = pool.desc
    seq_len = np.empty(d["max_seqs"], np.int32)
    fpt = np.empty(d["max_seqs"] * d["max_pages_per_seq"], np.int32)
    mp = np.empty(d["num_full_pages"] * PAGE_SIZE, np.int32)
    free = np.empty(d["num_full_pages"], np.int32)
    nfree = np.zeros(1, np.int32)
    _check(library().hswa_pool_read_tables(pool.handle, _p(seq_len), _p(fpt), _p(mp), _p(free),
                                           _p(nfree)))
    return {"seq_len": seq_len, "fpt": fpt.reshape(d["max_seqs"], d["max_pages_per_seq"]),
            "map": mp, "free": free[:int(nfree[0])]}


# ---------------------------------------------------------------------------
# Attention


def kv_cache_shapes(num_pages: int, num_kv_heads: int, head_dim: int):
    """Shapes of one layer's K pages (bf16, token-major) and V pages (fp16,
    dim-major)."""
    return ((num_pages, num_kv_heads, PAGE_SIZE, head_dim),
            (num_pages, num_kv_heads, head_dim, PAGE_SIZE))


def kv_cache_alloc(num_pages: int, num_kv_heads: int, head_dim: int, device, fill=None):
    """Allocates one layer's K (bf16) and V (fp16) page buffers on `device`,
    uninitialised or filled with `fill`."""
    import torch
    ks, vs = kv_cache_shapes(num_pages, num_kv_heads, head_dim)
    if fill is None:
        return (torch.empty(ks, dtype=torch.bfloat16, device=device),
                torch.empty(vs, dtype=torch.float16, device=device))
    return (torch.full(ks, fill, dtype=torch.bfloat16, device=device),
            torch.full(vs, fill, dtype=torch.float16, device=device))


def kv_cache_alloc_fp8(num_pages: int, num_kv_heads: int, head_dim: int, device, fill=None):
    """One layer's FP8 pages: K codes [pages, Hkv, 16, d] and V codes
    [pages, Hkv, d, 16] (uint8, OCP e4m3) with fp32 scales [pages, Hkv, 16]
    for K and for V.  `fill` (an int code) fills the code buffers and NaN
    the scales; None leaves them uninitialised."""
    import torch
    ks, vs = kv_cache_shapes(num_pages, num_kv_heads, head_dim)
    sc = (num_pages, num_kv_heads, PAGE_SIZE)
    if fill is None:
        return (torch.empty(ks, dtype=torch.uint8, device=device),
                torch.empty(vs, dtype=torch.uint8, device=device),
                torch.empty(sc, dtype=torch.float32, device=device),
                torch.empty(sc, dtype=torch.float32, device=device))
    return (torch.full(ks, fill, dtype=torch.uint8, device=device),
            torch.full(vs, fill, dtype=torch.uint8, device=device),
            torch.full(sc, float("nan"), dtype=torch.float32, device=device),
            torch.full(sc, float("nan"), dtype=torch.float32, device=device))


def _expect(name, t, dtypes, shape=None, min_rows=None, device=True):
    """Checks a tensor argument before its address reaches a kernel: the
    dtype, the shape (None entries are free), a lower bound on the leading
    dimension, and that it lives in device memory (a host address handed to
    a kernel would fault)."""
    if t is None:
        return
    if str(t.dtype) not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(dtypes)}, not {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != w
                                         for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if min_rows is not None and t.shape[0] < min_rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, the call needs {min_rows}")


_BF16, _F16, _F32, _I32, _U8 = ("torch.bfloat16",), ("torch.float16",), ("torch.float32",), \
    ("torch.int32",), ("torch.uint8",)


def _args(kind, window, q, k_new, v_new, seq_ids, cu_q, total_q, max_q_len, max_seq_len,
          view, k_cache, v_cache, out, vlen, scale, k_scale=None,
          v_scale=None, q_pos=None) -> _capi.AttnArgs:
    fp8 = k_scale is not None
    _expect("k_cache", k_cache, _U8 if fp8 else _BF16, (None, None, PAGE_SIZE, None))
    hkv, d = k_cache.shape[1], k_cache.shape[3]
    _expect("v_cache", v_cache, _U8 if fp8 else _F16, (k_cache.shape[0], hkv, d, PAGE_SIZE))
    _expect("k_scale", k_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    _expect("v_scale", v_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    if fp8 and v_scale is None:
        raise ValueError("FP8 pages need both k_scale and v_scale")
    _expect("q", q, _BF16, (None, None, d), total_q)
    _expect("k_new", k_new, _BF16, (None, hkv, d), total_q)
    _expect("v_new", v_new, _BF16, (None, hkv, d), total_q)
    _expect("seq_ids", seq_ids, _I32, (None,))
    _expect("cu_q", cu_q, _I32, (seq_ids.shape[0] + 1,))
    _expect("q_pos", q_pos, _I32, (seq_ids.shape[0],))
    hq_ = q.shape[1] if q is not None else None
    _expect("out", out, _F32 + _F16, (None, hq_, d), total_q)
    _expect("vlen", vlen, _I32, (None,), total_q)
    a = _capi.AttnArgs()
    a.kind = kind
    a.window = window
    hq, d = (q.shape[-2], q.shape[-1]) if q is not None else (k_new.shape[-2], k_new.shape[-1])
    a.num_q_heads = hq
    a.num_kv_heads = k_cache.shape[1]
    a.head_dim = d
    a.scale = scale
    a.num_seqs = seq_ids.shape[0]
    a.seq_ids = _dptr(seq_ids)
    a.cu_q = _dptr(cu_q)
    a.total_q = total_q
    a.max_q_len = max_q_len
    a.max_seq_len = max_seq_len
    a.q = _dptr(q)
    a.k_new = _dptr(k_new)
    a.v_new = _dptr(v_new)
    a.pool = view
    a.k_cache = _dptr(k_cache)
    a.v_cache = _dptr(v_cache)
    a.out = _dptr(out)
    a.vlen_out = _dptr(vlen)
    a.kv_dtype = HSWA_KV_FP8 if k_scale is not None else HSWA_KV_BF16
    # the output tensor's dtype selects the output type
    if out is not None and str(out.dtype) not in ("torch.float32", "torch.float16"):
        raise ValueError(f"out must be float32 or float16, not {out.dtype}")
    a.out_dtype = 1 if out is not None and str(out.dtype) == "torch.float16" else 0
    a.k_scale = _dptr(k_scale)
    a.v_scale = _dptr(v_scale)
    a.q_pos = _dptr(q_pos)
    return a


def hswa_prefill_chunk(kind: int, window: int, q, k_new, v_new, seq_ids, cu_q,
                       max_q_len: int, view, k_cache, v_cache, out, vlen=None,
                       scale: float = 0.0, stream=None, q_pos=None, k_scale=None,
                       v_scale=None) -> None:
    """q [T, Hq, d] bf16; k_new/v_new [T, Hkv, d] bf16 or None; seq_ids [B] and
    cu_q [B+1] int32 device tensors; out [T, Hq, d] fp32 or fp16; vlen [T]
    int32; q_pos [B] int32 (optional): each sequence's first row position.
    With ``k_scale``/``v_scale`` the pages are FP8 (kv_cache_alloc_fp8)."""
    a = _args(kind, window, q, k_new, v_new, seq_ids, cu_q, q.shape[0], max_q_len, 0, view,
              k_cache, v_cache, out, vlen, scale, k_scale, v_scale, q_pos)
    _check(library().hswa_prefill_chunk(C.byref(a), _stream(stream)))


def hswa_decode_workspace_bytes(kind: int, window: int, num_seqs: int, num_q_heads: int,
                                num_kv_heads: int, head_dim: int, max_seq_len: int,
                                total_q: Optional[int] = None) -> int:
    """Workspace bytes of a decode call; ``total_q`` is the row count of a
    multi-row call (None: one row per sequence)."""
    a = _capi.AttnArgs()
    a.kind, a.window, a.num_seqs = kind, window, num_seqs
    a.num_q_heads, a.num_kv_heads, a.head_dim = num_q_heads, num_kv_heads, head_dim
    a.max_seq_len = max_seq_len
    a.total_q = num_seqs if total_q is None else total_q
    return int(library().hswa_decode_workspace_bytes(C.byref(a)))


def hswa_decode(kind: int, window: int, q, k_new, v_new, seq_ids, max_seq_len: int, view,
                k_cache, v_cache, out, workspace=None, vlen=None, scale: float = 0.0,
                stream=None, cu_q=None, max_q_len: int = 1, k_scale=None,
                v_scale=None, q_pos=None) -> None:
    """Decode step.  Without ``cu_q``: one query row per sequence (q [B, Hq, d])
    at position seq_len - 1.  With ``cu_q`` (device int32 [B+1]): 1..4 rows per
    sequence, its last positions (q [T, Hq, d]); ``max_q_len`` bounds them.
    With ``k_scale``/``v_scale`` the pages are FP8 (kv_cache_alloc_fp8)."""
    a = _args(kind, window, q, k_new, v_new, seq_ids, cu_q, q.shape[0],
              max_q_len if cu_q is not None else 1, max_seq_len, view, k_cache, v_cache, out,
              vlen, scale, k_scale, v_scale, q_pos)
    ws = _dptr(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(library().hswa_decode(C.byref(a), ws, nbytes, _stream(stream)))


def hswa_decode_noalloc(kind: int, window: int, q, k_new, v_new, seq_ids, max_seq_len: int,
                        view, k_cache, v_cache, out, vlen=None, scale: float = 0.0,
                        stream=None, cu_q=None, max_q_len: int = 1, k_scale=None,
                        v_scale=None, q_pos=None) -> None:
    """hswa_decode without a workspace: the split-K state goes to the
    library's device scratch (no allocation).  Calls on one GPU share it, so
    keep them on one stream."""
    a = _args(kind, window, q, k_new, v_new, seq_ids, cu_q, q.shape[0],
              max_q_len if cu_q is not None else 1, max_seq_len, view, k_cache, v_cache, out,
              vlen, scale, k_scale, v_scale, q_pos)
    _check(library().hswa_decode_noalloc(C.byref(a), _stream(stream)))


def hswa_append_kv(kind: int, k_new, v_new, seq_ids, view, k_cache, v_cache, cu_q=None,
                   max_q_len: int = 1, stream=None, k_scale=None, v_scale=None,
                   q_pos=None) -> None:
    """Writes k_new/v_new rows into this layer's pages (no attention); with
    ``k_scale``/``v_scale`` the pages are FP8 and the rows are quantized."""
    a = _args(kind, 1, None, k_new, v_new, seq_ids, cu_q, k_new.shape[0], max_q_len, 1, view,
              k_cache, v_cache, None, None, 0.0, k_scale, v_scale, q_pos)
    a.num_q_heads = k_new.shape[1]
    _check(library().hswa_append_kv(C.byref(a), _stream(stream)))


# ---------------------------------------------------------------------------
# Window-masked tier transfer


def hswa_pool_window_counts(pool: Pool, kind: int, seq_ids: Sequence[int]) -> np.ndarray:
    """Tokens a window-masked transfer moves per sequence (FULL: the length,
    SWA: min(length, W - 1))."""
    ids = _i32(seq_ids)
    out = np.empty(max(ids.size, 1), np.int32)
    _check(library().hswa_pool_window_counts(pool.handle, kind, ids.size, _p(ids), _p(out)))
    return out[:ids.size]


def _xfer_args(kind, seq_ids, cu_tok, total_tok, max_tok, view, k_cache, v_cache, buf_k, buf_v,
               first_pos, k_scale=None, v_scale=None, buf_k_scale=None, buf_v_scale=None):
    fp8 = k_scale is not None
    _expect("k_cache", k_cache, _U8 if fp8 else _BF16, (None, None, PAGE_SIZE, None))
    hkv, d = k_cache.shape[1], k_cache.shape[3]
    _expect("v_cache", v_cache, _U8 if fp8 else _F16, (k_cache.shape[0], hkv, d, PAGE_SIZE))
    _expect("k_scale", k_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    _expect("v_scale", v_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    scales = (v_scale, buf_k_scale, buf_v_scale)
    if any((t is None) == fp8 for t in scales):
        raise ValueError("FP8 pages need k_scale, v_scale, buf_k_scale and buf_v_scale; "
                         "BF16 pages none of them")
    _expect("seq_ids", seq_ids, _I32, (None,))
    _expect("cu_tok", cu_tok, _I32, (seq_ids.shape[0] + 1,))
    _expect("first_pos", first_pos, _I32, (seq_ids.shape[0],))
    # the packed buffers may be pinned host memory; the library checks that
    words = _U8 if fp8 else _BF16 + _F16 + ("torch.int16",)
    _expect("buf_k", buf_k, words, (None, hkv, d), total_tok, device=False)
    _expect("buf_v", buf_v, words, (None, hkv, d), total_tok, device=False)
    _expect("buf_k_scale", buf_k_scale, _F32, (None, hkv), total_tok, device=False)
    _expect("buf_v_scale", buf_v_scale, _F32, (None, hkv), total_tok, device=False)
    a = _capi.XferArgs()
    a.kind = kind
    a.num_kv_heads = k_cache.shape[1]
    a.head_dim = k_cache.shape[-1]
    a.num_seqs = seq_ids.shape[0]
    a.seq_ids = _dptr(seq_ids)
    a.cu_tok = _dptr(cu_tok)
    a.first_pos = _dptr(first_pos)
    a.total_tok = total_tok
    a.max_tok = max_tok
    a.pool = view
    a.k_cache = _dptr(k_cache)
    a.v_cache = _dptr(v_cache)
    a.buf_k = _dptr(buf_k)
    a.buf_v = _dptr(buf_v)
    a.kv_dtype = HSWA_KV_FP8 if fp8 else HSWA_KV_BF16
    a.k_scale, a.v_scale = _dptr(k_scale), _dptr(v_scale)
    a.buf_k_scale, a.buf_v_scale = _dptr(buf_k_scale), _dptr(buf_v_scale)
    return a


def hswa_kv_offload(kind: int, seq_ids, cu_tok, total_tok: int, max_tok: int, view, k_cache,
                    v_cache, buf_k, buf_v, stream=None, first_pos=None, k_scale=None,
                    v_scale=None, buf_k_scale=None, buf_v_scale=None) -> None:
    """Copies n_i = cu_tok[i+1]-cu_tok[i] positions of each listed sequence
    (from first_pos[i], or its last n_i) from this layer's pages into buf_k
    (bf16) / buf_v (fp16), [T, Hkv, d], pinned host or device tensors.  FP8
    pages (k_scale/v_scale given): buf_k/buf_v are uint8 codes [T, Hkv, d]
    and buf_k_scale/buf_v_scale fp32 [T, Hkv]."""
    a = _xfer_args(kind, seq_ids, cu_tok, total_tok, max_tok, view, k_cache, v_cache, buf_k,
                   buf_v, first_pos, k_scale, v_scale, buf_k_scale, buf_v_scale)
    _check(library().hswa_kv_offload(C.byref(a), _stream(stream)))


def hswa_kv_restore(kind: int, seq_ids, cu_tok, total_tok: int, max_tok: int, view, k_cache,
                    v_cache, buf_k, buf_v, stream=None, first_pos=None, k_scale=None,
                    v_scale=None, buf_k_scale=None, buf_v_scale=None) -> None:
    """Writes buf_k/buf_v (and, for FP8 pages, the scale buffers) back into
    this layer's pages at those positions."""
    a = _xfer_args(kind, seq_ids, cu_tok, total_tok, max_tok, view, k_cache, v_cache, buf_k,
                   buf_v, first_pos, k_scale, v_scale, buf_k_scale, buf_v_scale)
    _check(library().hswa_kv_restore(C.byref(a), _stream(stream)))


def hswa_kv_copy(kind: int, src_ids, dst_ids, first_pos, end_pos, max_tok: int, view, k_cache,
                 v_cache, stream=None, k_scale=None, v_scale=None) -> None:
    """Copies this layer's K/V of positions [first_pos[i], end_pos[i]) from
    sequence src_ids[i] to dst_ids[i] (device int32 tensors), page to page,
    e.g. after hswa_pool_fork.  With ``k_scale``/``v_scale`` the pages are
    FP8 and each position's scales copy with its codes."""
    fp8 = k_scale is not None
    _expect("k_cache", k_cache, _U8 if fp8 else _BF16, (None, None, PAGE_SIZE, None))
    hkv, d = k_cache.shape[1], k_cache.shape[3]
    _expect("v_cache", v_cache, _U8 if fp8 else _F16, (k_cache.shape[0], hkv, d, PAGE_SIZE))
    _expect("k_scale", k_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    _expect("v_scale", v_scale, _F32, (k_cache.shape[0], hkv, PAGE_SIZE))
    if fp8 != (v_scale is not None):
        raise ValueError("FP8 pages need both k_scale and v_scale")
    for name, t in (("src_ids", src_ids), ("dst_ids", dst_ids), ("first_pos", first_pos),
                    ("end_pos", end_pos)):
        _expect(name, t, _I32, (src_ids.shape[0],))
    a = _capi.KvCopyArgs()
    a.kind, a.num_kv_heads, a.head_dim = kind, hkv, d
    a.num_seqs = src_ids.shape[0]
    a.src_ids, a.dst_ids = _dptr(src_ids), _dptr(dst_ids)
    a.first_pos, a.end_pos = _dptr(first_pos), _dptr(end_pos)
    a.max_tok = max_tok
    a.pool = view
    a.k_cache, a.v_cache = _dptr(k_cache), _dptr(v_cache)
    a.kv_dtype = HSWA_KV_FP8 if fp8 else HSWA_KV_BF16
    a.k_scale, a.v_scale = _dptr(k_scale), _dptr(v_scale)
    _check(library().hswa_kv_copy(C.byref(a), _stream(stream)))
