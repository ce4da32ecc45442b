"""Window-masked KV transfer between the device pools and host memory.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (MiMo-V2.5 inference page, section 2.1 "KVCache Dual
Pool", point "Data Transfer", and "KVCache asynchronous layer-by-layer
pulling"): moving KV between cache tiers goes by the SWA mask, so only the
valid window of a SWA layer crosses the link, while a Full layer moves its
whole sequence.  The SWA layers then prefetch so little that the host->device
pull can hide behind compute layer by layer.

Readings taken where the pages leave a step open:

* The SWA mask of a sequence of length L is the window the next query reads,
  positions [max(0, L - W + 1), L): W - 1 keys plus the query itself make the
  W-key window.  After eviction these are exactly the positions whose map
  entry is >= 0 (tests check the two agree).
* The host copy is packed: sequences in the order listed, positions
  ascending, each token [Hkv][d] for K and for V.  It holds what the pool
  holds: K as the bf16 input, V as the fp16 value of the bf16 input (the
  pool's V format), so a restore puts back the same bits.
* FP8 pages (Baidu Day0 hybrid-attention article, Layered quantization,
  point 2) cross the link as they are stored: each token's e4m3 codes
  [Hkv][d] for K and for V (V token-major like K) and its fp32 scale per
  (token, head) for each, so the same mask moves 2 bytes per element plus
  8 bytes per (token, head).
"""
from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np

from oracle import fp8

FULL = 0
SWA = 1


def transfer_positions(kind: int, length: int, window: int) -> range:
    """Positions of one sequence that a window-masked transfer moves."""
    if length < 0:
        raise ValueError("negative length")
    if kind == FULL:
        return range(0, length)
    if kind == SWA:
        if window < 1:
            raise ValueError("window must be >= 1")
        return range(max(0, length - window + 1), length)
    raise ValueError(f"unknown layer kind {kind}")


def transfer_counts(kind: int, lengths: Sequence[int], window: int) -> List[int]:
    return [len(transfer_positions(kind, L, window)) for L in lengths]


def transfer_bytes(kind: int, lengths: Sequence[int], window: int, hkv: int, d: int) -> int:
    """Bytes a window-masked transfer moves: K (2 B) and V (2 B) per element."""
    return sum(transfer_counts(kind, lengths, window)) * hkv * d * 4


def transfer_bytes_fp8(kind: int, lengths: Sequence[int], window: int, hkv: int,
                       d: int) -> int:
    """Bytes a window-masked transfer of FP8 pages moves: a code byte of K
    and of V per element, and an fp32 K and V scale per (token, head)."""
    return sum(transfer_counts(kind, lengths, window)) * hkv * (2 * d + 8)


def host_image(kind: int, window: int, seqs: Iterable[Tuple[np.ndarray, np.ndarray]]):
    """Packed host buffers a transfer of these sequences holds.

    seqs yields, per sequence in listed order, (k, v): the full bf16 inputs
    [L, Hkv, d] as uint16 bit patterns.  Returns (host_k uint16, host_v
    uint16 fp16 bit patterns), each [tokens, Hkv, d].
    """
    ks, vs = [], []
    for k, v in seqs:
        k = np.asarray(k, dtype=np.uint16)
        v = np.asarray(v, dtype=np.uint16)
        pos = transfer_positions(kind, k.shape[0], window)
        sel = slice(pos.start, pos.stop)
        ks.append(k[sel])
        # bf16 bits -> float32 (exact) -> float16 with round to nearest even
        v32 = (v[sel].astype(np.uint32) << 16).view(np.float32)
        vs.append(v32.astype(np.float16).view(np.uint16))
    if not ks:
        return np.zeros((0,), np.uint16), np.zeros((0,), np.uint16)
    return np.concatenate(ks), np.concatenate(vs)


def host_image_fp8(kind: int, window: int, seqs: Iterable[Tuple[np.ndarray, np.ndarray]]):
    """Packed buffers a transfer of FP8 pages holds.

    seqs yields, per sequence in listed order, (k, v): the full inputs
    [L, Hkv, d] as fp32 values (bf16 inputs convert exactly).  Each moved
    token holds what the quantizing append stored for it (one tile per
    (token, head) row).  Returns (codes_k, codes_v) uint8 [tokens, Hkv, d]
    and (scale_k, scale_v) float32 [tokens, Hkv].
    """
    out = [[], [], [], []]
    for k, v in seqs:
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        pos = transfer_positions(kind, k.shape[0], window)
        sel = slice(pos.start, pos.stop)
        ck, sk = fp8.quantize_rows(k[sel])
        cv, sv = fp8.quantize_rows(v[sel])
        for lst, x in zip(out, (ck, cv, sk, sv)):
            lst.append(x)
    if not out[0]:
        return (np.zeros((0,), np.uint8), np.zeros((0,), np.uint8),
                np.zeros((0,), np.float32), np.zeros((0,), np.float32))
    return tuple(np.concatenate(lst) for lst in out)
