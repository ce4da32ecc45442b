"""fp64 attention with explicit window masks -- the oracle's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (MiMo-V2.5 inference page, section 1.1 and the
introduction): causal attention in which a SWA layer lets each query see only
the most recent W tokens and a Full layer lets it see the whole prefix.

Readings taken where the pages leave a step open:

* The window holds W keys counting the query itself: query position i sees
  keys j with max(0, i - W + 1) <= j <= i.  (Section 2.1, prefix-tree point
  1, asks for the last W tokens to be valid, which is the same count.)
* Softmax scale tau = 1/sqrt(head_dim) unless a caller passes another one.
* Grouped-query attention (the page compares against a "pure GQA"
  architecture, section 4.2): query head h reads KV head floor(h / g) with
  g = Hq / Hkv, i.e. contiguous groups.
* Every query attends to itself (its K/V is written before attention), so a
  window is never empty.

K and V are contiguous per sequence, [L, Hkv, d]; the oracle never sees pages,
rings or chunks.  Chunked prefill and decode are this same formula evaluated
at the chunk's (or the new token's) absolute positions.
"""
from __future__ import annotations

import numpy as np

FULL = 0
SWA = 1


def key_range(pos: int, kind: int, window: int):
    """Half-open key range [lo, hi) that query position ``pos`` attends to."""
    if pos < 0:
        raise ValueError("negative position")
    if kind == FULL:
        lo = 0
    elif kind == SWA:
        if window < 1:
            raise ValueError("window must be >= 1")
        lo = max(0, pos - window + 1)
    else:
        raise ValueError(f"unknown layer kind {kind}")
    return lo, pos + 1


def valid_length(pos: int, kind: int, window: int) -> int:
    """Number of keys the query at ``pos`` attends to (its valid window)."""
    lo, hi = key_range(pos, kind, window)
    return hi - lo


def attend(q, positions, k, v, kind: int, window: int, scale: float | None = None):
    """Attention outputs for the given query rows of one sequence.

    q          [n, Hq, d]   query rows (any float dtype; used in fp64)
    positions  [n]          absolute position of each row in the sequence
    k, v       [L, Hkv, d]  contiguous keys/values of the sequence, L > max(positions)
    kind       FULL or SWA; ``window`` is W (ignored for FULL)
    returns    [n, Hq, d] float64

    For row r at position i, head h, kv head kappa = h // g:
        s_j = tau * <q[r, h], k[j, kappa]>      for j in the key range of i
        o   = sum_j exp(s_j - max s) v[j, kappa] / sum_j exp(s_j - max s)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, dk = k.shape
    if dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    tau = 1.0 / np.sqrt(d) if scale is None else float(scale)
    positions = [int(p) for p in positions]
    if len(positions) != n:
        raise ValueError("one position per query row")
    out = np.empty((n, hq, d), dtype=np.float64)
    for r, pos in enumerate(positions):
        lo, hi = key_range(pos, kind, window)
        if hi > L:
            raise ValueError("position beyond the stored keys")
        for kv in range(hkv):
            heads = slice(kv * g, (kv + 1) * g)
            s = tau * (q[r, heads] @ k[lo:hi, kv].T)          # [g, |J|]
            w = np.exp(s - s.max(axis=1, keepdims=True))
            out[r, heads] = (w @ v[lo:hi, kv]) / w.sum(axis=1, keepdims=True)
    return out


def attend_sequence(q, k, v, kind: int, window: int, scale: float | None = None,
                    start: int = 0):
    """Outputs for consecutive query rows at positions start .. start+n-1."""
    n = np.asarray(q).shape[0]
    return attend(q, range(start, start + n), k, v, kind, window, scale)
