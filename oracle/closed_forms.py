"""Counts of scored (query, key) pairs and resident KV, and their ratios.

TEST INFRASTRUCTURE ONLY (see the package docstring).

MiMo-V2.5 inference page, section 1.1: with 70 layers of which 10 are Full
and 60 are SWA with a 128-token window, attention compute of the hybrid
model is about 1/7 of an all-Full model.  Section 1.2: KV storage drops to
nearly 1/7 as well.  Section 2.1 ("KVCache Dual Pool"): the dual pool raises
KV capacity efficiency about 7x.  All three are the long-sequence limits of
the counts below (the SWA terms stop growing once N exceeds W).

Parity unpinned: section 5.1 of the same page quotes an effective KV
capacity of about 5x for decode.  It does not follow from these counts at
long context (it equals 5 only near N = 2k tokens) and the page gives no
derivation, so no test asserts it.
"""
from __future__ import annotations


def pairs_full(n: int) -> int:
    """Pairs scored by causal Full attention over n positions: sum_{i<n} (i+1)."""
    return n * (n + 1) // 2


def pairs_swa(n: int, window: int) -> int:
    """Pairs scored by SWA over n positions: sum_{i<n} min(i+1, W)."""
    if n <= window:
        return pairs_full(n)
    return n * window - window * (window - 1) // 2


def stack_pair_ratio(n: int, n_swa: int, n_full: int, window: int) -> float:
    """Scored pairs of a hybrid stack relative to the same stack all Full."""
    hybrid = n_swa * pairs_swa(n, window) + n_full * pairs_full(n)
    return hybrid / ((n_swa + n_full) * pairs_full(n))


def stack_kv_ratio(n: int, n_swa: int, n_full: int, window: int) -> float:
    """Resident KV tokens of a hybrid stack relative to all Full (W per SWA layer)."""
    return (n_swa * min(n, window) + n_full * n) / ((n_swa + n_full) * n)


def capacity_gain(n: int, n_swa: int, n_full: int, window: int) -> float:
    """How many times more tokens fit in a fixed KV budget: 1 / KV ratio."""
    return 1.0 / stack_kv_ratio(n, n_swa, n_full, window)


def attention_flops(pairs: int, num_q_heads: int, head_dim: int) -> int:
    """Multiply-adds of QK^T and PV counted as 2 flops each: 4 * d * Hq per pair."""
    return 4 * head_dim * num_q_heads * pairs
