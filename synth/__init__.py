"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws numbers and sizes: it holds none of the attention or
pool arithmetic.  Every draw is reproducible from (seed, role, index) so the
two sides can be fed identical inputs without one side producing them for
the other.

Value recipe: N(0, 1) fp32 rounded to bf16 (round to nearest even), the
distribution the workload descriptions fix.  Integer recipe: inclusive
uniform lengths, uniform random permutations of page ids.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

try:  # torch is used only to hold the drawn values in device memory
    import torch
except ImportError:  # pragma: no cover - torch is present in this image
    torch = None

# Role offsets so that different tensors drawn from one base seed never share
# a stream.
ROLE_Q, ROLE_K, ROLE_V = 1, 2, 3
ROLE_LEN, ROLE_PERM, ROLE_RING = 11, 12, 13
ROLE_ACCEPT = 14


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from a tuple of non-negative ints (splitmix64)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x = (x ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


def seed_for(*parts: int) -> int:
    return _mix(*parts)


def bf16_normal(shape: Sequence[int], *seed_parts: int, device="cpu"):
    """N(0,1) draws rounded to bf16, as a torch bf16 tensor on ``device``.

    The same seed gives the same tensor for a given device type; tests that
    compare two sides draw once and move the tensor, never redraw.
    """
    if torch is None:
        raise RuntimeError("torch is required for bf16 tensors")
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*seed_parts))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, device=device,
                    dtype=torch.float32)
    return x.to(torch.bfloat16)


def bf16_normal_np(shape: Sequence[int], *seed_parts: int) -> np.ndarray:
    """Same recipe on the host, returned as float64 values exactly equal to
    the bf16 numbers (bf16 -> fp64 is exact)."""
    t = bf16_normal(shape, *seed_parts, device="cpu")
    return t.to(torch.float64).numpy()


def to_f64(t) -> np.ndarray:
    """bf16/fp32 torch tensor (any device) -> float64 numpy array, exact."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def uniform_lengths(n: int, lo: int, hi: int, *seed_parts: int) -> List[int]:
    """n integers uniform on the inclusive range [lo, hi]."""
    rng = np.random.default_rng(seed_for(ROLE_LEN, *seed_parts))
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def permutation(n: int, *seed_parts: int) -> np.ndarray:
    """A uniform random permutation of 0..n-1 as int32."""
    rng = np.random.default_rng(seed_for(ROLE_PERM, *seed_parts))
    return rng.permutation(n).astype(np.int32)


def uniform_ints(n: int, lo: int, hi: int, *seed_parts: int) -> List[int]:
    """n integers uniform on [lo, hi] from their own stream (e.g. how many
    draft tokens of a step are accepted)."""
    rng = np.random.default_rng(seed_for(ROLE_ACCEPT, *seed_parts))
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def sample_indices(n: int, k: int, *seed_parts: int) -> List[int]:
    """k distinct sorted indices from range(n) (all of them if k >= n)."""
    if k >= n:
        return list(range(n))
    rng = np.random.default_rng(seed_for(ROLE_LEN + 100, *seed_parts))
    return sorted(int(x) for x in rng.choice(n, size=k, replace=False))


# ---------------------------------------------------------------------------
# Workload descriptions (sizes only).  Each mirrors one of the five
# workloads: numbers are the workload's, the recipe is the one above.


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    page_size: int = 16
    seed: int = 0


@dataclasses.dataclass(frozen=True)
class SwaSingleChunk(Workload):
    """One SWA layer, one sequence, one prefill chunk then decode steps."""
    prefill_len: int = 1024
    decode_steps: int = 16


@dataclasses.dataclass(frozen=True)
class SwaChunkedPrefill(Workload):
    """SWA-only chunked prefill over a batch of sequences."""
    num_seqs: int = 8
    len_lo: int = 2048
    len_hi: int = 16384
    chunk: int = 2048


@dataclasses.dataclass(frozen=True)
class MixedDecode(Workload):
    """Decode over one Full and one SWA layer."""
    num_seqs: int = 256
    ctx_lo: int = 4096
    ctx_hi: int = 32768
    ring_slots: int = 128


@dataclasses.dataclass(frozen=True)
class HybridStack(Workload):
    """Attention-only stack of SWA and Full layers, chunked prefill."""
    seq_len: int = 65536
    chunk: int = 4096
    pattern: str = "SSSSSSF" * 10


@dataclasses.dataclass(frozen=True)
class LongDecode(Workload):
    """Long-context hybrid decode over a 6:1 SWA:Full pattern."""
    num_seqs: int = 64
    ctx_lo: int = 131072
    ctx_hi: int = 262144
    pattern: str = "SSSSSSF" * 2
    ring_slots: int = 128 + 256


@dataclasses.dataclass(frozen=True)
class MtpDecode(Workload):
    """Multi-token decode: each step verifies one token plus draft tokens
    (three MTP layers give three drafts) over one Full and one SWA layer,
    then keeps the accepted prefix."""
    num_seqs: int = 256
    ctx_lo: int = 4096
    ctx_hi: int = 32768
    drafts: int = 3
    ring_slots: int = 128 + 16


C1 = SwaSingleChunk("swa_single_chunk_1x1024_h8kv2_d64", 8, 2, 64, 128, seed=100)
C2 = SwaChunkedPrefill("swa_chunked_prefill_8seq_2k-16k_h64kv8_d128", 64, 8, 128, 128, seed=200)
C3 = MixedDecode("mixed_decode_256seq_4k-32k_full+swa_h64kv8_d128", 64, 8, 128, 128, seed=300)
C4 = HybridStack("hybrid_stack_70L_64k_chunk4k_h64kv8_d128", 64, 8, 128, 128, seed=400)
C5 = LongDecode("long_decode_64seq_128k-256k_14L_h64kv8_d128", 64, 8, 128, 128, seed=500)

@dataclasses.dataclass(frozen=True)
class TierTransfer(Workload):
    """Window-masked offload and restore of a hybrid stack's KV between HBM
    and pinned host memory, then the first decode step."""
    num_seqs: int = 16
    ctx_lo: int = 4096
    ctx_hi: int = 32768
    pattern: str = "SSSSSSF" * 2
    ring_slots: int = 128


MTP = MtpDecode("mtp_decode_256seq_4k-32k_q4_full+swa_h64kv8_d128", 64, 8, 128, 128, seed=600)

TIER = TierTransfer("tier_transfer_16seq_4k-32k_14L_h64kv8_d128", 64, 8, 128, 128, seed=700)

WORKLOADS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5, "MTP": MTP, "TIER": TIER}
