"""Host-side checks of bench.py's own C-ABI argument builder (no GPU).

The kernels write 4 or 2 bytes per output element as out_dtype says, so the
builder must set out_dtype from the output buffer it passes."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hybrid_sliding_window_hswa_amd import _capi  # noqa: E402


class _Cx:
    torch = torch


def _build(out):
    t = torch.zeros(4, dtype=torch.int32)
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    return bench._attn_args(_Cx(), 1, 16, 8, 2, 64, t, t, 2, 1, 16, _capi.PoolView(), q, None,
                            None, kc, kc, out)


def test_out_dtype_follows_the_output_buffer():
    assert _build(torch.zeros((2, 8, 64), dtype=torch.float32)).out_dtype == 0
    assert _build(torch.zeros((2, 8, 64), dtype=torch.float16)).out_dtype == 1
    assert _build(None).out_dtype == 0
    with pytest.raises(ValueError):
        _build(torch.zeros((2, 8, 64), dtype=torch.bfloat16))
