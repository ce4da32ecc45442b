"""The V pages' input domain: the append converts bf16 V to fp16 (the PV
product runs on the fp16 MFMA) with round to nearest even, for every one of
the 65,536 bf16 bit patterns exactly as the binary16 definition says:

- every bf16 value with 2^-14 <= |v| <= 65280 is exact in fp16 (65280 is the
  largest bf16 below fp16's limit of 65504);
- smaller magnitudes round to fp16 subnormals (error <= 2^-25);
- |v| >= 65536 (the next bf16 value) becomes +-inf, inf stays inf, NaN stays
  NaN.

The oracle's conversion (numpy, itself pinned against an encoder written
from the IEEE 754 binary16 definition in tests/test_oracle_transfer.py) is
the reference; the page contents come back through the transfer kernel.
"""
import numpy as np
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H

from harness import Setup, dev

pytestmark = pytest.mark.gpu


def test_append_converts_every_bf16_v_value_by_the_binary16_definition(gpu):
    hkv, d = 4, 128
    T = 65536 // (hkv * d)                       # 128 tokens hold every bit pattern
    st = Setup(H.FULL, 16, 16, 1, T // 16 + 1, T // 16 + 2, hkv, d, seed=171)
    H.hswa_pool_import(st.pool, [0], [T])     # Full slots for all, no ring check
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, hkv, d)
    v_new = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev())
    k_new = torch.zeros((T, hkv, d), dtype=torch.bfloat16, device=dev())
    sid = torch.zeros(1, dtype=torch.int32, device=dev())
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev())
    H.hswa_append_kv(H.FULL, k_new, v_new, sid, st.view, st.kc, st.vc, cu, T)
    bk = torch.empty((T, hkv, d), dtype=torch.bfloat16, device=dev())
    bv = torch.empty((T, hkv, d), dtype=torch.float16, device=dev())
    H.hswa_kv_offload(H.FULL, sid, cu, T, T, st.view, st.kc, st.vc, bk, bv)
    torch.cuda.synchronize()
    got = bv.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    v32 = (bits.reshape(-1).astype(np.uint32) << 16).view(np.float32)
    with np.errstate(over="ignore"):  # the patterns past fp16's range become inf, as checked below
        want = v32.astype(np.float16)
    nan = np.isnan(v32)
    assert np.all(np.isnan(got[nan].view(np.float16)))
    assert np.array_equal(got[~nan], want.view(np.uint16)[~nan])
    # the stated domain, read off the same conversion
    a = np.abs(v32)
    exact = (a >= 2.0 ** -14) & (a <= 65280.0)
    assert np.array_equal(got[exact].view(np.float16).astype(np.float32), v32[exact])
    big = ~nan & (a >= 65536.0)
    assert np.all(np.isinf(got[big].view(np.float16)))
    assert np.all(np.sign(got[big].view(np.float16)) == np.sign(v32[big]))
    small = ~nan & (a < 2.0 ** -14)
    err = np.abs(got[small].view(np.float16).astype(np.float64) - v32[small].astype(np.float64))
    assert float(err.max()) <= 2.0 ** -25
