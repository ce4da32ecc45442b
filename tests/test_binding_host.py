"""The Python binding's argument checks (host only, no kernel runs): a
tensor of the wrong dtype, shape, row count or memory kind is refused before
its address reaches the library."""
import pytest
import torch

import hybrid_sliding_window_hswa_amd as H


def _q(rows=10, hq=8, d=64, dtype=torch.bfloat16):
    return torch.zeros((rows, hq, d), dtype=dtype)


def test_accepts_matching_tensor():
    H._expect("q", _q(), H._BF16, (None, None, 64), 10, device=False)
    H._expect("q", None, H._BF16, (None, None, 64), 10)   # absent arguments pass


@pytest.mark.parametrize("call,msg", [
    (lambda: H._expect("q", _q(dtype=torch.float16), H._BF16, (None, None, 64), 10,
                       device=False), "must be torch.bfloat16"),
    (lambda: H._expect("q", _q(), H._BF16, (None, None, 128), 10, device=False),
     "expected"),
    (lambda: H._expect("q", _q(), H._BF16, (None, 64), 10, device=False), "expected"),
    (lambda: H._expect("q", _q(), H._BF16, (None, None, 64), 11, device=False),
     "the call needs 11"),
    (lambda: H._expect("q", _q(), H._BF16, (None, None, 64), 10), "device tensor"),
])
def test_refuses_mismatch(call, msg):
    with pytest.raises(ValueError, match=msg):
        call()


def test_attention_args_refuse_host_tensors():
    kc, vc = H.kv_cache_alloc(4, 2, 64, "cpu")
    q = _q(4, 8, 64)
    ids = torch.zeros(1, dtype=torch.int32)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    out = torch.zeros((4, 8, 64))
    with pytest.raises(ValueError, match="device tensor"):
        H.hswa_prefill_chunk(H.SWA, 16, q, None, None, ids, cu, 4, H._capi.PoolView(), kc, vc,
                             out)
