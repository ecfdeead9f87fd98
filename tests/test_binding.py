"""Host-side checks of the Python binding (no GPU): caller-provided outputs
are validated before anything is launched."""
import pytest
import torch

import mla_paged_kv_fwd_amd as mla


def test_caller_outputs_are_checked():
    q = torch.empty((2, 1, 16, 576), dtype=torch.bfloat16)
    bad_out = [torch.empty((2, 1, 16, 511), dtype=torch.bfloat16),
               torch.empty((2, 1, 16, 512), dtype=torch.float32),
               torch.empty((2, 2, 16, 512), dtype=torch.bfloat16),
               torch.empty((2, 1, 16, 1024), dtype=torch.bfloat16)[..., ::2]]
    for out in bad_out:
        with pytest.raises(mla.MlaError):
            mla._outputs(q, out, None)
    for lse in (torch.empty((2, 1, 15), dtype=torch.float32),
                torch.empty((2, 1, 16), dtype=torch.bfloat16)):
        with pytest.raises(mla.MlaError):
            mla._outputs(q, None, lse)
    # right dtype and shape, but host memory: rejected as well
    with pytest.raises(mla.MlaError):
        mla._outputs(q, torch.empty((2, 1, 16, 512), dtype=torch.bfloat16), None)


def test_inputs_are_checked_before_any_launch():
    q = torch.empty((2, 1, 16, 576), dtype=torch.bfloat16)
    kc = torch.empty((4, 64, 576), dtype=torch.bfloat16)
    bt = torch.zeros((2, 2), dtype=torch.int32)
    with pytest.raises(mla.MlaError):
        mla._validate(q[..., :575], kc, bt, None, False)
    with pytest.raises(mla.MlaError):
        mla._validate(q, kc, bt, None, True)  # a bf16 cache passed as FP8 records
    with pytest.raises(mla.MlaError):
        mla._validate(q, kc, bt, torch.zeros((2,), dtype=torch.int64), False)
    with pytest.raises(mla.MlaError):
        mla._validate(q, kc, bt, None, False)  # host tensors
