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


def test_batch_agreement_is_checked():
    """seqlens and block_table rows must match q's batch: the kernels index
    them by q's request index and size out and the workspace from q."""
    q = torch.empty((2, 1, 16, 576), dtype=torch.bfloat16)
    kc = torch.empty((4, 64, 576), dtype=torch.bfloat16)
    with pytest.raises(mla.MlaError, match="block_table"):
        mla._validate(q, kc, torch.zeros((3, 2), dtype=torch.int32), None, False)
    with pytest.raises(mla.MlaError, match="block_table"):
        mla._validate(q, kc, torch.zeros((1, 2), dtype=torch.int32), None, False)


class _FakeCuda:
    """Stands in for a device tensor in host-side checks (no GPU here)."""

    def __init__(self, t):
        self._t = t
        self.dtype, self.shape, self.device = t.dtype, t.shape, torch.device("cuda", 0)
        self.is_cuda = True

    def dim(self):
        return self._t.dim()

    def numel(self):
        return self._t.numel()

    def is_contiguous(self):
        return self._t.is_contiguous()


def test_caller_plan_and_workspace_are_checked():
    q = _FakeCuda(torch.empty((2, 1, 16, 576), dtype=torch.bfloat16))
    good_meta = _FakeCuda(torch.empty((8, 8), dtype=torch.int32))
    good_sb = _FakeCuda(torch.empty((3,), dtype=torch.int32))
    mla._check_plan(q, good_meta, good_sb, 8)
    mla._check_plan(q, None, None, None)
    for meta, sb, parts in ((good_meta, good_sb, 16),                               # parts disagree
                            (_FakeCuda(torch.empty((8, 7), dtype=torch.int32)), good_sb, 8),
                            (good_meta, _FakeCuda(torch.empty((2,), dtype=torch.int32)), 8),
                            (good_meta, _FakeCuda(torch.empty((3,), dtype=torch.int64)), 8),
                            (good_meta, None, 8),
                            (torch.empty((8, 8), dtype=torch.int32), good_sb, 8)):  # host memory
        with pytest.raises(mla.MlaError):
            mla._check_plan(q, meta, sb, parts)
    need = 1000
    assert mla._workspace(q, 8, _FakeCuda(torch.empty((need,), dtype=torch.uint8)), need) is not None
    for ws in (_FakeCuda(torch.empty((need - 1,), dtype=torch.uint8)),
               _FakeCuda(torch.empty((need,), dtype=torch.int8)),
               _FakeCuda(torch.empty((2, need), dtype=torch.uint8)),
               torch.empty((need,), dtype=torch.uint8)):                         # host memory
        with pytest.raises(mla.MlaError):
            mla._workspace(q, 8, ws, need)


def test_seqlens_batch_agreement_is_checked():
    q = torch.empty((2, 1, 16, 576), dtype=torch.bfloat16)
    kc = torch.empty((4, 64, 576), dtype=torch.bfloat16)
    bt = torch.zeros((2, 2), dtype=torch.int32)
    for n in (1, 3):
        with pytest.raises(mla.MlaError, match="seqlens"):
            mla._validate(q, kc, bt, torch.zeros((n,), dtype=torch.int32), False)
