"""GPU test of the allocation-free decode (mla_decode_fwd_noalloc) through
the C ABI: two calls in a row, the second with a smaller problem, each equal
bit for bit to mla_decode_fwd / mla_decode_fwd_fp8 with the same plan size,
and within the parity bar of the oracle; and a problem larger than the
scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import compare, oracle_all, to_device
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu

WORKSPACE = -3


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_decode_equals_decode(fp8):
    import mla_paged_kv_fwd_amd as mla

    problems = [([300, 1000, 2100, 64, 0, 5], 2, 128, True, 500),  # the larger call first
                ([37, 100], 1, 16, False, 501)]
    for seqlens, s_q, h_q, causal, seed in problems:
        print(f"noalloc fp8={fp8} seqlens={seqlens} s_q={s_q} h_q={h_q}", flush=True)
        case = W.make_case(seqlens, s_q, h_q, seed=seed, causal=causal, fp8=fp8, spare_pages=1,
                           poison=True)
        q, kc, bt, sl = to_device(case)
        assert 0 < mla.noalloc_scratch_need(case.batch, s_q, h_q, fp8) <= (128 << 20)
        ref_out, ref_lse = mla.decode(q, kc, bt, sl, case.scale, causal, fp8=fp8)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        mla.decode_noalloc(q, kc, bt, sl, case.scale, causal, out=out, lse=lse, fp8=fp8)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        o_ref, l_ref = oracle_all(case)
        compare(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref,
                f"noalloc fp8={fp8} {seqlens}")


def test_noalloc_long_context_plan_equals_decode():
    # 128 rows per request with parts long enough for one part per CU: both
    # calls plan one part per CU (the 128-row kernel) from the table's width
    import mla_paged_kv_fwd_amd as mla

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    one_per_cu = (cus + 7) // 8 * 8
    length = 8192
    batch = -(-48 * one_per_cu // (length // 64))
    assert mla.default_num_parts(1, 128, batch=batch, max_seqlen=length) == one_per_cu
    print(f"noalloc long context: batch {batch} x {length}, parts {one_per_cu}", flush=True)
    sl = np.full(batch, length, dtype=np.int32)
    q, kc, bt, slt = W.make_device_inputs(sl, 1, 128, False, seed=502)
    scale = 1.0 / np.sqrt(W.D_QK)
    assert 0 < mla.noalloc_scratch_need(batch, 1, 128) <= (128 << 20)
    ref_out, ref_lse = mla.decode(q, kc, bt, slt, scale, False)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    mla.decode_noalloc(q, kc, bt, slt, scale, False, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_noalloc_refuses_problems_beyond_its_scratch():
    import mla_paged_kv_fwd_amd as mla

    # 16384 requests x 128 rows: the split workspace alone is over 4 GB
    batch, s_q, h_q = 16384, 1, 128
    assert mla.noalloc_scratch_need(batch, s_q, h_q) > (128 << 20)
    q = torch.empty((batch, s_q, h_q, 576), dtype=torch.bfloat16, device="cuda")
    kc = torch.empty((4, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((batch, 1), dtype=torch.int32, device="cuda")
    sl = torch.ones((batch,), dtype=torch.int32, device="cuda")
    out = torch.empty((batch, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device="cuda")
    rc = mla.lib().mla_decode_fwd_noalloc(
        mla._ptr(q), mla._ptr(kc), 0, kc.shape[0], mla._ptr(bt), 1, mla._ptr(sl), batch, s_q,
        h_q, 0.04, 0, mla._ptr(out), mla._ptr(lse), mla._stream())
    assert rc == WORKSPACE
