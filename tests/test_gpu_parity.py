"""GPU parity: libmla (through its C ABI) against the fp64 CPU oracle on the
same seeded inputs.  Small cases compare every output; the full-size workloads
compare a deterministic sample of rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare, oracle_all, run_gpu, sample_rows, to_device
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def test_tiny_workload_matches_oracle():
    case = W.make_config("tiny")
    out, lse = run_gpu(case)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, "tiny")


SHAPES = [
    # seqlens, s_q, h_q, causal, fp8
    ([1, 63, 64, 65, 127, 128, 200, 1000], 1, 16, False, False),
    ([1, 63, 64, 65, 127, 128, 200, 1000], 2, 16, True, False),
    ([2, 64, 129, 700], 1, 32, False, False),
    ([2, 65, 300], 2, 32, True, False),
    ([3, 64, 190, 513], 1, 64, False, False),
    ([5, 64, 257], 1, 128, False, False),
    ([2, 66, 130, 400], 2, 128, True, False),
    ([1, 63, 64, 65, 200, 1000], 1, 16, False, True),
    ([2, 65, 300], 2, 32, True, True),
    ([5, 64, 257], 1, 128, False, True),
    ([1, 31, 32, 33, 63, 64, 65, 700], 1, 64, False, True),
    ([2, 66, 130, 400], 2, 128, True, True),
    # 32 rows: run as one 64-row group with 32 padding rows
    ([1, 63, 64, 65, 200, 1000], 2, 16, True, True),
    ([3, 64, 190, 513], 1, 32, False, True),
    # four query tokens per request (multi-token prediction drafts)
    ([3, 4, 5, 64, 131, 700], 4, 16, True, False),
    ([3, 4, 5, 64, 131, 700], 4, 32, False, False),
    ([4, 70, 300], 4, 128, True, False),
    ([4, 70, 300], 4, 64, True, True),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,causal,fp8", SHAPES)
def test_shapes_with_poisoned_tails_match_oracle(seqlens, s_q, h_q, causal, fp8):
    case = W.make_case(seqlens, s_q, h_q, seed=100 + h_q + s_q, causal=causal, fp8=fp8,
                       spare_pages=3, poison=True)
    out, lse = run_gpu(case)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, f"{seqlens} s_q={s_q} h_q={h_q} causal={causal} fp8={fp8}")


GROWING = [
    # seqlens, s_q, h_q, causal, num_parts, fp8: RoPE keys scaled up along the
    # sequence, so each row's running max keeps rising (the 16-row kernel
    # rescales, the 64-row kernels restart segments)
    ([300, 1000, 2100], 1, 128, False, 8, False),
    ([1000, 3000], 2, 64, True, 4, False),
    ([1000, 3000], 1, 64, False, 4, False),
    ([300, 1000, 2100], 2, 128, True, 8, False),
    ([300, 1000, 2100], 2, 16, True, 8, False),
    ([300, 1000, 2100], 1, 128, False, 64, False),
    ([300, 1000, 2100], 1, 128, False, 8, True),
    ([1000, 3000], 2, 32, True, 4, True),
    ([300, 1000, 2100], 4, 64, True, 8, False),
    # 16 rows: the 16-row kernel's lazy rescale
    ([300, 1000, 2100], 1, 16, False, 8, False),
    ([300, 1000, 2100], 1, 16, False, 8, True),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,causal,num_parts,fp8", GROWING)
def test_growing_scores_match_oracle(seqlens, s_q, h_q, causal, num_parts, fp8):
    case = W.make_case(seqlens, s_q, h_q, seed=12 + h_q, causal=causal, fp8=fp8, spare_pages=1,
                       poison=True, rope_ramp=0.05)
    out, lse = run_gpu(case, num_parts=num_parts)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse,
            f"growing {seqlens} s_q={s_q} h_q={h_q} parts={num_parts} fp8={fp8}")


WIDE = [
    # seqlens, s_q, h_q, causal, fp8: query rows scaled by their own power of
    # two and a quarter of their entries made 2^12 smaller, so scores span a
    # wide range and small query entries must keep their weight (a path that
    # rounded q to a narrow format, or accumulated the scores in lower
    # precision, would fail here)
    ([5, 64, 257, 700], 1, 128, False, True),
    ([2, 66, 130, 400], 2, 64, True, True),
    ([300, 64], 1, 16, False, True),
    ([5, 64, 257], 1, 128, False, False),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,causal,fp8", WIDE)
def test_wide_range_queries_match_oracle(seqlens, s_q, h_q, causal, fp8):
    case = W.make_case(seqlens, s_q, h_q, seed=40 + h_q, causal=causal, fp8=fp8, spare_pages=1,
                       poison=True)
    rng = np.random.default_rng(41 + h_q)
    rows = (case.q.astype(np.uint32) << 16).view(np.float32).reshape(-1, case.q.shape[-1]).copy()
    rows *= np.exp2(rng.integers(-12, 6, size=(rows.shape[0], 1))).astype(np.float32)
    rows[rng.random(rows.shape) < 0.25] *= np.float32(2.0 ** -12)
    case.q = W.bf16_bits(rows.reshape(case.q.shape))
    out, lse = run_gpu(case)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, f"wide queries {seqlens} s_q={s_q} h_q={h_q} fp8={fp8}")


@pytest.mark.parametrize("num_parts", [1, 7, 64, 256, 1024])
def test_result_does_not_depend_on_the_split(num_parts):
    case = W.make_case([900, 33, 2000, 64], 2, 32, seed=7, causal=True, spare_pages=2, poison=True)
    out, lse = run_gpu(case, num_parts=num_parts)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, f"num_parts={num_parts}")


@pytest.mark.parametrize("num_parts", [1, 7, 64, 256])
def test_result_does_not_depend_on_the_split_256_rows(num_parts):
    case = W.make_case([900, 33, 2000, 64], 2, 128, seed=17, causal=True, spare_pages=2,
                       poison=True)
    out, lse = run_gpu(case, num_parts=num_parts)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, f"M=256 num_parts={num_parts}")


def test_empty_requests_and_empty_causal_rows():
    # L = 0 requests, and L = 1 under s_q = 2 causal (row 0 sees no key)
    case = W.make_case([0, 1, 70, 0, 1], 2, 16, seed=8, causal=True, spare_pages=1, poison=True)
    out, lse = run_gpu(case, num_parts=8)
    ref_out, ref_lse = oracle_all(case)
    assert np.isneginf(ref_lse[0]).all() and np.isneginf(ref_lse[1, 0]).all()
    compare(out, lse, ref_out, ref_lse, "empty rows")


def test_empty_requests_with_16_rows():
    case = W.make_case([0, 5, 0, 130, 0], 1, 16, seed=18, spare_pages=1, poison=True)
    out, lse = run_gpu(case, num_parts=8)
    ref_out, ref_lse = oracle_all(case)
    assert np.isneginf(ref_lse[0]).all() and np.isneginf(ref_lse[4]).all()
    compare(out, lse, ref_out, ref_lse, "empty requests, 16 rows")


def test_gpu_plan_equals_oracle_plan():
    import mla_paged_kv_fwd_amd as mla

    rng = np.random.default_rng(3)
    cases = [([37, 100], 1, 16, 8), ([4096] * 128, 1, 16, 256), ([131072] * 8, 1, 128, 256),
             ([0, 5, 0, 0, 64, 65, 0], 2, 32, 7), ([1], 1, 16, 1024), ([0, 0], 1, 16, 8),
             (list(rng.integers(0, 3000, size=16384)), 1, 16, 4096), ([64] * 1025, 1, 64, 333)]
    for _ in range(10):
        n = int(rng.integers(1, 3000))
        cases.append((list(rng.integers(0, 9000, size=n)), int(rng.choice([1, 2])),
                      int(rng.choice([16, 32, 64, 128])), int(rng.integers(1, 2000))))
    for seqlens, s_q, h_q, parts in cases:
        sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
        meta, sb, _ = mla.get_metadata(sl, s_q, h_q, parts)
        torch.cuda.synchronize()
        ref_meta, ref_sb = oracle.plan(seqlens, parts, oracle.plan_overhead(s_q, h_q))
        np.testing.assert_array_equal(meta.cpu().numpy(), np.array(ref_meta, dtype=np.int32))
        np.testing.assert_array_equal(sb.cpu().numpy(), np.array(ref_sb, dtype=np.int32))


def test_repeat_runs_are_bitwise_identical():
    case = W.make_case([700, 1500, 90], 1, 64, seed=9)
    dev = to_device(case)
    o1, l1 = run_gpu(case, dev=dev)
    o2, l2 = run_gpu(case, dev=dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_permutation_does_not_change_gpu_result():
    a = W.make_case([300, 1000], 1, 16, seed=10, permute=False)
    b = W.make_case([300, 1000], 1, 16, seed=10, permute=True, spare_pages=5)
    oa, la = run_gpu(a, num_parts=8)
    ob, lb = run_gpu(b, num_parts=8)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("name", ["membound", "computebound", "fp8", "longctx"])
def test_full_size_workloads_on_sampled_rows(name):
    case = W.make_config(name)
    print(f"{name}: batch={case.batch} pages={case.num_pages}", flush=True)
    out, lse = run_gpu(case)
    rows = sample_rows(case, 40, seed=11)
    ref_out, ref_lse, _ = oracle.decode_rows(case.q, case.cache, case.kind, case.block_table,
                                             case.seqlens, case.scale, case.causal, rows)
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    compare(out[b, i, h], lse[b, i, h], ref_out, ref_lse, name)
    # a property over every row: all outputs finite
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


ROWS128 = [
    # seqlens, s_q, h_q, causal, num_parts: 128 or more rows per request on
    # plans of a few parts (the 64-row kernel, parts that walk many requests)
    # and four row groups (M = 512)
    ([1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 95, 96, 97, 1000, 2500], 1, 128, False, 3),
    ([1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 95, 96, 97, 1000, 2500], 1, 128, False, 37),
    ([2, 17, 33, 250, 1200], 2, 64, True, 5),
    ([4, 18, 34, 251, 900], 4, 128, True, 6),
    ([4, 18, 34, 251, 900], 4, 32, False, 64),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,causal,num_parts", ROWS128)
def test_128_row_groups_match_oracle(seqlens, s_q, h_q, causal, num_parts):
    case = W.make_case(seqlens, s_q, h_q, seed=300 + h_q + s_q, causal=causal, spare_pages=2,
                       poison=True)
    out, lse = run_gpu(case, num_parts=num_parts)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse,
            f"128-row {seqlens} s_q={s_q} h_q={h_q} causal={causal} parts={num_parts}")


def _one_part_per_cu():
    import mla_paged_kv_fwd_amd as mla

    # a long context for 128 rows per request: the plan of one part per CU
    return mla.default_num_parts(1, 128, batch=1, max_seqlen=1 << 24)


ROWS128_KERNEL = [
    # seqlens (repeated), s_q, h_q, causal: 128 rows per request over a bf16
    # cache on a plan of one part per CU, which runs the 128-row kernel.
    # Lengths on both sides of its 16-token unit and 32-token step
    # boundaries, repeated so that parts walk several requests.
    ([1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 95, 96, 97, 1000, 2500], 12, 1, 128, False),
    ([2, 17, 33, 250, 1200], 40, 2, 64, True),
    ([4, 18, 34, 251, 900], 30, 4, 32, False),
]


@pytest.mark.parametrize("seqlens,reps,s_q,h_q,causal", ROWS128_KERNEL)
def test_128_row_kernel_matches_oracle(seqlens, reps, s_q, h_q, causal):
    parts = _one_part_per_cu()
    case = W.make_case(seqlens * reps, s_q, h_q, seed=350 + h_q + s_q, causal=causal, spare_pages=2,
                       poison=True)
    print(f"128-row kernel: {len(case.seqlens)} requests s_q={s_q} h_q={h_q} parts={parts}", flush=True)
    out, lse = run_gpu(case, num_parts=parts)
    ref_out, ref_lse = oracle_all(case)
    compare(out, lse, ref_out, ref_lse, f"128-row kernel {len(case.seqlens)} requests s_q={s_q} h_q={h_q}")


def test_plan_size_follows_the_context_length():
    import mla_paged_kv_fwd_amd as mla

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    one_per_cu = (cus + 7) // 8 * 8
    assert _one_part_per_cu() == one_per_cu
    short = mla.default_num_parts(1, 128)  # the 64-row kernel's plan: two work-groups per part
    assert short == max(8, (cus // 2 + 7) // 8 * 8)
    pages_needed = 48 * one_per_cu
    assert mla.default_num_parts(1, 128, batch=pages_needed, max_seqlen=64) == one_per_cu
    assert mla.default_num_parts(1, 128, batch=pages_needed - 1, max_seqlen=64) == short
    # other shapes and the FP8 cache keep the one-round size of their kernel
    assert mla.default_num_parts(2, 128, batch=64, max_seqlen=1 << 20) == mla.default_num_parts(2, 128)
    assert mla.default_num_parts(1, 128, fp8=True, batch=64, max_seqlen=1 << 20) == \
        mla.default_num_parts(1, 128, fp8=True)
