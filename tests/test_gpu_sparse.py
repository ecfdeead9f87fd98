"""GPU parity of sparse decode (through the C ABI) against the oracle: rows
attend only to the tokens their lists name."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare, to_device
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _lists(seqlens, s_q, topk, rng, dup=False, full=False):
    """Random lists padded with -1 after a random length (junk after the
    padding starts must be ignored)."""
    idx = np.full((len(seqlens), s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        for i in range(s_q):
            if L == 0:
                continue
            pick = rng.integers(0, L, topk) if (dup or L < topk) else rng.choice(L, topk, replace=False)
            n = topk if full else int(rng.integers(0, topk + 1))
            idx[b, i, :n] = pick[:n]
            if n + 2 < topk:
                idx[b, i, n + 2] = pick[n + 2]  # junk after the -1
    return idx


def _run(case, idx, num_parts=None):
    import mla_paged_kv_fwd_amd as mla

    q, kc, bt, _ = to_device(case)
    out, lse = mla.decode_sparse(q, kc, bt, torch.from_numpy(idx).cuda(), case.scale,
                                 fp8=(case.kind == 1), num_parts=num_parts)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


CASES = [
    # seqlens, s_q, h_q, topk, fp8
    ([300, 5, 1000, 64], 1, 16, 100, False),
    ([300, 5, 1000, 64], 2, 32, 100, True),
    ([700, 2100], 1, 64, 256, False),
    ([700, 2100, 130], 2, 128, 200, False),
    ([700, 2100, 130], 1, 128, 200, True),
    ([4000, 50], 4, 64, 512, True),
    ([300, 5, 1000, 64], 4, 16, 333, True),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,topk,fp8", CASES)
def test_sparse_decode_matches_oracle(seqlens, s_q, h_q, topk, fp8):
    print(f"sparse {seqlens} s_q={s_q} h_q={h_q} topk={topk} fp8={fp8}", flush=True)
    rng = np.random.default_rng(60 + h_q + topk)
    case = W.make_case(seqlens, s_q, h_q, seed=61 + h_q, fp8=fp8, spare_pages=2, poison=True)
    idx = _lists(seqlens, s_q, topk, rng, dup=(h_q == 32))
    out, lse = _run(case, idx)
    ref, ref_lse = oracle.decode_sparse(case.q, case.cache, case.kind, case.block_table, idx,
                                        case.scale)
    compare(out, lse, ref, ref_lse, f"sparse {seqlens} h_q={h_q} topk={topk} fp8={fp8}")


@pytest.mark.parametrize("h_q,fp8", [(16, True), (64, False)])
def test_sparse_lists_longer_than_one_load_chunk(h_q, fp8):
    # the list-length scan reads 2048 entries per round trip: lists of 2600
    # entries whose first negative entry lies in the second chunk, in the
    # first chunk with junk after it in the second, or nowhere
    rng = np.random.default_rng(68 + h_q)
    seqlens, topk = [3000, 2700], 2600
    case = W.make_case(seqlens, 2, h_q, seed=69 + h_q, fp8=fp8, spare_pages=1, poison=True)
    idx = _lists(seqlens, 2, topk, rng, full=True)
    for (b, i), n in {(0, 0): 2100, (0, 1): 1500, (1, 0): 2047}.items():
        idx[b, i, n] = -1
        idx[b, i, n + 1:] = rng.integers(-5, 10**6, topk - n - 1)  # junk past the first -1
    out, lse = _run(case, idx)
    ref, ref_lse = oracle.decode_sparse(case.q, case.cache, case.kind, case.block_table, idx,
                                        case.scale)
    compare(out, lse, ref, ref_lse, f"sparse long lists h_q={h_q} fp8={fp8}")


@pytest.mark.parametrize("h_q,fp8", [(128, False), (64, True), (16, False), (32, True)])
def test_sparse_growing_scores_restart(h_q, fp8):
    # RoPE keys scaled up along the sequence and lists in ascending order, so
    # each row's running max keeps rising along its list: the 64-row kernels
    # restart segments, staging the first token ids again (h_q = 16 and 32
    # run as one padded 64-row group)
    rng = np.random.default_rng(66 + h_q)
    seqlens = [3000, 1200]
    case = W.make_case(seqlens, 2, h_q, seed=67 + h_q, fp8=fp8, spare_pages=1, poison=True,
                       rope_ramp=0.05)
    idx = np.sort(_lists(seqlens, 2, 900, rng, full=True), axis=-1)
    out, lse = _run(case, idx, num_parts=3)
    ref, ref_lse = oracle.decode_sparse(case.q, case.cache, case.kind, case.block_table, idx,
                                        case.scale)
    compare(out, lse, ref, ref_lse, f"sparse growing h_q={h_q} fp8={fp8}")


@pytest.mark.parametrize("num_parts", [1, 7, 256])
def test_sparse_result_does_not_depend_on_the_split(num_parts):
    rng = np.random.default_rng(62)
    case = W.make_case([3000, 800], 2, 64, seed=63, spare_pages=1, poison=True)
    idx = _lists([3000, 800], 2, 700, rng, full=True)
    out, lse = _run(case, idx, num_parts=num_parts)
    ref, ref_lse = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, idx, case.scale)
    compare(out, lse, ref, ref_lse, f"sparse num_parts={num_parts}")


def test_full_lists_equal_dense_decode_on_the_gpu():
    import mla_paged_kv_fwd_amd as mla

    case = W.make_case([500, 1000], 1, 128, seed=64, spare_pages=1, poison=True)
    idx = np.full((2, 1, 1000), -1, dtype=np.int32)
    idx[0, 0, :500] = np.arange(500)
    idx[1, 0, :] = np.arange(1000)
    out, lse = _run(case, idx)
    q, kc, bt, sl = to_device(case)
    dense, dense_lse = mla.decode(q, kc, bt, sl, case.scale, False)
    torch.cuda.synchronize()
    compare(out, lse, dense.float().cpu().numpy(), dense_lse.cpu().numpy(), "sparse = dense")


def test_sparse_fp8_workload_on_sampled_rows():
    # the FP8 workload's cache (64 x 16384 tokens) with 2048 listed tokens per
    # query token, h_q 128; 24 rows checked against the oracle
    import mla_paged_kv_fwd_amd as mla

    rng = np.random.default_rng(65)
    batch, L, h_q, topk = 64, 16384, 128, 2048
    q, kc, bt, sl, _, _, _, scale, _ = W.make_config_device("fp8")
    idx = np.stack([rng.choice(L, topk, replace=False) for _ in range(batch)]).astype(np.int32)[:, None]
    out, lse = mla.decode_sparse(q, kc, bt, torch.from_numpy(idx).cuda(), scale, fp8=True)
    torch.cuda.synchronize()
    rows = np.stack([rng.integers(0, batch, 24), np.zeros(24, int), rng.integers(0, h_q, 24)], 1)
    # the oracle needs host copies of the bytes the rows touch: the whole cache
    cache = kc.cpu().numpy()
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, ref_lse = oracle.decode_sparse(qh, cache, 1, bt.cpu().numpy(), idx, scale, rows=rows)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    compare(o[rows[:, 0], 0, rows[:, 2]], l[rows[:, 0], 0, rows[:, 2]], ref, ref_lse, "sparse fp8 workload")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
