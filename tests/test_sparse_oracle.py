"""Pins of the oracle's sparse decode (rows attend to listed tokens only)
against the dense decode it must reduce to, torch's scaled_dot_product_attention
on the gathered keys (a library routine), and closed forms."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_oracle import _contiguous_keys, _q_rows, _sdpa


def _lists(seqlens, s_q, topk, rng, dup=False):
    """Random lists of random lengths, padded with -1 (and some junk after
    the first -1, which must be ignored)."""
    idx = np.full((len(seqlens), s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        for i in range(s_q):
            if L == 0:
                continue
            pick = rng.integers(0, L, topk) if dup else rng.choice(L, size=min(topk, L), replace=False)
            n = int(rng.integers(0, len(pick) + 1))
            idx[b, i, :n] = pick[:n]
            if n + 1 < topk:
                idx[b, i, n + 1:] = pick[n + 1:topk] if len(pick) >= topk else -1
    return idx


def _listed(lst):
    """The entries before the first negative one."""
    neg = np.nonzero(lst < 0)[0]
    return lst[: neg[0]] if len(neg) else lst


def test_full_lists_equal_the_dense_decode():
    seqlens = [1, 64, 130, 300]
    case = W.make_case(seqlens, 2, 8, seed=50)
    topk = max(seqlens)
    idx = np.full((len(seqlens), 2, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        idx[b, :, :L] = np.arange(L)
    out, lse = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, idx, case.scale)
    ref, ref_lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


def test_causal_prefix_lists_equal_the_causal_decode():
    seqlens, s_q = [4, 65, 200], 4
    case = W.make_case(seqlens, s_q, 4, seed=51, causal=True)
    topk = max(seqlens)
    idx = np.full((len(seqlens), s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        for i in range(s_q):
            n = max(0, L - (s_q - 1 - i))
            idx[b, i, :n] = np.arange(n)
    out, lse = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, idx, case.scale)
    ref, ref_lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, True)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("fp8", [False, True])
def test_random_lists_match_sdpa_on_the_gathered_keys(fp8):
    rng = np.random.default_rng(52)
    seqlens, s_q, h_q, topk = [70, 300, 129], 2, 4, 96
    case = W.make_case(seqlens, s_q, h_q, seed=53, fp8=fp8, permute=False)
    idx = _lists(seqlens, s_q, topk, rng, dup=True)  # duplicates count twice
    out, lse = oracle.decode_sparse(case.q, case.cache, case.kind, case.block_table, idx, case.scale)
    for b in range(len(seqlens)):
        keys = _contiguous_keys(case, b)
        for i in range(s_q):
            sel = _listed(idx[b, i])
            if len(sel) == 0:
                assert np.all(out[b, i] == 0) and np.all(np.isneginf(lse[b, i]))
                continue
            ro, rl = _sdpa(_q_rows(case, b, i), keys[sel], case.scale)
            np.testing.assert_allclose(out[b, i], ro, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], rl, rtol=1e-12, atol=1e-12)


def test_order_of_a_list_does_not_matter():
    rng = np.random.default_rng(54)
    case = W.make_case([500, 90], 1, 8, seed=55)
    idx = np.stack([rng.choice(L, 80, replace=False) for L in (500, 90)]).astype(np.int32)[:, None]
    out, lse = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, idx, case.scale)
    perm = idx[:, :, rng.permutation(80)]
    out2, lse2 = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, perm, case.scale)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-13)


def test_empty_and_single_entry_lists():
    case = W.make_case([40, 40], 1, 4, seed=56)
    idx = np.full((2, 1, 16), -1, dtype=np.int32)
    idx[0, 0, 3] = 5                       # after the first -1: not listed
    idx[1, 0, 0] = 33                      # one listed token
    idx[1, 0, 5] = 7                       # after the first -1: not listed
    out, lse = oracle.decode_sparse(case.q, case.cache, 0, case.block_table, idx, case.scale)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    k = W.bf16_to_f32(case.cache[case.block_table[1, 0], 33]).astype(np.float64)
    np.testing.assert_array_equal(out[1, 0], np.broadcast_to(k[:512], (4, 512)))
    np.testing.assert_allclose(lse[1, 0], case.scale * (_q_rows(case, 1, 0) @ k), rtol=1e-13)
