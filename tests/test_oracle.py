"""Pins for the CPU oracle: library routines, closed forms and invariants.

Each test is chosen so that a plausible slip in the oracle (a dropped RoPE
term, a wrong page/slot index, a transposed operand, a wrong log base, a
misplaced scale, a causal off-by-one) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    facts = {}
    with open(os.path.join(GOLDEN, "format_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                facts[k.strip()] = int(v)
    return facts


def _contiguous_keys(case, b):
    """Keys of request b for a case built with permute=False (pages stored in order)."""
    pages = [(int(L) + 63) // 64 for L in case.seqlens]
    start = sum(pages[:b])
    if case.kind == 0:
        rows = case.cache[start:start + pages[b]].reshape(-1, W.D_QK)[: case.seqlens[b]]
        return W.bf16_to_f32(rows).astype(np.float64)
    recs = case.cache[start:start + pages[b]].reshape(-1, W.FP8_RECORD)[: case.seqlens[b]]
    return np.stack([oracle.fp8_record_values(r) for r in recs]) if len(recs) else np.zeros((0, 576))


def _sdpa(qrows, keys, scale):
    """torch scaled_dot_product_attention + logsumexp in fp64 (library routines)."""
    q = torch.from_numpy(qrows)[None]            # [1, n, 576]
    k = torch.from_numpy(keys)[None]             # [1, L, 576]
    v = torch.from_numpy(np.ascontiguousarray(keys[:, :512]))[None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0].numpy()
    lse = torch.logsumexp(scale * (q[0] @ k[0].T), dim=-1).numpy()
    return out, lse


def _q_rows(case, b, i):
    return W.bf16_to_f32(case.q[b, i]).astype(np.float64)  # [h_q, 576]


def test_format_sizes_match_pages():
    f = _facts()
    assert oracle.fp8_record_bytes() == f["fp8_bytes_per_token"] == W.FP8_RECORD
    assert oracle.bf16_token_bytes() == f["bf16_bytes_per_token"] == 2 * W.D_QK
    assert f["page_tokens"] == f["page_tokens_fr"] == oracle.PAGE == W.PAGE
    # 512 e4m3 codes + 4 fp32 scales + 64 bf16 RoPE dims
    assert 512 + 4 * 4 + 64 * 2 == f["fp8_bytes_per_token"]


@pytest.mark.parametrize("seqlens,s_q,h_q", [
    ([37, 100], 1, 16),
    ([1, 2, 63, 64, 65, 127, 128, 200], 1, 4),
    ([5, 64, 129], 2, 3),
])
def test_noncausal_matches_torch_sdpa(seqlens, s_q, h_q):
    case = W.make_case(seqlens, s_q, h_q, seed=11, permute=False)
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    for b in range(case.batch):
        keys = _contiguous_keys(case, b)
        for i in range(s_q):
            ro, rl = _sdpa(_q_rows(case, b, i), keys, case.scale)
            np.testing.assert_allclose(out[b, i], ro, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], rl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s_q", [2, 4])
def test_causal_rows_see_bottom_right_prefix(s_q):
    # Query row i of s_q sees keys [0, L - (s_q - 1 - i)); with s_q = 4 and
    # L = 3 the oldest row sees nothing
    seqlens, h_q = [3, 64, 65, 130], 4
    case = W.make_case(seqlens, s_q, h_q, seed=12, permute=False, causal=True)
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, True)
    for b in range(case.batch):
        keys = _contiguous_keys(case, b)
        for i in range(s_q):
            n = seqlens[b] - (s_q - 1 - i)
            if n <= 0:
                assert np.all(out[b, i] == 0) and np.all(np.isneginf(lse[b, i]))
                continue
            ro, rl = _sdpa(_q_rows(case, b, i), keys[:n], case.scale)
            np.testing.assert_allclose(out[b, i], ro, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], rl, rtol=1e-12, atol=1e-12)
    # the newest row equals the non-causal result
    out_nc, lse_nc = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    np.testing.assert_array_equal(out[:, s_q - 1], out_nc[:, s_q - 1])
    np.testing.assert_array_equal(lse[:, s_q - 1], lse_nc[:, s_q - 1])


def test_single_token_returns_its_value():
    case = W.make_case([1, 1], 1, 8, seed=13)
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    for b in range(2):
        k0 = W.bf16_to_f32(case.cache[case.block_table[b, 0], 0]).astype(np.float64)
        np.testing.assert_array_equal(out[b, 0], np.broadcast_to(k0[:512], (8, 512)))
        ref = case.scale * torch.from_numpy(_q_rows(case, b, 0)) @ torch.from_numpy(k0)
        np.testing.assert_allclose(lse[b, 0], ref.numpy(), rtol=1e-13, atol=1e-13)


def test_uniform_scores_give_mean_and_log_n():
    seqlens = [1, 7, 64, 65, 300]
    case = W.make_case(seqlens, 1, 2, seed=14, permute=False)
    case.q[:] = 0  # every score is 0
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    for b, L in enumerate(seqlens):
        keys = _contiguous_keys(case, b)
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(keys[:, :512].mean(0), (2, 512)),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b, 0], math.log(L), rtol=0, atol=1e-14)


def test_page_permutation_is_invisible():
    seqlens = [37, 100, 130]
    a = W.make_case(seqlens, 1, 4, seed=15, permute=False)
    b = W.make_case(seqlens, 1, 4, seed=15, permute=True, spare_pages=3)
    assert not np.array_equal(a.block_table, b.block_table)
    oa, la = oracle.decode(a.q, a.cache, 0, a.block_table, a.seqlens, a.scale, False)
    ob, lb = oracle.decode(b.q, b.cache, 0, b.block_table, b.seqlens, b.scale, False)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_poisoned_tails_and_spare_pages_are_never_read():
    seqlens = [37, 100, 1]
    clean = W.make_case(seqlens, 2, 4, seed=16, spare_pages=2, causal=True)
    dirty = W.make_case(seqlens, 2, 4, seed=16, spare_pages=2, causal=True, poison=True)
    oc, lc = oracle.decode(clean.q, clean.cache, 0, clean.block_table, clean.seqlens, clean.scale, True)
    od, ld = oracle.decode(dirty.q, dirty.cache, 0, dirty.block_table, dirty.seqlens, dirty.scale, True)
    np.testing.assert_array_equal(oc, od)
    np.testing.assert_array_equal(lc, ld)
    # a length-1 request under s_q=2 causal leaves row 0 empty: out 0, lse -inf
    assert np.all(od[2, 0] == 0) and np.all(np.isneginf(ld[2, 0]))


@pytest.mark.parametrize("cut", [1, 63, 64, 65, 199])
def test_split_then_lse_merge_equals_whole(cut):
    case = W.make_case([200], 1, 3, seed=17)
    rows = oracle.all_rows(1, 1, 3)
    whole_o, whole_l, _ = oracle.decode_rows(case.q, case.cache, 0, case.block_table, case.seqlens,
                                             case.scale, False, rows)
    for r in range(3):
        parts = []
        for lo, hi in [(0, cut), (cut, 200)]:
            o, l, _ = oracle.decode_rows(case.q, case.cache, 0, case.block_table, case.seqlens,
                                         case.scale, False, rows[r:r + 1], windows=[[lo, hi]])
            parts.append((o[0], l[0]))
        mo, ml = oracle.lse_merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
        np.testing.assert_allclose(mo, whole_o[r], rtol=1e-12, atol=1e-14)
        assert abs(ml - whole_l[r]) < 1e-12


def test_lse_merge_ignores_empty_parts():
    o = np.array([[1.0, 2.0], [5.0, 6.0]])
    mo, ml = oracle.lse_merge(o, np.array([0.5, -np.inf]))
    np.testing.assert_array_equal(mo, [1.0, 2.0])
    assert ml == 0.5
    mo, ml = oracle.lse_merge(o, np.array([-np.inf, -np.inf]))
    assert np.all(mo == 0) and ml == -np.inf


def test_head_permutation_permutes_outputs():
    case = W.make_case([70, 9], 1, 6, seed=18)
    perm = np.array([3, 0, 5, 1, 4, 2])
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    qp = np.ascontiguousarray(case.q[:, :, perm])
    outp, lsep = oracle.decode(qp, case.cache, 0, case.block_table, case.seqlens, case.scale, False)
    np.testing.assert_array_equal(outp, out[:, :, perm])
    np.testing.assert_array_equal(lsep, lse[:, :, perm])


def test_duplicated_tokens_add_log_k():
    base = W.make_case([50], 1, 4, seed=19, permute=False)
    keys = base.cache.reshape(-1, W.D_QK)[:50]
    k = 3
    dup = W.make_case([150], 1, 4, seed=19, permute=False)
    dup.q[:] = base.q
    dup.cache.reshape(-1, W.D_QK)[:150] = np.repeat(keys, k, axis=0)
    o1, l1 = oracle.decode(base.q, base.cache, 0, base.block_table, base.seqlens, base.scale, False)
    o2, l2 = oracle.decode(dup.q, dup.cache, 0, dup.block_table, dup.seqlens, dup.scale, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + math.log(k), rtol=0, atol=1e-12)


def test_hard_attention_limit_picks_argmax_value():
    case = W.make_case([90], 1, 4, seed=20, permute=False)
    keys = _contiguous_keys(case, 0)
    q = _q_rows(case, 0, 0)
    out, _ = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, 1000.0, False)
    best = np.argmax(q @ keys.T, axis=1)
    np.testing.assert_allclose(out[0, 0], keys[best, :512], atol=1e-6)


def test_large_scores_stay_finite_and_match_sdpa():
    case = W.make_case([130], 1, 4, seed=21, permute=False)
    out, lse = oracle.decode(case.q, case.cache, 0, case.block_table, case.seqlens, 10 * case.scale, False)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    ro, rl = _sdpa(_q_rows(case, 0, 0), _contiguous_keys(case, 0), 10 * case.scale)
    np.testing.assert_allclose(out[0, 0], ro, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(lse[0, 0], rl, rtol=1e-12)


def test_fp8_cache_matches_sdpa_on_dequantised_keys():
    case = W.make_case([37, 100], 1, 8, seed=22, permute=False, fp8=True)
    out, lse = oracle.decode(case.q, case.cache, 1, case.block_table, case.seqlens, case.scale, False)
    for b in range(2):
        ro, rl = _sdpa(_q_rows(case, b, 0), _contiguous_keys(case, b), case.scale)
        np.testing.assert_allclose(out[b, 0], ro, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[b, 0], rl, rtol=1e-12)


def test_fp8_cache_is_close_to_bf16_cache():
    # Same latent values, two cache formats: within e4m3's rounding of the keys.
    bf = W.make_case([256], 1, 8, seed=23, permute=False)
    f8 = W.make_case([256], 1, 8, seed=23, permute=False, fp8=True)
    ob, lb = oracle.decode(bf.q, bf.cache, 0, bf.block_table, bf.seqlens, bf.scale, False)
    of, lf = oracle.decode(f8.q, f8.cache, 1, f8.block_table, f8.seqlens, f8.scale, False)
    assert np.max(np.abs(ob - of)) < 0.05
    assert np.max(np.abs(lb - lf)) < 0.05
    assert np.max(np.abs(ob - of)) > 0  # the FP8 path really dequantises
