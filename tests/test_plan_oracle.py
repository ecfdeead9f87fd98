"""Pins for the split-KV plan definition: coverage, contiguity, balance."""
import numpy as np
import pytest

import oracle


def _walk(meta, seqlens):
    """Expand each part's range into its (b, j) pages."""
    pages = [(L + 63) // 64 for L in seqlens]
    out = []
    for m in meta:
        got = []
        if m[0] >= 0:
            b, j = m[0], m[1]
            while True:
                if pages[b] == 0:
                    b, j = b + 1, 0
                    continue
                got.append((b, j))
                if (b, j) == (m[2], m[3]):
                    break
                j += 1
                if j == pages[b]:
                    b, j = b + 1, 0
        out.append(got)
    return out


CASES = [
    ([37, 100], 4, 1),
    ([4096] * 16, 256, 1),
    ([0, 5, 0, 0, 64, 65, 0], 7, 2),
    ([1], 1024, 3),
    ([131072] * 2, 256, 3),
    ([0, 0], 8, 1),
    ([7] * 300, 16, 5),
    (list(np.random.default_rng(0).integers(0, 9000, 50)), 97, 3),
]


@pytest.mark.parametrize("seqlens,parts,c", CASES)
def test_plan_covers_every_page_once_in_order(seqlens, parts, c):
    meta, split_base = oracle.plan(seqlens, parts, c)
    assert len(meta) == parts and len(split_base) == len(seqlens) + 1
    flat = [pg for got in _walk(meta, seqlens) for pg in got]
    expect = [(b, j) for b, L in enumerate(seqlens) for j in range((L + 63) // 64)]
    assert flat == expect


@pytest.mark.parametrize("seqlens,parts,c", CASES)
def test_plan_is_balanced_and_split_slots_consistent(seqlens, parts, c):
    meta, split_base = oracle.plan(seqlens, parts, c)
    walked = _walk(meta, seqlens)
    pages = [(L + 63) // 64 for L in seqlens]
    total = sum(c + n for n in pages if n > 0)
    if total == 0:
        assert all(m[0] == -1 for m in meta) and split_base[-1] == 0
        return
    P = min(parts, total)
    touching = {b: [] for b in range(len(seqlens))}
    for p, got in enumerate(walked):
        reqs = sorted({b for b, _ in got})
        for b in reqs:
            touching[b].append(p)
        cost = len(got) + c * len(reqs)
        # each part gets its share of the cost line, plus at most one uncharged overhead
        assert cost <= -(-total // P) + c, (p, cost)
        if p >= P:
            assert not got
    for b in range(len(seqlens)):
        ps = touching[b]
        assert split_base[b + 1] - split_base[b] == len(ps)
        assert ps == list(range(ps[0], ps[0] + len(ps))) if ps else pages[b] == 0
    for p, m in enumerate(meta):
        if m[0] >= 0:
            assert m[4] == touching[m[0]].index(p)
