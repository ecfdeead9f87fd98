"""Device-side input checks (mla_check_block_table, mla_check_sparse_indices)
on good inputs and on inputs with planted faults; with MLA_CHECK=1 the
binding refuses to launch a decode, sparse decode or cache write on bad
inputs.  The checks read only entries inside the table, so feeding them bad
data is safe; no decode kernel ever sees the bad inputs here."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _inputs():
    seqlens = np.array([100, 0, 700, 64, 3000, 1], dtype=np.int32)
    q, kc, bt, sl = W.make_device_inputs(seqlens, 1, 16, False, 140)
    return q, kc, bt, sl


def test_block_table_check_passes_good_inputs_and_locates_faults():
    import mla_paged_kv_fwd_amd as mla

    q, kc, bt, sl = _inputs()
    pages = kc.shape[0]
    assert mla.check_block_table(bt, sl, pages) == (0, None)
    # unused entries past a request's pages are -1 already and must not count
    assert (bt[0, 2:] == -1).all()
    bad = bt.clone()
    bad[4, 17] = pages          # outside the pool
    bad[2, 3] = -1              # a hole inside request 2's pages
    bad[2, 9] = pages + 5
    assert mla.check_block_table(bad, sl, pages) == (2, (2, 3))
    sl_bad = sl.clone()
    sl_bad[0] = 64 * bt.shape[1] + 1   # needs one page more than the table holds
    assert mla.check_block_table(bt, sl_bad, pages) == (1, (0, None))
    sl_bad[5] = -3
    assert mla.check_block_table(bt, sl_bad, pages) == (2, (0, None))


def test_sparse_check_covers_entries_before_the_list_end_only():
    import mla_paged_kv_fwd_amd as mla

    q, kc, bt, sl = _inputs()
    pages = kc.shape[0]
    rng = np.random.default_rng(141)
    idx = np.full((6, 2, 50), -1, dtype=np.int32)
    for b, L in enumerate([100, 0, 700, 64, 3000, 1]):
        for i in range(2):
            if L:
                n = min(L, 50)
                idx[b, i, :n] = rng.choice(L, n, replace=False)
    idx[1, 0, 5] = 10 ** 9      # after the list's end (request 1's lists are empty): ignored
    good = torch.from_numpy(idx).cuda()
    assert mla.check_sparse_indices(bt, good, pages) == (0, None)
    idx[3, 1, 7] = 64 * bt.shape[1]    # page past the table's width
    idx[0, 0, 40] = 64 * 3             # page 3 of request 0: a -1 entry
    assert mla.check_sparse_indices(bt, torch.from_numpy(idx).cuda(), pages) == (2, (0, 40))


def test_checked_calls_refuse_bad_inputs(monkeypatch):
    import mla_paged_kv_fwd_amd as mla

    q, kc, bt, sl = _inputs()
    # the calls see a pool one page short; the planted page is that last page,
    # outside the pool they are given but still real memory
    short = kc[:-1]
    bad = bt.clone()
    bad[4, 2] = short.shape[0]
    monkeypatch.setenv("MLA_CHECK", "1")
    with pytest.raises(mla.MlaError, match="block table"):
        mla.decode(q, short, bad, sl, 576 ** -0.5, False)
    k_new = torch.zeros((6, 1, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError, match="block table"):
        mla.kv_cache_write(k_new, bad, sl, short)
    idx = torch.full((6, 1, 8), -1, dtype=torch.int32, device="cuda")
    idx[4, 0, 0] = 64 * 2
    with pytest.raises(mla.MlaError, match="sparse lists"):
        mla.decode_sparse(q, short, bad, idx, 576 ** -0.5)
    # the same calls on good inputs run, checked
    out, lse = mla.decode(q, kc, bt, sl, 576 ** -0.5, False)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
