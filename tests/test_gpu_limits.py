"""GPU parity at the interface's limits: the largest batch (16384 requests,
short ragged lengths with empty ones, so every part walks many request
segments) and the largest num_parts (16384, far more parts than pages), on
rows sampled for the oracle plus an all-finite property over every row."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu

MAX_BATCH = 16384
MAX_PARTS = 16384


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _host(q, kc, bt, sl):
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    cache = kc.cpu().numpy() if kc.dtype == torch.uint8 else \
        kc.view(torch.int16).cpu().numpy().view(np.uint16)
    return qh, cache, bt.cpu().numpy(), sl.cpu().numpy()


def _check_sampled(out, lse, q, kc, bt, sl, s_q, h_q, fp8, causal, scale, rng, label, n=48):
    qh, cache, bth, slh = _host(q, kc, bt, sl)
    nonempty = np.flatnonzero(slh > 0)
    b = np.concatenate([rng.choice(nonempty, n - 4), rng.choice(np.flatnonzero(slh == 0), 4)])
    rows = np.stack([b, rng.integers(0, s_q, n), rng.integers(0, h_q, n)], 1)
    ref, ref_lse, _ = oracle.decode_rows(qh, cache, 1 if fp8 else 0, bth, slh, scale, causal, rows)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    compare(o[rows[:, 0], rows[:, 1], rows[:, 2]], l[rows[:, 0], rows[:, 1], rows[:, 2]], ref,
            ref_lse, label)
    assert np.all(np.isfinite(o))
    # row i of request b sees L_b - (s_q - 1 - i) keys when causal, else L_b
    vis = slh[:, None] - ((s_q - 1 - np.arange(s_q))[None, :] if causal else 0) > 0
    assert np.all(np.isfinite(l[vis])) and np.all(np.isneginf(l[~vis]))


@pytest.mark.parametrize("s_q,h_q,fp8,causal", [(1, 16, False, False), (2, 64, True, True)])
def test_largest_batch(s_q, h_q, fp8, causal):
    import mla_paged_kv_fwd_amd as mla

    rng = np.random.default_rng(120 + h_q)
    seqlens = rng.integers(1, 200, MAX_BATCH).astype(np.int32)
    seqlens[rng.choice(MAX_BATCH, 300, replace=False)] = 0
    print(f"largest batch: {MAX_BATCH} requests s_q={s_q} h_q={h_q} fp8={fp8}", flush=True)
    q, kc, bt, sl = W.make_device_inputs(seqlens, s_q, h_q, fp8, 121)
    scale = 576 ** -0.5
    out, lse = mla.decode(q, kc, bt, sl, scale, causal, fp8=fp8)
    torch.cuda.synchronize()
    _check_sampled(out, lse, q, kc, bt, sl, s_q, h_q, fp8, causal, scale, rng,
                   f"batch {MAX_BATCH} h_q={h_q}")


@pytest.mark.parametrize("h_q,fp8", [(16, True), (128, False)])
def test_largest_num_parts(h_q, fp8):
    import mla_paged_kv_fwd_amd as mla

    rng = np.random.default_rng(130 + h_q)
    seqlens = np.array([0, 3000, 1, 640, 0, 2049, 77], dtype=np.int32)
    print(f"num_parts {MAX_PARTS}: seqlens {seqlens.tolist()} h_q={h_q} fp8={fp8}", flush=True)
    q, kc, bt, sl = W.make_device_inputs(seqlens, 1, h_q, fp8, 131)
    scale = 576 ** -0.5
    out, lse = mla.decode(q, kc, bt, sl, scale, False, num_parts=MAX_PARTS, fp8=fp8)
    torch.cuda.synchronize()
    _check_sampled(out, lse, q, kc, bt, sl, 1, h_q, fp8, False, scale, rng,
                   f"num_parts {MAX_PARTS} h_q={h_q}", n=24)
