"""The FP8 cache format's own error across shapes, on the GPU and on the
oracle side by side.

The same N(0,1) latent rows (rounded to bf16) are written once as bf16 rows
and once as 656-byte FP8 records by the oracle's cache writer, and decoded
from both caches with the same queries.  For every shape the test checks:

- each GPU decode against the oracle on sampled rows (the usual parity bar);
- that the GPU's FP8-minus-bf16 shift equals the oracle's own shift on the
  same rows within the sum of the two parity bars, i.e. the GPU path adds no
  error of its own on top of what the format costs;
- that the shift is a real quantisation effect: above zero and below the
  E4M3 step (3 mantissa bits: a value moves by at most 2^-4 of itself).

Shapes: h_q in {16, 64, 128} x L in {4096, 16384, 65536}, s_q = 1, two
requests.  The format is the one the pages describe (FlashMLA FP8 cache,
"Key Contributions": 656 bytes per token against 1152 in bf16, the RoPE
slice kept in bf16)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare

pytestmark = pytest.mark.gpu

SHAPES = [(h_q, L) for h_q in (16, 64, 128) for L in (4096, 16384, 65536)]
MAX_ABS, REL_L2 = 2e-2, 1e-2  # the parity bar of each side


def _caches(batch, length, h_q, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    pages_per = length // W.PAGE
    pages = batch * pages_per
    bt = rng.permutation(pages).astype(np.int32).reshape(batch, pages_per)
    sl = np.full((batch,), length, dtype=np.int32)
    rows = W.bf16_bits(rng.standard_normal((batch, length, W.D_QK), dtype=np.float32))
    q = W.bf16_bits(rng.standard_normal((batch, 1, h_q, W.D_QK), dtype=np.float32))
    c16 = oracle.kv_write(rows, bt, sl, np.zeros((pages, W.PAGE, W.D_QK), dtype=np.uint16), 0)
    c8 = oracle.kv_write(rows, bt, sl, np.zeros((pages, W.PAGE, W.FP8_RECORD), dtype=np.uint8), 1)
    return q, c16, c8, bt, sl


@pytest.mark.parametrize("h_q,length", SHAPES)
def test_fp8_shift_matches_the_oracle_shift(h_q, length):
    import mla_paged_kv_fwd_amd as mla

    batch = 2
    q, c16, c8, bt, sl = _caches(batch, length, h_q, seed=1000 * h_q + length // 1024)
    scale = 1.0 / math.sqrt(W.D_QK)
    print(f"h_q={h_q} L={length}", flush=True)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(sl).cuda()
    k16 = torch.from_numpy(c16.view(np.int16)).view(torch.bfloat16).cuda()
    k8 = torch.from_numpy(c8).cuda()
    o16, l16 = mla.decode(qd, k16, btd, sld, scale, False)
    o8, l8 = mla.decode(qd, k8, btd, sld, scale, False, fp8=True)
    torch.cuda.synchronize()
    o16, l16 = o16.float().cpu().numpy(), l16.cpu().numpy()
    o8, l8 = o8.float().cpu().numpy(), l8.cpu().numpy()
    del k16, k8

    rng = np.random.default_rng(h_q + length)
    n = 24
    rows = np.stack([rng.integers(0, batch, n), np.zeros(n, dtype=np.int64), rng.integers(0, h_q, n)],
                    axis=1).astype(np.int32)
    r16, rl16, _ = oracle.decode_rows(q, c16, 0, bt, sl, scale, False, rows)
    r8, rl8, _ = oracle.decode_rows(q, c8, 1, bt, sl, scale, False, rows)
    b, i, h = rows[:, 0], rows[:, 1], rows[:, 2]
    compare(o16[b, i, h], l16[b, i, h], r16, rl16, f"bf16 h_q={h_q} L={length}")
    compare(o8[b, i, h], l8[b, i, h], r8, rl8, f"fp8 h_q={h_q} L={length}")

    gpu_shift = o8[b, i, h].astype(np.float64) - o16[b, i, h]
    ref_shift = r8 - r16
    ref_norm = np.linalg.norm(r16)
    gap = gpu_shift - ref_shift
    shift_rel = np.linalg.norm(ref_shift) / ref_norm
    lse_shift = np.abs(rl8 - rl16)
    print(f"h_q={h_q} L={length}: oracle shift rel_l2={shift_rel:.3e} max_abs={np.abs(ref_shift).max():.3e} "
          f"lse max={lse_shift.max():.3e}; gpu-oracle shift gap max_abs={np.abs(gap).max():.3e} "
          f"rel_l2={np.linalg.norm(gap) / ref_norm:.3e}; gpu lse shift max="
          f"{np.abs(l8[b, i, h] - l16[b, i, h]).max():.3e}", flush=True)
    assert np.abs(gap).max() <= 2 * MAX_ABS
    assert np.linalg.norm(gap) / ref_norm <= 2 * REL_L2
    assert 1e-4 < shift_rel < 2 ** -4
    assert lse_shift.max() < 0.05
