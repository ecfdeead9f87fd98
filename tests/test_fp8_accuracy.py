"""The FP8 cache format's own error, on the oracle: the same bf16 latent rows
decoded from a bf16 cache and from FP8 records written by the oracle's cache
writer.  The study the benchmark repeats on the GPU at full size; here the
error is bounded from the E4M3 step size."""
import math

import numpy as np

import oracle
import workloads as W


def test_fp8_cache_moves_decode_by_about_the_e4m3_step():
    rng = np.random.default_rng(44)
    batch, length, h_q = 2, 700, 16
    case = W.make_case([length] * batch, 1, h_q, seed=45)
    rows = W.bf16_bits(rng.normal(0, 1, (batch, length, 576)).astype(np.float32))
    pages = case.num_pages
    bf16_cache = oracle.kv_write(rows, case.block_table, case.seqlens,
                                 np.zeros((pages, 64, 576), dtype=np.uint16), 0)
    fp8_cache = oracle.kv_write(rows, case.block_table, case.seqlens,
                                np.zeros((pages, 64, 656), dtype=np.uint8), 1)
    scale = 1.0 / math.sqrt(576)
    o16, l16 = oracle.decode(case.q, bf16_cache, 0, case.block_table, case.seqlens, scale, False)
    o8, l8 = oracle.decode(case.q, fp8_cache, 1, case.block_table, case.seqlens, scale, False)
    rel = np.linalg.norm(o8 - o16) / np.linalg.norm(o16)
    # E4M3 keeps 3 mantissa bits, so a latent value moves by at most 2^-4 of
    # itself.  The decode output moves by about 3% here (1.1% at the full FP8
    # workload on the GPU): the test holds it below the E4M3 step and above 0
    assert 1e-3 < rel < 2 ** -4
    # the scores move by a small fraction of their unit spread
    assert np.abs(l8 - l16).max() < 0.02
