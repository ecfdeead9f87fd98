"""GPU parity of the cache writer (through the C ABI) against the oracle's
writer: byte-exact cache contents, every other slot untouched; then decode
over the written cache against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare, run_gpu
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _rows(rng, batch, n_new):
    """bf16 rows with per-tile magnitudes from 2^-24 to 2^12, tiles near
    2^-70 (below the writer's fast-division range), zero tiles, signed zeros
    and values that land on E4M3 subnormals after scaling."""
    x = rng.normal(0, 1, (batch, n_new, 576)).astype(np.float32)
    tiles = x[..., :512].reshape(batch, n_new, 4, 128)
    tiles *= np.exp2(rng.integers(-24, 13, size=(batch, n_new, 4, 1))).astype(np.float32)
    tiles[rng.random(tiles.shape[:3]) < 0.05] *= np.float32(2.0 ** -70)
    small = rng.random(tiles.shape) < 0.05
    tiles[small] *= np.float32(2.0 ** -14)          # subnormal codes
    tiles[rng.random(tiles.shape[:3]) < 0.05] = 0.0  # whole zero tiles
    x[..., :512] = tiles.reshape(batch, n_new, 512)
    x[rng.random(x.shape) < 0.01] = -0.0
    return W.bf16_bits(x)


def _setup(seqlens, n_new, kind, seed):
    rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    pages = (seqlens.astype(np.int64) + 63) // 64
    n_pages = int(pages.sum()) + 3
    width = max(1, int(pages.max()))
    bt = np.full((len(seqlens), width), -1, dtype=np.int32)
    perm = rng.permutation(n_pages).astype(np.int32)
    k = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[k:k + n]
        k += n
    shape = (n_pages, 64, 576) if kind == 0 else (n_pages, 64, 656)
    dtype = np.uint16 if kind == 0 else np.uint8
    cache = rng.integers(0, 1 << (16 if kind == 0 else 8), size=shape).astype(dtype)
    k_new = _rows(rng, len(seqlens), n_new)
    return k_new, bt, seqlens, cache


def _gpu_write(k_new, bt, seqlens, cache, kind):
    import mla_paged_kv_fwd_amd as mla

    kn = torch.from_numpy(k_new.view(np.int16)).view(torch.bfloat16).cuda()
    kc = torch.from_numpy(cache.view(np.int16) if kind == 0 else cache).cuda()
    if kind == 0:
        kc = kc.view(torch.bfloat16)
    mla.kv_cache_write(kn, torch.from_numpy(bt).cuda(), torch.from_numpy(seqlens).cuda(), kc,
                       fp8=(kind == 1))
    torch.cuda.synchronize()
    out = kc.view(torch.int16).cpu().numpy().view(np.uint16) if kind == 0 else kc.cpu().numpy()
    return out


CASES = [
    # seqlens, n_new: decode appends (n_new = s_q), a request shorter than
    # n_new, an empty request, and a right-aligned prefill
    ([1, 70, 0, 130, 64], 2),
    ([37, 100], 1),
    ([300, 5, 129, 64], 300),
    ([4096] * 4, 4096),
]


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("seqlens,n_new", CASES)
def test_writer_matches_oracle_byte_for_byte(seqlens, n_new, kind):
    print(f"kv write kind={kind} seqlens={seqlens[:6]} n_new={n_new}", flush=True)
    k_new, bt, sl, cache = _setup(seqlens, n_new, kind, seed=20 + n_new + kind)
    ref = oracle.kv_write(k_new, bt, sl, cache, kind)
    got = _gpu_write(k_new, bt, sl, cache, kind)
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{len(diff)} bytes differ; first at {diff[:5].tolist()}")


@pytest.mark.parametrize("kind", [0, 1])
def test_decode_after_writing_the_new_tokens(kind):
    # append s_q = 2 new tokens per request, then decode over the whole cache
    case = W.make_case([65, 300, 2], 2, 16, seed=31, causal=True, fp8=(kind == 1), spare_pages=1)
    rng = np.random.default_rng(32)
    k_new = W.bf16_bits(rng.normal(0, 1, (case.batch, 2, 576)).astype(np.float32))
    written = _gpu_write(k_new, case.block_table, case.seqlens, case.cache, kind)
    np.testing.assert_array_equal(
        written, oracle.kv_write(k_new, case.block_table, case.seqlens, case.cache, kind))
    case.cache = written
    out, lse = run_gpu(case)
    ref_out, ref_lse = oracle.decode(case.q, case.cache, case.kind, case.block_table, case.seqlens,
                                     case.scale, case.causal)
    compare(out, lse, ref_out, ref_lse, f"decode after write kind={kind}")
