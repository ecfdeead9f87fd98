"""The decode step (plan, attention, combine) and the sparse call captured in
a HIP graph through the C ABI.  Every replay, with eager work clobbering the
outputs and scratch buffers between replays, must equal the eager result bit
for bit; the replayed result is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import compare, oracle_all, to_device
from tests.libmla_loader import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _replay_checks(step, outs, scratch):
    """Eager step, capture, then three replays with eager work in between."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        for t in scratch:
            t.fill_(0x7F if t.dtype == torch.uint8 else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t.view(torch.uint8) if t.dtype == torch.bfloat16 else t,
                               r.view(torch.uint8) if r.dtype == torch.bfloat16 else r), \
                f"replay {i} differs from the eager result"


@pytest.mark.parametrize("h_q,fp8", [(16, False), (128, True), (64, False)])
def test_decode_step_replays_in_a_graph(h_q, fp8):
    import mla_paged_kv_fwd_amd as mla

    seqlens, s_q = [300, 1000, 2100, 64, 0], 2
    print(f"graph decode h_q={h_q} fp8={fp8}", flush=True)
    case = W.make_case(seqlens, s_q, h_q, seed=90 + h_q, causal=True, fp8=fp8, spare_pages=1,
                       poison=True)
    q, kc, bt, sl = to_device(case)
    batch = len(seqlens)
    parts = mla.default_num_parts(s_q, h_q, fp8=fp8)
    meta = torch.empty((parts, mla.META_INTS), dtype=torch.int32, device="cuda")
    sb = torch.empty((batch + 1,), dtype=torch.int32, device="cuda")
    ws = torch.empty((mla.workspace_bytes(batch, s_q, h_q, parts),), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((batch, s_q, h_q, W.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        rc = mla.lib().mla_get_metadata(mla._ptr(sl), batch, s_q, h_q, parts, mla._ptr(meta),
                                        mla._ptr(sb), mla._stream())
        assert rc == 0
        mla.decode(q, kc, bt, sl, case.scale, True, meta=meta, split_base=sb, num_parts=parts,
                   workspace=ws, out=out, lse=lse, fp8=fp8)

    _replay_checks(step, [out, lse], [meta, sb, ws])
    ref_out, ref_lse = oracle_all(case)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse,
            f"graph decode h_q={h_q} fp8={fp8}")


@pytest.mark.parametrize("h_q,fp8", [(16, True), (128, False)])
def test_sparse_call_replays_in_a_graph(h_q, fp8):
    import mla_paged_kv_fwd_amd as mla

    seqlens, s_q, topk = [700, 2100, 130], 2, 300
    print(f"graph sparse h_q={h_q} fp8={fp8}", flush=True)
    rng = np.random.default_rng(91 + h_q)
    case = W.make_case(seqlens, s_q, h_q, seed=92 + h_q, fp8=fp8, spare_pages=1, poison=True)
    idx = np.full((len(seqlens), s_q, topk), -1, dtype=np.int32)
    for b, L in enumerate(seqlens):
        for i in range(s_q):
            n = min(L, topk) - 17 * i
            idx[b, i, :n] = rng.choice(L, n, replace=False)
    q, kc, bt, _ = to_device(case)
    idx_d = torch.from_numpy(idx).cuda()
    parts = mla.default_num_parts(1, h_q, fp8=fp8, sparse=True)
    ws = torch.empty((mla.sparse_workspace_bytes(len(seqlens), s_q, h_q, topk, parts, fp8=fp8),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((len(seqlens), s_q, h_q, W.D_V), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(seqlens), s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        mla.decode_sparse(q, kc, bt, idx_d, case.scale, fp8=fp8, num_parts=parts, workspace=ws,
                          out=out, lse=lse)

    _replay_checks(step, [out, lse], [ws])
    ref, ref_lse = oracle.decode_sparse(case.q, case.cache, case.kind, case.block_table, idx,
                                        case.scale)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse,
            f"graph sparse h_q={h_q} fp8={fp8}")
