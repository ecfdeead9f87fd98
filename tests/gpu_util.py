"""Helpers for the GPU parity tests: host Case -> device tensors, library call,
comparison with the oracle at the stated tolerances."""
import numpy as np
import torch

import oracle

# Parity bar for floating-point outputs
MAX_ABS = 2e-2      # max |out_gpu - out_ref|
REL_L2 = 1e-2       # ||out_gpu - out_ref||_2 / ||out_ref||_2 over the compared rows
LSE_ABS = 1e-3      # max |lse_gpu - lse_ref|


def to_device(case):
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).cuda()
    if case.kind == 0:
        kc = torch.from_numpy(case.cache.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        kc = torch.from_numpy(case.cache).cuda()
    bt = torch.from_numpy(case.block_table).cuda()
    sl = torch.from_numpy(case.seqlens).cuda()
    return q, kc, bt, sl


def run_gpu(case, num_parts=None, dev=None):
    import mla_paged_kv_fwd_amd as mla

    q, kc, bt, sl = dev if dev is not None else to_device(case)
    out, lse = mla.decode(q, kc, bt, sl, case.scale, case.causal, num_parts=num_parts,
                          fp8=(case.kind == 1))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_all(case):
    return oracle.decode(case.q, case.cache, case.kind, case.block_table, case.seqlens, case.scale,
                         case.causal)


def compare(out, lse, ref_out, ref_lse, label=""):
    """out/ref_out [..., 512]; lse/ref_lse [...] aligned.  Raises on failure."""
    out = np.asarray(out, dtype=np.float64).reshape(-1, 512)
    ref_out = np.asarray(ref_out, dtype=np.float64).reshape(-1, 512)
    lse = np.asarray(lse, dtype=np.float64).reshape(-1)
    ref_lse = np.asarray(ref_lse, dtype=np.float64).reshape(-1)
    empty = np.isneginf(ref_lse)
    assert np.all(np.isneginf(lse[empty])), f"{label}: empty rows need lse=-inf"
    assert np.all(out[empty] == 0), f"{label}: empty rows need out=0"
    full = ~empty
    assert np.all(np.isfinite(out[full])) and np.all(np.isfinite(lse[full])), f"{label}: non-finite"
    d = out[full] - ref_out[full]
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref_out[full]), 1e-30)) if d.size else 0.0
    dl = float(np.max(np.abs(lse[full] - ref_lse[full]))) if full.any() else 0.0
    msg = f"{label}: max_abs={max_abs:.3e} rel_l2={rel:.3e} lse_abs={dl:.3e}"
    print(msg, flush=True)
    assert max_abs <= MAX_ABS and rel <= REL_L2 and dl <= LSE_ABS, msg
    return max_abs, rel, dl


def sample_rows(case, n, seed):
    """Deterministic sample of (b, i, h) rows, always including the corners."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, case.batch, size=n)
    i = rng.integers(0, case.s_q, size=n)
    h = rng.integers(0, case.h_q, size=n)
    rows = np.stack([b, i, h], axis=1)
    corners = np.array([[0, 0, 0], [case.batch - 1, case.s_q - 1, case.h_q - 1],
                        [0, case.s_q - 1, case.h_q - 1], [case.batch - 1, 0, 0]])
    return np.unique(np.concatenate([corners, rows]), axis=0).astype(np.int32)
