"""Python binding of libmla: MLA decode over a paged latent KV cache on MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/mla.h``: every
step of the computation runs in the library's HIP kernels.  PyTorch provides
device memory and the current stream only.  If ``libmla.so`` has not been
built, every call raises; there is no fallback path.
"""
import ctypes
import os

import torch

__all__ = [
    "MlaError", "lib", "D_QK", "D_V", "PAGE", "FP8_RECORD", "META_INTS",
    "default_num_parts", "plan_overhead", "workspace_bytes", "get_metadata",
    "get_metadata_host", "decode", "decode_attn", "decode_combine", "decode_sparse",
    "sparse_workspace_bytes", "kv_cache_write", "decode_noalloc", "noalloc_scratch_need",
    "status_string",
]

D_QK = 576
D_V = 512
PAGE = 64
FP8_RECORD = 656
META_INTS = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")
# measured ceilings of the part (include/mla_ceiling.h); loaded by bench.py only
CEILING_LIB_PATH = os.path.join(_HERE, "libmla_ceiling.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_metadata_ints": (_SZ, [_I]),
    "mla_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "mla_plan_overhead": (_I, [_I, _I]),
    "mla_default_num_parts": (_I, [_I, _I, _I]),
    "mla_default_num_parts_ex": (_I, [_I, _I, _I, _I, _I]),
    "mla_default_num_parts_for": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "mla_get_metadata": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "mla_get_metadata_host": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "mla_decode_fwd": (_I, [_P, _P, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I, _P, _SZ,
                            _P, _P, _P]),
    "mla_decode_fwd_fp8": (_I, [_P, _P, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I, _P,
                                _SZ, _P, _P, _P]),
    "mla_decode_attn": (_I, [_P, _P, _I, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I, _P,
                             _SZ, _P, _P, _P]),
    "mla_decode_combine": (_I, [_P, _I, _I, _I, _I, _P, _SZ, _P, _P, _P]),
    "mla_kv_cache_write": (_I, [_P, _I, _I, _P, _I, _P, _P, _I64, _P]),
    "mla_sparse_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "mla_decode_sparse": (_I, [_P, _P, _I, _I64, _P, _I, _P, _I, _I, _I, _I, _F, _I, _P, _SZ, _P,
                               _P, _P]),
    "mla_kv_cache_write_fp8": (_I, [_P, _I, _I, _P, _I, _P, _P, _I64, _P]),
    "mla_check_block_table": (_I, [_P, _I, _P, _I, _I64, _P, _P]),
    "mla_noalloc_scratch_need": (_SZ, [_I, _I, _I, _I]),
    "mla_decode_fwd_noalloc": (_I, [_P, _P, _I, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _P]),
    "mla_check_sparse_indices": (_I, [_P, _I, _I64, _P, _I, _I, _I, _P, _P]),
}


class MlaError(RuntimeError):
    pass


def lib():
    """Load libmla.so (built in-tree by ``mla_paged_kv_fwd_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MlaError(f"{LIB_PATH} is not built; run `python -m mla_paged_kv_fwd_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().mla_status_string(int(status)).decode()


def _check(status, what):
    if status != 0:
        raise MlaError(f"{what}: {status_string(status)} ({status})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def plan_overhead(s_q, h_q):
    return lib().mla_plan_overhead(s_q, h_q)


def workspace_bytes(batch, s_q, h_q, num_parts):
    return lib().mla_workspace_bytes(batch, s_q, h_q, num_parts)


def default_num_parts(s_q, h_q, device=None, fp8=False, sparse=False, batch=None, max_seqlen=None):
    """Plan size that fills the GPU in one round for this shape and cache
    format (sparse=True: sparse decode of h_q heads).  With batch and
    max_seqlen (the longest request, or an upper bound), the size the library
    measures fastest for them (mla_default_num_parts_for)."""
    dev = torch.cuda.current_device() if device is None else int(device)
    if batch is not None and max_seqlen is not None:
        n = lib().mla_default_num_parts_for(dev, int(batch), int(max_seqlen), s_q, h_q, 1 if fp8 else 0,
                                            1 if sparse else 0)
    else:
        n = lib().mla_default_num_parts_ex(dev, s_q, h_q, 1 if fp8 else 0, 1 if sparse else 0)
    if n < 0:
        _check(n, "mla_default_num_parts")
    return n


def get_metadata(seqlens, s_q, h_q, num_parts=None, fp8=False, max_seqlen=None):
    """Plan split-KV work on the GPU.  seqlens: int32 CUDA tensor [batch];
    without num_parts, the size that suits the cache format (fp8) and, given
    max_seqlen (the longest request or an upper bound), the batch's lengths.

    Returns (meta int32 [num_parts, 8], split_base int32 [batch + 1], num_parts).
    """
    if seqlens.dtype != torch.int32 or not seqlens.is_cuda or not seqlens.is_contiguous():
        raise MlaError("seqlens must be a contiguous int32 CUDA tensor")
    batch = seqlens.shape[0]
    if num_parts is None:
        num_parts = default_num_parts(s_q, h_q, seqlens.device.index, fp8=fp8, batch=batch,
                                      max_seqlen=max_seqlen)
    meta = torch.empty((num_parts, META_INTS), dtype=torch.int32, device=seqlens.device)
    split_base = torch.empty((batch + 1,), dtype=torch.int32, device=seqlens.device)
    _check(lib().mla_get_metadata(_ptr(seqlens), batch, s_q, h_q, num_parts, _ptr(meta),
                                  _ptr(split_base), _stream()), "mla_get_metadata")
    return meta, split_base, num_parts


def get_metadata_host(seqlens, s_q, h_q, num_parts):
    """Host twin of get_metadata on CPU int32 tensors (no GPU needed)."""
    sl = torch.as_tensor(seqlens, dtype=torch.int32).contiguous()
    batch = sl.shape[0]
    meta = torch.empty((num_parts, META_INTS), dtype=torch.int32)
    split_base = torch.empty((batch + 1,), dtype=torch.int32)
    _check(lib().mla_get_metadata_host(_ptr(sl), batch, s_q, h_q, num_parts, _ptr(meta),
                                       _ptr(split_base)), "mla_get_metadata_host")
    return meta, split_base


def _validate(q, kcache, block_table, seqlens, fp8):
    """Dtypes, shapes and placement of the inputs (seqlens may be None)."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[-1] != D_QK:
        raise MlaError("q must be bf16 [batch, s_q, h_q, 576]")
    if fp8:
        if kcache.dtype != torch.uint8 or tuple(kcache.shape[1:]) != (PAGE, FP8_RECORD):
            raise MlaError("fp8 kcache must be uint8 [pages, 64, 656]")
    else:
        if kcache.dtype != torch.bfloat16 or tuple(kcache.shape[1:]) != (PAGE, D_QK):
            raise MlaError("kcache must be bf16 [pages, 64, 576]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise MlaError("block_table must be int32 [batch, width]")
    if seqlens is not None and (seqlens.dtype != torch.int32 or seqlens.dim() != 1):
        raise MlaError("seqlens must be int32 [batch]")
    # the kernels index seqlens and block_table rows by q's batch index, and
    # size out and the workspace from q
    if block_table.shape[0] != q.shape[0]:
        raise MlaError("block_table must have one row per request of q")
    if seqlens is not None and seqlens.shape[0] != q.shape[0]:
        raise MlaError("seqlens must have one entry per request of q")
    for t in (q, kcache, block_table, seqlens):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise MlaError("all tensors must be contiguous CUDA tensors")


def _check_plan(q, meta, split_base, num_parts):
    """A caller's plan must have the shapes the kernels index: meta
    [num_parts, 8] and split_base [batch + 1], int32, on q's device."""
    if meta is None and split_base is None:
        return
    if meta is None or split_base is None or num_parts is None:
        raise MlaError("pass meta, split_base and num_parts together")
    for t, shape, name in ((meta, (int(num_parts), META_INTS), "meta"),
                           (split_base, (q.shape[0] + 1,), "split_base")):
        if (t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_cuda
                or t.device != q.device or not t.is_contiguous()):
            raise MlaError(f"{name} must be a contiguous int32 CUDA tensor {list(shape)} on q's device")


def _outputs(q, out, lse):
    """The caller's out / lse after checks, or new ones: the kernels write
    every element, so a wrong shape would be a write out of bounds."""
    b, s_q, h_q, _ = q.shape
    if out is None:
        out = torch.empty((b, s_q, h_q, D_V), dtype=torch.bfloat16, device=q.device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (b, s_q, h_q, D_V)
          or not out.is_cuda or not out.is_contiguous()):
        raise MlaError("out must be a contiguous bf16 CUDA tensor [batch, s_q, h_q, 512]")
    if lse is None:
        lse = torch.empty((b, s_q, h_q), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (b, s_q, h_q)
          or not lse.is_cuda or not lse.is_contiguous()):
        raise MlaError("lse must be a contiguous fp32 CUDA tensor [batch, s_q, h_q]")
    return out, lse


def _workspace(q, num_parts, workspace, need=None):
    if need is None:
        b, s_q, h_q, _ = q.shape
        need = workspace_bytes(b, s_q, h_q, num_parts)
    if workspace is None:
        return torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    if (workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_cuda
            or workspace.device != q.device or not workspace.is_contiguous()):
        raise MlaError("workspace must be a contiguous 1-D uint8 CUDA tensor on q's device")
    if workspace.numel() < need:
        raise MlaError(f"workspace holds {workspace.numel()} bytes; {need} needed")
    return workspace


def decode_attn(q, kcache, block_table, seqlens, softmax_scale, causal, meta, split_base,
                num_parts, workspace, out=None, lse=None, fp8=False):
    """Attention kernel only (the first half of decode)."""
    _validate(q, kcache, block_table, seqlens, fp8)
    _check_plan(q, meta, split_base, num_parts)
    workspace = _workspace(q, num_parts, workspace)
    out, lse = _outputs(q, out, lse)
    b, s_q, h_q, _ = q.shape
    _check(lib().mla_decode_attn(
        _ptr(q), _ptr(kcache), 1 if fp8 else 0, kcache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seqlens), b, s_q, h_q, float(softmax_scale), int(bool(causal)),
        _ptr(meta), _ptr(split_base), num_parts, _ptr(workspace), workspace.numel(), _ptr(out),
        _ptr(lse), _stream()), "mla_decode_attn")
    return out, lse


def decode_combine(split_base, num_parts, workspace, out, lse):
    """LSE merge of split partials (the second half of decode)."""
    if out.dtype != torch.bfloat16 or out.dim() != 4 or out.shape[-1] != D_V:
        raise MlaError("out must be bf16 [batch, s_q, h_q, 512]")
    b, s_q, h_q, _ = out.shape
    if not out.is_cuda or not out.is_contiguous():
        raise MlaError("out must be a contiguous CUDA tensor")
    if (lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (b, s_q, h_q)
            or lse.device != out.device or not lse.is_contiguous()):
        raise MlaError("lse must be a contiguous fp32 CUDA tensor [batch, s_q, h_q] on out's device")
    if (split_base.dtype != torch.int32 or tuple(split_base.shape) != (b + 1,)
            or split_base.device != out.device or not split_base.is_contiguous()):
        raise MlaError("split_base must be a contiguous int32 CUDA tensor [batch + 1] on out's device")
    workspace = _workspace(out, num_parts, workspace, workspace_bytes(b, s_q, h_q, num_parts))
    _check(lib().mla_decode_combine(_ptr(split_base), b, s_q, h_q, num_parts, _ptr(workspace),
                                    workspace.numel(), _ptr(out), _ptr(lse), _stream()),
           "mla_decode_combine")
    return out, lse


def _checks_enabled():
    """MLA_CHECK=1 in the environment runs the device-side input checks
    before each decode, sparse decode and cache write (one synchronisation
    each); off by default."""
    return os.environ.get("MLA_CHECK", "") not in ("", "0")


def _check_result(res):
    v = [int(x) & 0xFFFFFFFFFFFFFFFF for x in res.cpu().tolist()]
    if v[0] == 0:
        return 0, None
    where = v[1] & 0xFFFFFFFF
    return v[0], (v[1] >> 32, None if where == 0xFFFFFFFF else where)


def check_block_table(block_table, seqlens, num_pages):
    """Device-side check that every request's length fits the table and every
    block-table entry it uses is a page of the pool.  Synchronises.

    Returns (bad_requests, first) with first = None, or (request, logical
    page) for the smallest bad request; the page is None for a bad length."""
    res = torch.empty((2,), dtype=torch.int64, device=block_table.device)
    _check(lib().mla_check_block_table(_ptr(seqlens), seqlens.shape[0], _ptr(block_table),
                                       block_table.shape[1], int(num_pages), _ptr(res), _stream()),
           "mla_check_block_table")
    return _check_result(res)


def check_sparse_indices(block_table, indices, num_pages):
    """Device-side check that every list entry before its list's end names a
    logical page inside the table whose entry is a page of the pool.
    Synchronises.  Returns (bad_lists, first) with first = None, or
    (list b * s_q + i, list position) for the smallest bad list."""
    b, s_q, topk = indices.shape
    res = torch.empty((2,), dtype=torch.int64, device=indices.device)
    _check(lib().mla_check_sparse_indices(_ptr(block_table), block_table.shape[1], int(num_pages),
                                          _ptr(indices), topk, b, s_q, _ptr(res), _stream()),
           "mla_check_sparse_indices")
    return _check_result(res)


def _raise_if_bad(result, what):
    n, first = result
    if n:
        raise MlaError(f"{what}: {n} bad, first at {first}")


def decode(q, kcache, block_table, seqlens, softmax_scale, causal, meta=None, split_base=None,
           num_parts=None, workspace=None, out=None, lse=None, fp8=False):
    """MLA decode: returns (out bf16 [b, s_q, h_q, 512], lse fp32 [b, s_q, h_q])."""
    _validate(q, kcache, block_table, seqlens, fp8)
    if _checks_enabled():
        _raise_if_bad(check_block_table(block_table, seqlens, kcache.shape[0]),
                      "block table / seqlens")
    b, s_q, h_q, _ = q.shape
    if meta is None and split_base is None:
        # the table's width bounds the longest request
        meta, split_base, num_parts = get_metadata(seqlens, s_q, h_q, num_parts, fp8=fp8,
                                                   max_seqlen=block_table.shape[1] * PAGE)
    _check_plan(q, meta, split_base, num_parts)
    out, lse = _outputs(q, out, lse)
    workspace = _workspace(q, num_parts, workspace)
    fn = lib().mla_decode_fwd_fp8 if fp8 else lib().mla_decode_fwd
    _check(fn(_ptr(q), _ptr(kcache), kcache.shape[0], _ptr(block_table), block_table.shape[1],
              _ptr(seqlens), b, s_q, h_q, float(softmax_scale), int(bool(causal)), _ptr(meta),
              _ptr(split_base), num_parts, _ptr(workspace), workspace.numel(), _ptr(out),
              _ptr(lse), _stream()), "mla_decode_fwd")
    return out, lse


def noalloc_scratch_need(batch, s_q, h_q, fp8=False):
    """Scratch bytes decode_noalloc needs for this problem on the current
    device (it accepts up to MLA_NOALLOC_SCRATCH_BYTES, 128 MiB)."""
    return lib().mla_noalloc_scratch_need(batch, s_q, h_q, 1 if fp8 else 0)


def decode_noalloc(q, kcache, block_table, seqlens, softmax_scale, causal, out=None, lse=None,
                   fp8=False):
    """decode() through the allocation-free entry point: the library plans and
    keeps the plan and the split partials in its own fixed scratch, so the
    call allocates nothing (pass out and lse to allocate nothing here
    either).  Calls that overlap on one GPU race on that scratch."""
    _validate(q, kcache, block_table, seqlens, fp8)
    out, lse = _outputs(q, out, lse)
    b, s_q, h_q, _ = q.shape
    _check(lib().mla_decode_fwd_noalloc(
        _ptr(q), _ptr(kcache), 1 if fp8 else 0, kcache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seqlens), b, s_q, h_q, float(softmax_scale), int(bool(causal)),
        _ptr(out), _ptr(lse), _stream()), "mla_decode_fwd_noalloc")
    return out, lse


def kv_cache_write(k_new, block_table, seqlens, kcache, fp8=False):
    """Store k_new (bf16 [batch, n_new, 576]) as the newest n_new tokens of
    every request: bf16 rows into a bf16 cache, or 656-byte FP8 records into
    a uint8 [pages, 64, 656] cache.  Writes kcache in place and returns it."""
    if k_new.dtype != torch.bfloat16 or k_new.dim() != 3 or k_new.shape[-1] != D_QK:
        raise MlaError("k_new must be bf16 [batch, n_new, 576]")
    if fp8:
        if kcache.dtype != torch.uint8 or tuple(kcache.shape[1:]) != (PAGE, FP8_RECORD):
            raise MlaError("fp8 kcache must be uint8 [pages, 64, 656]")
    elif kcache.dtype != torch.bfloat16 or tuple(kcache.shape[1:]) != (PAGE, D_QK):
        raise MlaError("kcache must be bf16 [pages, 64, 576]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise MlaError("block_table must be int32 [batch, width]")
    if seqlens.dtype != torch.int32 or seqlens.dim() != 1:
        raise MlaError("seqlens must be int32 [batch]")
    for t in (k_new, kcache, block_table, seqlens):
        if not t.is_cuda or not t.is_contiguous():
            raise MlaError("all tensors must be contiguous CUDA tensors")
    batch, n_new = k_new.shape[0], k_new.shape[1]
    if block_table.shape[0] != batch or seqlens.shape[0] != batch:
        raise MlaError("block_table and seqlens must have one row / entry per request of k_new")
    if _checks_enabled():
        _raise_if_bad(check_block_table(block_table, seqlens, kcache.shape[0]),
                      "block table / seqlens")
    fn = lib().mla_kv_cache_write_fp8 if fp8 else lib().mla_kv_cache_write
    _check(fn(_ptr(k_new), batch, n_new, _ptr(block_table), block_table.shape[1], _ptr(seqlens),
              _ptr(kcache), kcache.shape[0], _stream()), "mla_kv_cache_write")
    return kcache


def sparse_workspace_bytes(batch, s_q, h_q, topk, num_parts, fp8=False):
    return lib().mla_sparse_workspace_bytes(batch, s_q, h_q, topk, 1 if fp8 else 0, num_parts)


def decode_sparse(q, kcache, block_table, indices, softmax_scale, fp8=False, num_parts=None,
                  workspace=None, out=None, lse=None):
    """Sparse decode: query token (b, i) attends to the tokens listed in
    indices[b, i] (int32 [batch, s_q, topk] positions within request b; the
    list ends at its first negative entry).  Returns (out bf16, lse fp32)."""
    if indices.dtype != torch.int32 or indices.dim() != 3 or not indices.is_cuda or \
            not indices.is_contiguous():
        raise MlaError("indices must be a contiguous int32 CUDA tensor [batch, s_q, topk]")
    b, s_q, h_q, _ = q.shape
    if tuple(indices.shape[:2]) != (b, s_q):
        raise MlaError("indices must be [batch, s_q, topk] for q's batch and s_q")
    _validate(q, kcache, block_table, None, fp8)
    if block_table.shape[0] != b:
        raise MlaError("block_table must have one row per request")
    if _checks_enabled():
        _raise_if_bad(check_sparse_indices(block_table, indices, kcache.shape[0]), "sparse lists")
    topk = indices.shape[2]
    if num_parts is None:
        num_parts = default_num_parts(1, h_q, q.device.index, fp8=fp8, sparse=True)
    need = sparse_workspace_bytes(b, s_q, h_q, topk, num_parts, fp8)
    if need == 0:
        raise MlaError("sparse decode: lists too long for int32 positions")
    workspace = _workspace(q, num_parts, workspace, need)
    out, lse = _outputs(q, out, lse)
    _check(lib().mla_decode_sparse(
        _ptr(q), _ptr(kcache), 1 if fp8 else 0, kcache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(indices), topk, b, s_q, h_q, float(softmax_scale), num_parts,
        _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream()), "mla_decode_sparse")
    return out, lse
