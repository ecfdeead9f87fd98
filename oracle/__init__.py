"""CPU oracle for MLA paged-KV decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The decode library never does, and this
package never imports the library: the two share no code.

``mla_oracle.c`` holds the attention definition (fp64), the OCP E4M3FN decode
and encode, the FP8 record writer (the cache writer's definition) and the LSE
merge; ``plan.py`` holds the split-KV plan definition.  Every
function here is a thin ctypes wrapper or a plain loop.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import plan as _plan

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

D_QK = 576
D_V = 512
PAGE = 64

plan = _plan.plan
plan_overhead = _plan.overhead


def build():
    """Compile the oracle with gcc (OpenMP, -O2; no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.mla_oracle_decode_rows.argtypes = [
        P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int64, P,
        ctypes.c_double, ctypes.c_int, P, ctypes.c_int64, P, P, P]
    lib.mla_oracle_decode_rows.restype = ctypes.c_int
    lib.mla_oracle_lse_merge.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P, P]
    lib.mla_oracle_lse_merge.restype = None
    lib.mla_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.mla_oracle_e4m3_value.restype = ctypes.c_double
    lib.mla_oracle_fp8_record_values.argtypes = [P, P]
    lib.mla_oracle_fp8_record_values.restype = None
    lib.mla_oracle_fp8_record_bytes.restype = ctypes.c_int
    lib.mla_oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.mla_oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.mla_oracle_fp8_record_from_row.argtypes = [P, P]
    lib.mla_oracle_fp8_record_from_row.restype = None
    lib.mla_oracle_kv_write.argtypes = [P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int64, P,
                                        ctypes.c_int, P]
    lib.mla_oracle_kv_write.restype = None
    lib.mla_oracle_decode_sparse_rows.argtypes = [
        P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int64, P, ctypes.c_int,
        ctypes.c_double, P, ctypes.c_int64, P, P]
    lib.mla_oracle_decode_sparse_rows.restype = None
    lib.mla_oracle_bf16_token_bytes.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def decode_rows(q, cache, kind, block_table, seqlens, scale, causal, rows, windows=None):
    """Attention for the listed query rows.

    q: uint16 bf16 bits [batch, s_q, h_q, 576]; cache: uint16 [pages, 64, 576]
    (kind 0) or uint8 [pages, 64, 656] (kind 1); block_table: int32
    [batch, width]; seqlens: int32 [batch]; rows: int array [n, 3] of
    (b, i, h); windows: optional int64 [n, 2] key windows [lo, hi).
    Returns (out float64 [n, 512], lse float64 [n], threads used).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    cache = np.ascontiguousarray(cache)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = rows.shape[0]
    out = np.zeros((n, D_V), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    win = None
    if windows is not None:
        win = np.ascontiguousarray(np.asarray(windows, dtype=np.int64).reshape(-1, 2))
    _, s_q, h_q, _ = q.shape
    threads = lib.mla_oracle_decode_rows(
        _ptr(q), s_q, h_q, _ptr(cache), int(kind), _ptr(bt), bt.shape[1], _ptr(sl),
        float(scale), int(bool(causal)), _ptr(rows), n,
        _ptr(win) if win is not None else None, _ptr(out), _ptr(lse))
    return out, lse, threads


def all_rows(batch, s_q, h_q):
    """Every (b, i, h) triple in output order."""
    b, i, h = np.meshgrid(np.arange(batch), np.arange(s_q), np.arange(h_q), indexing="ij")
    return np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1).astype(np.int32)


def decode(q, cache, kind, block_table, seqlens, scale, causal):
    """Whole-batch decode: returns out [b, s_q, h_q, 512] and lse [b, s_q, h_q] (fp64)."""
    batch, s_q, h_q, _ = q.shape
    out, lse, _ = decode_rows(q, cache, kind, block_table, seqlens, scale, causal,
                              all_rows(batch, s_q, h_q))
    return out.reshape(batch, s_q, h_q, D_V), lse.reshape(batch, s_q, h_q)


def lse_merge(o_parts, lse_parts):
    """Merge per-part (normalised output, lse) of one row: returns (out, lse)."""
    lib = _load()
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n_parts, dv = o.shape
    out = np.zeros((dv,), dtype=np.float64)
    lse = np.zeros((1,), dtype=np.float64)
    lib.mla_oracle_lse_merge(_ptr(o), _ptr(l), n_parts, dv, _ptr(out), _ptr(lse))
    return out, float(lse[0])


def e4m3_value(code):
    return _load().mla_oracle_e4m3_value(int(code))


def fp8_record_values(record):
    lib = _load()
    rec = np.ascontiguousarray(record, dtype=np.uint8)
    assert rec.size == lib.mla_oracle_fp8_record_bytes()
    k = np.zeros((D_QK,), dtype=np.float64)
    lib.mla_oracle_fp8_record_values(_ptr(rec), _ptr(k))
    return k


def fp8_record_bytes():
    return _load().mla_oracle_fp8_record_bytes()


def bf16_token_bytes():
    return _load().mla_oracle_bf16_token_bytes()


def e4m3_encode(x):
    """OCP E4M3FN code of a finite fp32 value with |x| <= 448 (nearest, ties
    to the even code)."""
    return int(_load().mla_oracle_e4m3_encode(ctypes.c_float(float(x))))


def fp8_record_from_row(row):
    """One bf16 row (uint16 bits [576]) -> its 656-byte FP8 record."""
    row = np.ascontiguousarray(row, dtype=np.uint16).reshape(D_QK)
    rec = np.zeros(656, dtype=np.uint8)
    _load().mla_oracle_fp8_record_from_row(_ptr(row), _ptr(rec))
    return rec


def kv_write(k_new, block_table, seqlens, cache, kind):
    """Cache writer: returns a copy of `cache` with the rows of k_new (uint16
    bf16 bits [batch, n_new, 576]) written at the end of each request (kind 0:
    bf16 rows, cache uint16 [pages, 64, 576]; kind 1: FP8 records, cache uint8
    [pages, 64, 656])."""
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    batch, n_new = k_new.shape[0], k_new.shape[1]
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.array(cache, copy=True)
    _load().mla_oracle_kv_write(_ptr(k_new), batch, n_new, _ptr(bt), bt.shape[1], _ptr(sl),
                                int(kind), _ptr(out))
    return out


def decode_sparse(q, cache, kind, block_table, indices, scale, rows=None):
    """Sparse decode: row (b, i, h) attends to the cached tokens listed in
    indices[b, i, :] (int32 positions within request b; the list ends at its
    first negative entry).
    q uint16 [batch, s_q, h_q, 576].  Returns (out float64 [..., 512], lse
    float64 [...]) for all rows, or for the listed (b, i, h) rows."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    batch, s_q, h_q = q.shape[:3]
    cache = np.ascontiguousarray(cache)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    idx = np.ascontiguousarray(indices, dtype=np.int32).reshape(batch, s_q, -1)
    topk = idx.shape[2]
    whole = rows is None
    if whole:
        rows = all_rows(batch, s_q, h_q)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((rows.shape[0], D_V), dtype=np.float64)
    lse = np.zeros((rows.shape[0],), dtype=np.float64)
    lib.mla_oracle_decode_sparse_rows(_ptr(q), s_q, h_q, _ptr(cache), int(kind), _ptr(bt), bt.shape[1],
                                      _ptr(idx), topk, float(scale), _ptr(rows), rows.shape[0],
                                      _ptr(out), _ptr(lse))
    if whole:
        return out.reshape(batch, s_q, h_q, D_V), lse.reshape(batch, s_q, h_q)
    return out, lse
