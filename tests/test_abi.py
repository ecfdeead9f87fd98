"""CPU checks of the C ABI: exports, status codes, host-side validation and the
planner's host twin against the oracle plan.  No GPU call is made: every
argument error is reported before the library touches HIP."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from tests.libmla_loader import load_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = load_lib()
    names = _declared_functions()
    assert "mla_decode_fwd" in names and "mla_get_metadata" in names and "mla_decode_fwd_fp8" in names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = load_lib()
    lib.mla_status_string.restype = ctypes.c_char_p
    for code in (0, -1, -2, -3, -4, 7):
        s = lib.mla_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_sizes_and_overhead():
    lib = load_lib()
    lib.mla_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_metadata_ints.restype = ctypes.c_size_t
    assert lib.mla_metadata_ints(256) == 256 * 8
    assert lib.mla_workspace_bytes(128, 1, 16, 256) == (128 + 256) * 16 * 513 * 4
    assert lib.mla_workspace_bytes(0, 1, 16, 256) == 0
    for s_q in (1, 2, 4):
        for h_q in (16, 32, 64, 128):
            assert lib.mla_plan_overhead(s_q, h_q) == oracle.plan_overhead(s_q, h_q)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _decode(lib, **kw):
    args = dict(q=FAKE, kc=FAKE, num_pages=10, bt=FAKE, stride=4, sl=FAKE, batch=2, s_q=1, h_q=16,
                scale=0.04, causal=0, meta=FAKE, sb=FAKE, parts=8, ws=ctypes.c_void_p(0x10000),
                ws_bytes=1 << 30, out=FAKE, lse=FAKE)
    args.update(kw)
    fn = lib.mla_decode_fwd
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return fn(args["q"], args["kc"], args["num_pages"], args["bt"], args["stride"], args["sl"],
              args["batch"], args["s_q"], args["h_q"], args["scale"], args["causal"], args["meta"],
              args["sb"], args["parts"], args["ws"], args["ws_bytes"], args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID),
    (dict(kc=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(out=None), INVALID),
    (dict(batch=0), INVALID),
    (dict(num_pages=0), INVALID),
    (dict(stride=0), INVALID),
    (dict(causal=2), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-0.04), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(h_q=8), UNSUPPORTED),
    (dict(h_q=48), UNSUPPORTED),
    (dict(s_q=3), UNSUPPORTED),
    (dict(s_q=8), UNSUPPORTED),
    (dict(batch=100000), UNSUPPORTED),
    (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=1000), WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x10010)), WORKSPACE),
])
def test_argument_errors_are_reported_before_any_gpu_call(kw, expect):
    assert _decode(load_lib(), **kw) == expect


def test_metadata_argument_errors():
    lib = load_lib()
    fn = lib.mla_get_metadata
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert fn(None, 2, 1, 16, 8, FAKE, FAKE, None) == INVALID
    assert fn(FAKE, 2, 1, 16, 0, FAKE, FAKE, None) == INVALID
    assert fn(FAKE, 2, 1, 12, 8, FAKE, FAKE, None) == UNSUPPORTED
    assert fn(FAKE, 2, 1, 16, 100000, FAKE, FAKE, None) == UNSUPPORTED


@pytest.mark.parametrize("name", ["mla_kv_cache_write", "mla_kv_cache_write_fp8"])
def test_cache_writer_argument_errors(name):
    lib = load_lib()
    fn = getattr(lib, name)
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert fn(None, 2, 1, FAKE, 4, FAKE, FAKE, 10, None) == INVALID      # null k_new
    assert fn(FAKE, 2, 1, FAKE, 4, None, FAKE, 10, None) == INVALID      # null seqlens
    assert fn(FAKE, 2, 1, FAKE, 4, FAKE, None, 10, None) == INVALID      # null cache
    assert fn(FAKE, 0, 1, FAKE, 4, FAKE, FAKE, 10, None) == INVALID      # batch 0
    assert fn(FAKE, 2, 0, FAKE, 4, FAKE, FAKE, 10, None) == INVALID      # n_new 0
    assert fn(FAKE, 2, 1, FAKE, 0, FAKE, FAKE, 10, None) == INVALID      # stride 0
    assert fn(FAKE, 2, 1, FAKE, 4, FAKE, FAKE, 0, None) == INVALID       # no pages
    assert fn(FAKE, 16384, 1 << 17, FAKE, 4, FAKE, FAKE, 10, None) == UNSUPPORTED  # >= 2^31 rows


def test_sparse_decode_argument_errors():
    lib = load_lib()
    fn = lib.mla_decode_sparse
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    sz = lib.mla_sparse_workspace_bytes
    sz.restype = ctypes.c_size_t
    sz.argtypes = [ctypes.c_int] * 6
    need = sz(2, 1, 128, 2048, 1, 64)
    # the records are read in place: token ids (4 B per list entry), lengths,
    # plan and the one-token problems' split partials, for any h_q and format
    for h_q in (16, 128):
        dec = (2 + 64) * h_q * 513 * 4
        assert dec + 2 * 2048 * 4 <= sz(2, 1, h_q, 2048, 1, 64) < dec + 2 * 2048 * 4 + 8192
    assert sz(2, 1, 128, 2048, 0, 64) == need
    assert sz(0, 1, 128, 2048, 1, 64) == 0 and sz(2, 1, 128, 2048, 2, 64) == 0
    ws = ctypes.c_void_p(0x100000)

    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, fmt=1, pages=10, bt=FAKE, stride=4, idx=FAKE, topk=2048, batch=2,
                 s_q=1, h_q=128, scale=0.04, parts=64, ws=ws, ws_bytes=need, out=FAKE, lse=FAKE)
        a.update(kw)
        return fn(a["q"], a["kc"], a["fmt"], a["pages"], a["bt"], a["stride"], a["idx"], a["topk"],
                  a["batch"], a["s_q"], a["h_q"], a["scale"], a["parts"], a["ws"], a["ws_bytes"],
                  a["out"], a["lse"], None)
    assert call(idx=None) == INVALID
    assert call(fmt=2) == INVALID
    assert call(topk=0) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(h_q=48) == UNSUPPORTED
    assert call(batch=8192, s_q=4) == UNSUPPORTED          # 32768 one-token problems
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x100010)) == WORKSPACE
    # token ids are int32: page * 64 + slot must stay below 2^31
    assert call(pages=(2**31 - 1) // 64 + 1) == UNSUPPORTED
    # list positions are counted in int32: 16384 lists x 2^17 + 64 positions do not fit
    assert call(batch=16384, topk=2**17 + 1, ws_bytes=2**62) == UNSUPPORTED
    assert sz(16384, 1, 128, 2**17 + 1, 1, 64) == 0 and sz(16384, 1, 128, 2**17 - 64, 1, 64) > 0


def _host_plan(lib, seqlens, s_q, h_q, parts):
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    meta = np.full((parts, 8), 12345, dtype=np.int32)
    sb = np.full((len(sl) + 1,), 12345, dtype=np.int32)
    fn = lib.mla_get_metadata_host
    fn.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    st = fn(sl.ctypes.data, len(sl), s_q, h_q, parts, meta.ctypes.data, sb.ctypes.data)
    assert st == OK
    return meta, sb


PLAN_CASES = [
    ([37, 100], 1, 16, 8),
    ([4096] * 128, 1, 16, 256),
    ([131072] * 8, 1, 128, 256),
    ([0, 5, 0, 0, 64, 65, 0], 2, 32, 7),
    ([1], 1, 16, 1024),
    ([0, 0, 0], 1, 16, 8),
    ([7] * 300, 2, 64, 16),
    ([16384] * 64, 1, 128, 256),
]


@pytest.mark.parametrize("seqlens,s_q,h_q,parts", PLAN_CASES)
def test_host_planner_equals_oracle_plan(seqlens, s_q, h_q, parts):
    meta, sb = _host_plan(load_lib(), seqlens, s_q, h_q, parts)
    ref_meta, ref_sb = oracle.plan(seqlens, parts, oracle.plan_overhead(s_q, h_q))
    np.testing.assert_array_equal(meta, np.array(ref_meta, dtype=np.int32))
    np.testing.assert_array_equal(sb, np.array(ref_sb, dtype=np.int32))


def test_host_planner_random_batches_equal_oracle():
    rng = np.random.default_rng(7)
    lib = load_lib()
    for _ in range(60):
        batch = int(rng.integers(1, 40))
        seqlens = rng.integers(0, 3000, size=batch)
        seqlens[rng.random(batch) < 0.2] = 0
        parts = int(rng.integers(1, 300))
        s_q, h_q = int(rng.choice([1, 2])), int(rng.choice([16, 32, 64, 128]))
        meta, sb = _host_plan(lib, seqlens, s_q, h_q, parts)
        ref_meta, ref_sb = oracle.plan(list(seqlens), parts, oracle.plan_overhead(s_q, h_q))
        np.testing.assert_array_equal(meta, np.array(ref_meta, dtype=np.int32))
        np.testing.assert_array_equal(sb, np.array(ref_sb, dtype=np.int32))


def test_check_argument_errors():
    lib = load_lib()
    bt = lib.mla_check_block_table
    bt.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    assert bt(None, 4, FAKE, 8, 100, FAKE, None) == INVALID
    assert bt(FAKE, 4, FAKE, 8, 100, None, None) == INVALID
    assert bt(FAKE, 0, FAKE, 8, 100, FAKE, None) == INVALID
    assert bt(FAKE, 4, FAKE, 0, 100, FAKE, None) == INVALID
    assert bt(FAKE, 4, FAKE, 8, 0, FAKE, None) == INVALID
    assert bt(FAKE, 16385, FAKE, 8, 100, FAKE, None) == UNSUPPORTED
    sp = lib.mla_check_sparse_indices
    sp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert sp(FAKE, 8, 100, None, 64, 2, 1, FAKE, None) == INVALID
    assert sp(FAKE, 8, 100, FAKE, 0, 2, 1, FAKE, None) == INVALID
    assert sp(FAKE, 8, 100, FAKE, 64, 2, 0, FAKE, None) == INVALID
    assert sp(FAKE, 8, 100, FAKE, 64, 8192, 4, FAKE, None) == UNSUPPORTED


def _header_macro(name):
    m = re.search(r"#define\s+%s\s+(\d+)" % name, open(HEADER).read())
    assert m, name
    return int(m.group(1))


def test_header_limits_match_the_library():
    """MLA_MAX_BATCH and MLA_MAX_PARTS are the limits the calls enforce: at
    the limit the call gets past the size checks (the host planner succeeds;
    the decode call then stops at the workspace check, which comes after
    them), one past it the call returns MLA_ERR_UNSUPPORTED."""
    lib = load_lib()
    max_batch, max_parts = _header_macro("MLA_MAX_BATCH"), _header_macro("MLA_MAX_PARTS")
    fn = lib.mla_get_metadata_host
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]

    def host_plan(batch, parts):
        sl = np.full(batch, 100, dtype=np.int32)
        meta = np.zeros((parts, 8), dtype=np.int32)
        sb = np.zeros(batch + 1, dtype=np.int32)
        return fn(sl.ctypes.data, batch, 1, 16, parts, meta.ctypes.data, sb.ctypes.data)

    assert host_plan(max_batch, 64) == OK
    assert host_plan(max_batch + 1, 64) == UNSUPPORTED
    assert host_plan(7, max_parts) == OK
    assert host_plan(7, max_parts + 1) == UNSUPPORTED
    # decode: past the size checks means the workspace check answers
    assert _decode(lib, batch=max_batch, ws_bytes=256) == WORKSPACE
    assert _decode(lib, batch=max_batch + 1, ws_bytes=256) == UNSUPPORTED
    assert _decode(lib, parts=max_parts, ws_bytes=256) == WORKSPACE
    assert _decode(lib, parts=max_parts + 1, ws_bytes=256) == UNSUPPORTED


def test_ceiling_library_exports_its_header():
    """The ceilings library (bench.py's measured rates) exports every call
    include/mla_ceiling.h declares, and refuses bad arguments before any
    launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "mla_paged_kv_fwd_amd", "libmla_ceiling.so"))
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mla_ceiling.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(mla_ceiling_[a-z0-9_]+)\s*\(", text)))
    assert len(names) == 4
    for n in names:
        assert hasattr(lib, n), n
    lib.mla_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    assert lib.mla_ceiling_stream_read(None, 1024, 4, FAKE, None) == -1
    assert lib.mla_ceiling_mfma(2, 10, 1, FAKE, None) == -1
