"""Loads the in-tree libmla.so for the tests, building it first only if absent."""
import ctypes
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mla_paged_kv_fwd_amd", "libmla.so")
_lib = None


def ensure_built():
    if not os.path.exists(LIB):
        from mla_paged_kv_fwd_amd import build

        build.build()


def load_lib():
    global _lib
    if _lib is None:
        ensure_built()
        _lib = ctypes.CDLL(LIB)
    return _lib
