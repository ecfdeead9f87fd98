"""libmla used from plain C: tests/c_abi/decode_from_c plans and decodes a
small paged problem (s_q 2 causal, h_q 64, ragged lengths, pages handed out
in reverse) through include/mla.h and the HIP runtime only, and writes its
inputs and outputs; the oracle recomputes the outputs from those inputs."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.gpu_util import compare

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("fp8", [0, 1])
def test_decode_from_c_matches_oracle(fp8, tmp_path):
    exe = os.path.join(HERE, "c_abi", "decode_from_c")
    if not os.path.exists(exe):
        from tests.c_abi.build import build
        exe = build()
    print(f"decode_from_c fp8={fp8}", flush=True)
    r = subprocess.run([exe, str(tmp_path), str(fp8)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    batch, s_q, h_q, pages, width = map(int, (tmp_path / "shape.txt").read_text().split())
    q = np.fromfile(tmp_path / "q.bin", dtype=np.uint16).reshape(batch, s_q, h_q, 576)
    if fp8:
        cache = np.fromfile(tmp_path / "cache.bin", dtype=np.uint8).reshape(pages, 64, 656)
    else:
        cache = np.fromfile(tmp_path / "cache.bin", dtype=np.uint16).reshape(pages, 64, 576)
    bt = np.fromfile(tmp_path / "bt.bin", dtype=np.int32).reshape(batch, width)
    seqlens = np.fromfile(tmp_path / "seqlens.bin", dtype=np.int32)
    out_bits = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(batch, s_q, h_q, 512)
    out = (out_bits.astype(np.uint32) << 16).view(np.float32)
    lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(batch, s_q, h_q)
    ref, ref_lse = oracle.decode(q, cache, fp8, bt, seqlens, 576 ** -0.5, True)
    compare(out, lse, ref, ref_lse, f"C consumer fp8={fp8}")
