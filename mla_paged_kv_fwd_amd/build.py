"""Build libmla.so in-tree with hipcc for gfx950."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["api.hip", "plan.hip", "decode.hip", "decode_rows64.hip", "decode_rows64_fp8.hip",
           "decode_rows128.hip", "combine.hip", "kv_write.hip", "sparse.hip", "check.hip"]
# measured ceilings of the part (stream read, MFMA loops), a library of its own
CEILING_LIB = os.path.join(HERE, "libmla_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the direct-to-LDS asm names m0 as clobbered; the compiler reserves m0
    "-Wno-inline-asm",
]
# Per-source extras.  decode.hip: MFMA accumulators in VGPRs, so the
# online-softmax rescale multiplies them in place instead of shuttling them
# through AGPR copies (its accumulators fit in the 256 VGPRs).
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(lib + ".tmp", lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB)
    if verbose:
        print("built", LIB, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
