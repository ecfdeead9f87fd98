"""Build the plain-C consumer of libmla (tests/c_abi/decode_from_c) with gcc
against include/mla.h, the HIP runtime and the in-tree libmla.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "decode_from_c")


def build():
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "decode_from_c.c"), "-o", EXE,
           "-L/opt/rocm/lib", "-lamdhip64", "-L" + os.path.join(ROOT, "mla_paged_kv_fwd_amd"),
           "-lmla", "-Wl,-rpath,$ORIGIN/../../mla_paged_kv_fwd_amd", "-Wl,-rpath,/opt/rocm/lib",
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C consumer failed:\n" + r.stderr)
    return EXE


if __name__ == "__main__":
    print(build())
