"""bench.py's command-line contract on a machine without a GPU: several GPUs
are refused with a message, and the roofline helpers read the committed
counter summaries."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_measured_traffic_matches_sources_or_is_none():
    sys.path.insert(0, ROOT)
    import bench

    # every traffic line names a kernel and workload; a value comes back only
    # while the listed sources still hash to what was profiled
    for kernel, workload in [("decode_rowgroup_kernel<false, false>", "membound"),
                             ("decode_rows64_kernel<false>", "computebound"),
                             ("decode_rows128_kernel", "longctx"),
                             ("decode_rows64_fp8_kernel<false>", "fp8")]:
        t = bench.measured_traffic(kernel, workload)
        assert t is None or t > 0
    assert bench.measured_traffic("no_such_kernel", "membound") is None


def test_headline_profile_matches_the_kernel_source():
    # the default bench line reports the membound kernel's measured traffic;
    # a change to its sources needs a fresh counter profile under profiles/
    sys.path.insert(0, ROOT)
    import bench

    t = bench.measured_traffic("decode_rowgroup_kernel<false, false>", "membound")
    assert t is not None, "profiles/decode_rowgroup_kernel_membound.md is stale: re-profile"
    assert 600e6 < t < 700e6  # 608.5 MB algorithmic per launch


def test_sweep_flags_parse():
    for flag in ("--sweep", "--sweep-fp8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", flag],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and "one GPU" in r.stderr, r.stderr
