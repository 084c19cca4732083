"""The benchmark's contract, checked without a GPU.

bench.py runs on one GPU: any other --gpus exits before touching a device,
with a message.  Every case it names has a kernel whose sources exist, and
every committed profile summary parses into a command, a duration and
calibrated traffic that bench.py can attach to its roofline.
"""
import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_headline_is_the_largest_batch1_dense_gemv():
    # the headline workload: fp8 7168 x 16384 (117.6 MB per call), the largest
    # batch-1 dense GEMV; the default suite covers every workload shape
    assert bench.HEADLINE == "fp8b128_O7168_I16384"
    assert bench.HEADLINE in bench.SUITE
    import workloads as W
    for name in W.WORKLOADS:
        assert name in bench.SUITE, name
    assert "mq4v2rot_O8192_I8192" in bench.SUITE
    assert len(set(bench.CASE_NAMES)) == len(bench.CASE_NAMES)


def test_kernel_sources_exist_and_digest_is_stable():
    pkg = os.path.join(ROOT, "quantized_weight_decode_amd")
    for kernel, src in bench.KERNEL_SOURCES.items():
        assert os.path.exists(os.path.join(pkg, src)), src
        d = bench.kernel_digest(kernel)
        assert re.fullmatch(r"[0-9a-f]{64}", d) and d == bench.kernel_digest(kernel)


def test_profile_summaries_parse():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*__*.md")))
    assert paths, "no profile summaries committed"
    for path in paths:
        kernel, workload = os.path.basename(path)[:-3].split("__")
        assert kernel in bench.KERNEL_SOURCES, path
        assert workload in bench.CASE_NAMES, path
        text = open(path).read()
        assert "rocprofv3 --kernel-trace --stats" in text and "--pmc FETCH_SIZE" in text
        assert "--pmc WRITE_SIZE" in text
        row = re.search(r"^\| `[^`]+` \| (\d+) \| ([0-9.]+) \|", text, re.M)
        assert row and int(row.group(1)) > 0 and float(row.group(2)) > 0
        t = bench.profiled_traffic(kernel, workload)
        # None once the kernel's sources changed since the counters were taken
        assert t is None or t > 0


def test_sources_digest_covers_the_kernels_and_is_stable():
    d = bench.sources_digest()
    assert re.fullmatch(r"[0-9a-f]{64}", d) and d == bench.sources_digest()
    covered = {os.path.relpath(p, ROOT) for g in bench.SOURCE_GLOBS
               for p in glob.glob(os.path.join(ROOT, g))}
    for src in bench.KERNEL_SOURCES.values():
        assert os.path.join("quantized_weight_decode_amd", src) in covered, src
    assert "include/qgemv.h" in covered and "bench.py" in covered
