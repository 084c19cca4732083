"""Builds libqgemv.so (all HIP kernels + the C ABI) for gfx950 with hipcc, and
the benchmark's plain-read reference kernel into its own libqgemv_ceiling.so."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqgemv.so")
CEILING_SRC = os.path.join(HERE, "bench_csrc", "ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libqgemv_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed FP32 instructions
# (their host-pass warning about an unknown feature is harmless).
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, extra=()) -> str:
    """Compiles every source to an object in parallel, then links the library."""
    import concurrent.futures
    import tempfile
    flags = [f for f in HIPFLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="qgemv_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC, *flags, *extra, "-c", src, "-o", obj],
                               capture_output=True, text=True)
            return src, obj, r
        jobs = max(1, min(len(sources()), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, sources()))
        for src, _, r in results:
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError("hipcc failed compiling " + src)
        tmp = out + ".tmp"
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                            *[o for _, o, _ in results], "-o", tmp],
                           capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking " + out)
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_LIB) -> str:
    """The plain-read reference kernel (benchmark only; not part of the C ABI)."""
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, *HIPFLAGS, CEILING_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed compiling " + CEILING_SRC)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    print(build_ceiling())
