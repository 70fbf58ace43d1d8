"""Build libcnhwc.so (gfx950) in-tree from csrc/ with hipcc, and the benchmark's
machine-ceiling microbenchmarks (ceiling/ceiling.hip) into libcnhwc_ceiling.so.

Every translation unit is compiled with packed-fp32 instruction selection
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops) and a per-kernel
resource report; the build fails if any kernel spills to scratch memory.
Usage:  python -m convolution_nhwc_amd.build   (or call build()).
"""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcnhwc.so")
CEILING_SRC = os.path.join(HERE, "ceiling", "ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libcnhwc_ceiling.so")
ARCH = "gfx950"

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-variable",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = res.stdout + res.stderr
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, log))
    if verbose:
        print(log)
    return obj, log


def _scratch_offenders(log):
    """Kernels whose resource report shows scratch (spill) bytes."""
    bad, current = [], None
    for line in log.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append((current, int(m.group(1))))
    return bad


def build(jobs=None, verbose=False, allow_scratch=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, len(srcs))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    logs = "\n".join(r[1] for r in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(logs)
    bad = _scratch_offenders(logs)
    if bad and not allow_scratch:
        raise RuntimeError("kernels spill to scratch: %s" % bad)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [r[0] for r in results]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    build_ceiling()
    return LIB


def build_ceiling():
    """The machine-ceiling microbenchmarks the benchmark reports against."""
    tmp = CEILING_LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc()] + FLAGS + ["-shared", CEILING_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (CEILING_SRC, res.stdout + res.stderr))
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, allow_scratch="--allow-scratch" in sys.argv))
