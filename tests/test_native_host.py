"""CPU tests that build small native programs against the library's own
sources and run them on the host:

- the exhaustive check of the kernels' division by launch constants
  (``native/fastdiv_exhaustive.cpp`` on ``csrc/fastdiv.h``);
- the C ABI's host logic (validation, dispatcher, chunk planner, workspace
  sizing, pointer checks) built with AddressSanitizer and
  UndefinedBehaviorSanitizer on the host side and driven by
  ``native/abi_sanitize.c`` (no kernel is launched).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
NATIVE = os.path.join(HERE, "native")
BUILD = os.path.join(NATIVE, "_build")
CSRC = os.path.join(ROOT, "convolution_nhwc_amd", "csrc")


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        pytest.skip("hipcc not available")
    return exe


def test_fastdiv_exhaustive():
    """fdiv(q, make_fastdiv(d)) == q / d for every d <= 70000 and every
    q < 2^20, the top 4096 dividends below 2^31, the last multiples of d below
    2^31 and their neighbours, and 2^22 random pairs below 2^31."""
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "fastdiv_exhaustive")
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17",
                    os.path.join(NATIVE, "fastdiv_exhaustive.cpp"), "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0 and res.stdout.startswith("ok "), res.stdout + res.stderr
    assert int(res.stdout.split()[1]) > 70000 * (1 << 20)


SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _sources():
    import glob
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _build_sanitized():
    """Every library source compiled with the host-side sanitizers (device
    code is compiled as usual and never launched), linked with the driver;
    cached on a hash of the inputs."""
    import concurrent.futures
    import glob
    import hashlib
    inputs = _sources() + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + \
        [os.path.join(ROOT, "include", "cnhwc.h"), os.path.join(NATIVE, "abi_sanitize.c")]
    h = hashlib.sha256()
    for p in inputs:
        with open(p, "rb") as f:
            h.update(f.read())
    out = os.path.join(BUILD, "asan")
    exe = os.path.join(out, "abi_sanitize")
    stamp = os.path.join(out, "inputs.sha256")
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == h.hexdigest():
        return exe
    os.makedirs(out, exist_ok=True)
    cc = hipcc()
    common = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN

    def comp(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        r = subprocess.run([cc] + common + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj
    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(comp, _sources()))
    drv = os.path.join(out, "abi_sanitize.o")
    r = subprocess.run([cc, "-x", "c++", "-O1", "-std=c++17"] + SAN[:4] + ["-c",
                       os.path.join(NATIVE, "abi_sanitize.c"), "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([cc, "--offload-arch=gfx950"] + SAN + objs + [drv, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    with open(stamp, "w") as f:
        f.write(h.hexdigest())
    return exe


def test_abi_host_logic_under_asan_and_ubsan():
    """Validation, dispatch, chunk planning, workspace sizing, overrides and
    the pointer checks over fixed and 20000 pseudo-random descriptors, with
    AddressSanitizer and UndefinedBehaviorSanitizer on the host code: no
    finding, every expectation met ("feat(rocke): channel-packed and
    large-filter depthwise dgrad", the commit hardening the padding and
    lowering error path with a host-only test of it)."""
    exe = _build_sanitized()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0 and res.stdout.startswith("ok "), (res.stdout + res.stderr)[-6000:]
    assert int(res.stdout.split()[1]) > 100000
