"""The planners and the ABI's host logic under AddressSanitizer and UBSan.

The library's sources are compiled with -fsanitize=address,undefined and no
recovery on their host side only (the device code is built as usual and never
launched: no GPU is touched), linked with
tests/asan/host_driver.cpp, and run: any out-of-bounds access, leak or
undefined behaviour in the planners, the workspace sizing or the argument
checks aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_optimizer_step_02_amd", "csrc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.timeout(600)
def test_host_logic_is_clean_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    common = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC] + SAN
    objs = []
    procs = []
    for s in srcs + [os.path.join(ROOT, "tests", "asan", "host_driver.cpp")]:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        cmd = [hipcc, "-x", "hip"] + common + ["-c", s, "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(o)
    for s, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"compile {s}:\n{out}{err}"
    exe = str(tmp_path / "host_driver")
    link = [hipcc, "--offload-arch=gfx950", "-o", exe] + objs + SAN
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "0 failures" in r.stdout, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
