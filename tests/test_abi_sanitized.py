"""The ABI's host code (validation, workspace layouts, schedules) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the C ABI translation unit is rebuilt with both
sanitizers on its host side (device code unchanged), linked with the other kernel sources into
a separate library, and driven by tests/sanitize/abi_driver.cpp, whose calls either fail
validation before any launch or compute sizes and schedules only. Any sanitizer report is fatal."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++20", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_code_under_sanitizers(tmp_path):
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, *FLAGS]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip", *HOST_SAN]
        procs.append((subprocess.Popen(cmd + ["-c", src, "-o", obj], stdout=subprocess.PIPE,
                                       stderr=subprocess.PIPE, text=True), src))
        objs.append(obj)
    for p, src in procs:
        out, err = p.communicate()
        assert p.returncode == 0, (src, err[-3000:])
    lib = str(tmp_path / "libh3x_san.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *HOST_SAN, *objs, "-o", lib])
    exe = str(tmp_path / "abi_driver")
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", *HOST_SAN, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, drv, lib, f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
