"""The host code of libtq under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The library's sources are built with both sanitizers on their
host side (their device code unoptimised: it is never run here) and linked
with tests/host_sanitize/check_host.c, which calls every exported entry
point on valid and malformed host arguments that are answered before any
device work.  Any sanitizer report, or a failed check, fails the test."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_paged_kv_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SOURCES = ["tq_host.cpp", "write_kv.hip", "decode.hip", "window.hip", "qjl.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm compilers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-x", "hip", "-g0", "-fPIC", "-std=c++17", "-Xarch_host", "-O1",
             "-Xarch_device", "-O0", *SAN, "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for src, p in zip(SOURCES, procs):
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}: {out[-2000:]}"
    drv = str(tmp_path / "check_host.o")
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "host_sanitize", "check_host.c"), "-o", drv],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "check_host")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, drv, *objs],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
