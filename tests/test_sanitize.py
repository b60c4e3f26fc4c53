"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU calls).

* oracle/lt2_oracle.c with gcc -fsanitize=address,undefined, driven by
  tests/sanitize/oracle_driver.c: prefill, decode and backward of both gates on
  small seeded inputs, ragged lengths, degenerate and invalid sizes.
* every HIP source of the library with its host code sanitized (the GPU code
  is compiled as usual), driven by tests/sanitize/abi_driver.c through the C
  ABI: only calls that the host validation refuses, or that have nothing to
  do, so nothing is launched.
Any sanitizer report makes the driver exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-fopenmp", *SAN, "-o", exe, os.path.join(HERE, "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "lt2_oracle.c"), "-lm"])
    out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2"))
    assert "oracle driver: ok" in out


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not found")
def test_host_validation_under_sanitizers(tmp_path):
    from concurrent.futures import ThreadPoolExecutor

    from linear_attention_looped_amd import build as libbuild
    csrc = libbuild.CSRC
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    # host sanitizers only: each -fsanitize= is preceded by -Xarch_host
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]
    flags = [f for f in libbuild.cflags() if f != "-O3"] + ["-O1", *host_san]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([libbuild.hipcc(), *flags, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    clang = "/opt/rocm/llvm/bin/clang"
    drv = str(tmp_path / "abi_driver.o")
    run([clang, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "abi_driver.c"),
         "-o", drv])
    exe = str(tmp_path / "abi_driver")
    run([clang + "++", *SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime's own allocations at exit are not this library's
    out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi driver: ok" in out
