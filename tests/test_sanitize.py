"""AddressSanitizer + UndefinedBehaviorSanitizer builds, CPU only:

- the oracle's C code (plain gcc), driven by tests/sanitize/oracle_main.c: Philox
  known answers, noise and head estimators on ragged and empty shapes;
- the library's host code (hipcc, sanitizers on the host pass only; device code is
  built as usual), driven by tests/sanitize/capi_main.c: the host-side argument
  checks of every entry point and the size queries, with no GPU present.

A sanitizer finding aborts the driver, which fails the test."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_c_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-D_DEFAULT_SOURCE", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_main.c"),
          os.path.join(ROOT, "oracle", "dust_oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    out = _run([exe, os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.txt")], env=env, timeout=120)
    assert out.strip() == "ok"


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_library_host_checks_under_sanitizers(tmp_path):
    from zeroth_order_activation_amd import build as B
    flags = ["-O1", "-g", "-std=c++17", f"--offload-arch={B.ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", B.INCLUDE, "-I", B.CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        _run([B.HIPCC, *flags, *HOST_SAN, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))))
    clang = "/opt/rocm/bin/amdclang"
    main_o = str(tmp_path / "capi_main.o")
    _run([clang, "-std=c99", "-g", "-fsanitize=address,undefined", "-I", B.INCLUDE, "-c",
          os.path.join(SAN, "capi_main.c"), "-o", main_o])
    exe = str(tmp_path / "capi_san")
    _run([clang + "++", "-fsanitize=address,undefined", main_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # the HIP runtime keeps allocations to the end of the process: leaks are not checked
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([exe], env=env, timeout=300)
    assert out.strip() == "ok"
