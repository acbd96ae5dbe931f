"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The library's host-side validation: every source is built for gfx950 with
  the sanitizers on its host half only (``-Xarch_host -fsanitize=...``; the
  device code is untouched), linked with ``tests/sanitize/host_validation.c``,
  which calls every entry point with requests that are rejected (or have
  nothing to enqueue) before any HIP call, so no GPU is needed.
* The fp64 oracle (``oracle/gdn2_oracle.c``), serial and threaded, through
  ``tests/sanitize/oracle_checks.c``: every gate kind and both forms, with
  checks that need no stored values (split-and-resume, decay only, the two
  forms under scalar gates, central differences of the reverse pass).

Any sanitizer report fails the run (``halt_on_error``); leaks are reported
too, except one inside the OpenMP runtime's own thread pool.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_decay_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
LLVM = "/opt/rocm/llvm/bin/clang"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]

pytestmark = pytest.mark.skipif(not (os.path.exists(LLVM) and os.path.exists(HIPCC)),
                                reason="needs ROCm's clang and hipcc")


def _env(tmp):
    supp = os.path.join(tmp, "lsan.supp")
    with open(supp, "w") as f:
        f.write("leak:libomp.so\n")
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "3"
    return env


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san"))
    host_san = [x for s in SAN for x in ("-Xarch_host", s)]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    lib = os.path.join(out, "libgdn2_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, *objs, "-o", lib])
    return out


def test_host_validation_under_sanitizers(sanitized_library):
    out = sanitized_library
    exe = os.path.join(out, "host_validation")
    _run([LLVM, "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"),
          os.path.join(HERE, "host_validation.c"), "-L", out, "-lgdn2_san",
          f"-Wl,-rpath,{out}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=_env(out), timeout=300)
    assert "0 failures" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run([LLVM, "-O1", "-g", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "gdn2_oracle.c"),
          os.path.join(HERE, "oracle_checks.c"), "-lm", "-Wl,-rpath,/opt/rocm/llvm/lib", "-o", exe])
    r = _run([exe], env=_env(str(tmp_path)), timeout=300)
    assert "0 failures" in r.stdout
