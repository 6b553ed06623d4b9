"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/arp_oracle.c) built with both sanitizers, leak checking
  on, and driven by tests/sanitize/oracle_checks.c over every flag, both io
  dtypes, shared and per-head angles, one-token and ragged lengths, gates and
  per-head query multipliers.
* The library's host code (csrc/api.hip: descriptor checks, sizes, argument
  validation, the AdaScale schedule) compiled with both sanitizers on its host
  side only and linked with the library's other objects into
  tests/sanitize/abi_checks.cpp, whose calls are host-only or fail validation
  before anything is enqueued (no GPU is used).

Any sanitizer report aborts the program (-fno-sanitize-recover=all), which
fails the test with the report in the message."""
import glob
import os
import shutil
import subprocess

import pytest

from accumulated_rotation_positional_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
# host-side instrumentation only: each option applies to the host compilation
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-8000:]}"
    return r


def _env(leaks: bool):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", *SAN, "-fopenmp", os.path.join(HERE, "oracle_checks.c"),
          os.path.join(ROOT, "oracle", "arp_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=_env(leaks=True))
    assert "oracle checks passed" in r.stdout


@pytest.mark.skipif(not (os.path.exists(hip_build.HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    objs = {os.path.basename(p): p for p in glob.glob(os.path.join(hip_build.BUILD, "*.o"))}
    need = [s.replace(".hip", ".o") for s in hip_build.SOURCES]
    if not all(n in objs for n in need):
        hip_build.build()
        objs = {os.path.basename(p): p for p in glob.glob(os.path.join(hip_build.BUILD, "*.o"))}
    api = str(tmp_path / "api_san.o")
    _run([hip_build.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={hip_build.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
          "-c", os.path.join(hip_build.CSRC, "api.hip"), "-o", api])
    drv = str(tmp_path / "abi_checks.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", *SAN, "-c", os.path.join(HERE, "abi_checks.cpp"),
          "-o", drv])
    exe = str(tmp_path / "abi_checks")
    rest = [objs[n] for n in need if n != "api.o"]
    _run([CLANG, *SAN, api, drv, *rest, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", exe])
    # leak checking off: the HIP runtime's own allocations at exit are not ours
    r = _run([exe], env=_env(leaks=False))
    assert "abi checks passed" in r.stdout
