"""CPU sanitizer builds: AddressSanitizer and UndefinedBehaviorSanitizer over
the oracle and the library's host code.

* driver_oracle.cpp with oracle/spec_oracle.c, the depth planner and the
  status strings, built with gcc/g++ (leak checking on): Philox, softmax,
  accept/reject in every mode and edge case, every planted mistake, argument
  rejection, the planner.
* driver_host.cpp with every library source, built with hipcc, the
  sanitizers on the host side only: the host-side argument validation of
  every entry point (each call is refused before any launch, so no GPU is
  needed; leak checking is off because the HIP runtime's own allocations
  outlive main).

A sanitizer report fails the build's run, and so fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verification_accept_amd", "csrc")
INC = os.path.join(ROOT, "include")
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return res.returncode, res.stdout + res.stderr


def _clean(out):
    return "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out


def test_oracle_and_planner_under_asan_ubsan(tmp_path):
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not gcc or not gxx:
        pytest.skip("gcc/g++ not available")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-O1", "-g"]
    obj = str(tmp_path / "oracle.o")
    rc, out = _run([gcc, *san, "-c", os.path.join(ROOT, "oracle", "spec_oracle.c"), "-o", obj])
    assert rc == 0, out
    exe = str(tmp_path / "drv_oracle")
    rc, out = _run([gxx, *san, "-std=c++17", "-ffp-contract=off", "-I", INC,
                    os.path.join(SAN_DIR, "driver_oracle.cpp"), os.path.join(CSRC, "spec_plan.cpp"),
                    os.path.join(CSRC, "api.cpp"), obj, "-o", exe, "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1"})
    assert rc == 0 and _clean(out), out
    assert "all checks passed" in out


def test_host_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/lib/llvm/bin/clang++"
    if not os.path.exists(hipcc) or not os.path.exists(clangxx):
        pytest.skip("hipcc / ROCm clang++ not available")
    objs, procs = [], []
    for src in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.splitext(src)[0] + "_san.o"))
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
                   "-I", INC, "-I", CSRC, "-c", path, "-o", obj]
        elif src.endswith(".cpp"):
            cmd = [hipcc, "-x", "c++", "-O1", "-g", "-std=c++17", *HOST_SAN, "-I", INC, "-c", path,
                   "-o", obj]
        else:
            objs.pop()
            continue
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    drv = str(tmp_path / "driver_host_san.o")
    procs.append(subprocess.Popen([hipcc, "-x", "c++", "-O1", "-g", "-std=c++17", *HOST_SAN, "-I", INC, "-c",
                                   os.path.join(SAN_DIR, "driver_host.cpp"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out
    exe = str(tmp_path / "drv_host")
    rc, out = _run([clangxx, "-fsanitize=address,undefined", *objs, drv, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"})
    assert rc == 0 and _clean(out), out
    assert "all checks passed" in out
