"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two small programs are built for the CPU with the sanitizers and run:
  * tests/sanitize/plan_driver.cpp links the host part of libgdn (gdn_api.hip; the sanitizers
    instrument its host code only) with stub kernel launchers: a sweep of the AutoCP planner and the workspace
    layout over uniform and packed shapes, every documented argument error, and the forward's
    launch sequence;
  * tests/sanitize/oracle_driver.c runs the CPU oracle's forward and reverse mode on packed
    batches with empty, one-token and ragged sequences.
Any sanitizer report aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_04_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
# host code only (no device code is compiled), so the sanitizers apply to the host program
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_planner_under_sanitizers(tmp_path):
    hip = ["-x", "hip", "--offload-arch=gfx950", "--rocm-path=/opt/rocm", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    # the sanitizers instrument the host code only (-Xarch_host before each); gdn_api.hip's one
    # device object (the fixed scratch array) is compiled for gfx950 as usual
    host_san = [x for f in SAN_FLAGS for x in (["-Xarch_host", f] if f.startswith("-fsanitize") else [f])]
    objs = []
    for src in (os.path.join(CSRC, "gdn_api.hip"), os.path.join(SAN, "stubs.cpp"), os.path.join(SAN, "plan_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([CLANG, *hip, *host_san, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "plan_driver")
    _run([CLANG, *SAN_FLAGS, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    print(r.stdout.strip())
    assert r.stdout.startswith("ok"), r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN_FLAGS, os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    print(r.stdout.strip())
    assert r.stdout.startswith("ok"), r.stdout
