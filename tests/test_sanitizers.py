"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two instrumented builds, each in a temporary directory:

* the oracle (oracle/moe_oracle.c) with gcc, -fsanitize=address,undefined;
  the oracle's own pin and layer tests then run against it;
* libmoe with the sanitizers on its host code only (hipcc's device code is
  built as usual) and MOE_DEBUG's host-side index checks compiled in; the
  ABI tests then run against it: workspace sizing, argument validation,
  every error path that returns before a HIP call, and moe_check_buckets.

Each suite runs in a child process with the sanitizer runtime preloaded,
halting on the first report; the child also checks that the instrumented
library, not the regular one, is the one it loaded.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routed_expert_ffn_router_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")

# the child: point the package at the instrumented library, run the suites,
# and fail unless that library is the one loaded
CHILD = """
import sys
sys.path.insert(0, {root!r})
import {pkg} as m
m.LIB_PATH = {lib!r}
import pytest
rc = pytest.main([*{tests!r}, "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"])
loaded = m.lib()._name
assert loaded == {lib!r}, loaded
sys.exit(rc)
"""


def _exports(lib):
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    return out


def _run_child(pkg, lib, tests, preload, tmp):
    script = os.path.join(tmp, f"run_{pkg}.py")
    with open(script, "w") as fh:
        fh.write(CHILD.format(root=ROOT, pkg=pkg, lib=lib, tests=tests))
    env = dict(ENV, LD_PRELOAD=preload)
    r = subprocess.run([sys.executable, script], capture_output=True, text=True, env=env,
                       cwd=tmp, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    preload = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(preload) or not os.path.exists(preload):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
         "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "moe_oracle.c"),
         "-o", lib, "-lm"])
    syms = _exports(lib)
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    tests = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
             os.path.join(ROOT, "tests", "test_oracle_layer.py")]
    _run_child("oracle", lib, tests, preload, str(tmp_path))


def test_libmoe_host_code_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    # MOE_DEBUG: the host-side index checks are compiled in (and under the
    # sanitizers) as well
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
             "-DMOE_DEBUG",
             "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, *san, "-c", src, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out.decode()[-3000:]
    lib = str(tmp_path / "libmoe_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san,
                           "-shared-libsan", *objs, "-o", lib])
    syms = _exports(lib)
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    _run_child("routed_expert_ffn_router_amd", lib, [os.path.join(ROOT, "tests", "test_abi.py")],
               rt[-1], str(tmp_path))
