"""CPU sanitizer builds (no GPU):

* the oracle (``oracle/moe_oracle.c``) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer (every UB report fatal), and its pins run
  against that build in a child process (the wrapper loads the build named
  by MOE_ORACLE_LIB; the ASan runtime is preloaded into the interpreter);
* the C ABI's host validation (``api.hip``, ``plan.hip``)
  compiled host-only (no device code) with the same sanitizers and linked
  against stub launchers (``tests/sanitize/host_validation.cpp``), which
  drive every rejection path, the workspace-size functions over a range of
  sizes and the extreme int64 / int32 arguments.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "permutation_group_limited_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
UBSAN_OPTS = "halt_on_error=1:print_stacktrace=1"


def _gcc_runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="moe_sanitize_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_runtime("libasan.so") is None,
                    reason="gcc with AddressSanitizer not available")
def test_oracle_pins_under_asan_ubsan(tmpdir_mod):
    lib = os.path.join(tmpdir_mod, "libmoe_oracle_asan.so")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", lib, os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env.update({"MOE_ORACLE_LIB": lib, "LD_PRELOAD": _gcc_runtime("libasan.so"),
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": UBSAN_OPTS, "OMP_NUM_THREADS": "2"})
    tests = [os.path.join(ROOT, "tests", t) for t in (
        "test_oracle_router.py", "test_oracle_indices.py", "test_oracle_finalize.py",
        "test_oracle_dtypes.py", "test_oracle_scorefn.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + tests, env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_asan_ubsan(tmpdir_mod):
    exe = os.path.join(tmpdir_mod, "host_validation")
    srcs = [os.path.join(CSRC, s) for s in ("api.hip", "plan.hip")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "host_validation.cpp"))
    cmd = [HIPCC, "--offload-host-only", "-x", "hip", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer", "-fno-gpu-sanitize",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + ["-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ)
    env.update({"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": UBSAN_OPTS})
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host validation ok" in r.stdout
    assert "runtime error" not in out, out[-4000:]
