"""CPU: the oracle and the library's host-side code under AddressSanitizer
and UndefinedBehaviorSanitizer.

Each test builds an instrumented copy of a library into a temporary folder
and runs the CPU tests that exercise it in a child process with the
sanitizer runtime preloaded (any report aborts the child):

  - the oracle (gcc, -fsanitize=address,undefined) under the oracle pins and
    the input-guard tests;
  - the HIP library with its host code instrumented (hipcc, each sanitizer
    flag applied to the host pass only; device code is built as usual) under
    the C-ABI tests, which drive every host-side argument check, workspace
    sizing and status path without touching a GPU.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
HIP_SOURCES = ["heads.hip", "tree_attention.hip", "tree_accept.hip", "tree_commit.hip",
               "forward.hip", "probes.hip"]


def _child(tests, env_extra, marker_lib):
    """Run pytest on `tests` in a child with env_extra; the child also checks
    that the instrumented library is the one it loaded."""
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env.pop("PYTEST_ADDOPTS", None)
    res = subprocess.run([sys.executable, "-m", "pytest", *tests, "-x", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=1200)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "Sanitizer" not in out, out
    probe = ("import sys; sys.path.insert(0, %r); import oracle; "
             "from medusa_tree_verification_amd import binding as b; oracle.lib(); "
             "import os; p = os.environ.get('MEDUSA_VERIFY_TEST_LIB'); L = b._load(p) if p else None; "
             "m = open('/proc/self/maps').read(); print('LOADED' if %r in m else 'MISSING')"
             % (ROOT, os.path.basename(marker_lib)))
    res = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert "LOADED" in res.stdout, res.stdout + res.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "libmedusa_oracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib,
                           os.path.join(ROOT, "oracle", "medusa_oracle.c"), "-lm"])
    rt = [subprocess.check_output([gcc, f"-print-file-name={n}"], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    _child(["tests/test_oracle_pins.py", "tests/test_guards.py"],
           {"MEDUSA_ORACLE_LIB": lib, "LD_PRELOAD": ":".join(rt)}, lib)


def test_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rts:
        pytest.skip("hipcc or the clang sanitizer runtime not found")
    lib = str(tmp_path / "libmedusa_verify_san.so")
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", f]
    csrc = os.path.join(ROOT, "medusa_tree_verification_amd", "csrc")
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                           "-shared", *host, "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           "-o", lib, *[os.path.join(csrc, s) for s in HIP_SOURCES]],
                          stderr=subprocess.DEVNULL, timeout=1800)
    _child(["tests/test_abi.py"], {"MEDUSA_VERIFY_TEST_LIB": lib, "LD_PRELOAD": rts[-1]}, lib)
