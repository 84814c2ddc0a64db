"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.hip (argument validation, workspace layout, status strings, the
per-device scratch set-up) is rebuilt with the sanitizers on its host code
only, linked with the other translation units of the in-tree build, and the
CPU ABI tests (tests/test_abi.py) run against that library in a child
process with the sanitizer runtime preloaded.  No GPU is used: every call in
those tests fails validation before any HIP call that needs a device.  Any
sanitizer report aborts the child and fails this test.
"""

import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from transformer_head_self_amd import _build  # noqa: E402


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_tests_pass_under_sanitizers():
    rt = _asan_runtime()
    objs = [os.path.join(_build.BUILD_DIR, os.path.splitext(s)[0] + ".o")
            for s in _build.SOURCES if s != "api.hip"]
    if rt is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("the HIP toolchain or its sanitizer runtime is not installed")
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.skip(f"build the library first (missing {missing[0]})")
    hipcc = _build._hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as d:
        api_o = os.path.join(d, "api.o")
        lib = os.path.join(d, "libmha_sanitized.so")
        flags = [f for f in _build.FLAGS if f != "-O3"]
        res = subprocess.run([hipcc, "-O1", "-g", *flags, *san, "-c",
                              os.path.join(_build.CSRC, "api.hip"), "-o", api_o],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        res = subprocess.run([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", *san,
                              "-o", lib, api_o, *objs], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        env = dict(os.environ)
        env.update({
            "LD_PRELOAD": rt,
            "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:verbosity=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
            "TRANSFORMER_HEAD_SELF_AMD_LIB": lib,
        })
        res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                              os.path.join(ROOT, "tests", "test_abi.py")],
                             capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
        out = res.stdout + res.stderr
        assert res.returncode == 0, out[-4000:]
        assert "AddressSanitizer" in out            # the runtime was live in the child
        assert "runtime error" not in out           # no UBSan report
        assert " passed" in res.stdout and " failed" not in res.stdout
