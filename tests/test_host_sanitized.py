"""The library's host code (argument validation, shape rules, workspace
carve-up, checkpoint counters) built with AddressSanitizer and
UndefinedBehaviorSanitizer runs the CPU interface tests cleanly.  Only host
code is instrumented (each sanitizer flag applies to the host pass); no GPU
is touched: every call here is rejected or answered before any HIP call."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "communication_compressed_distributed_02_amd")


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_interface_checks_pass_under_asan_and_ubsan():
    sys.path.insert(0, PKG)
    import build as libbuild
    runtime = _clang_asan_runtime()
    if runtime is None or not os.path.exists(libbuild.HIPCC):
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "libob_adam_san.so")
        libbuild.build(extra_flags=san, out=so)
        log = os.path.join(tmp, "san")
        env = dict(os.environ, OB_ADAM_TEST_LIB=so, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:log_path=" + log,
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:log_path=" + log)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        reports = "".join(open(os.path.join(tmp, f)).read()[:3000] for f in os.listdir(tmp)
                          if f.startswith("san"))
        out = r.stdout[-3000:] + r.stderr[-3000:] + reports
        assert r.returncode == 0, out
        assert "passed" in r.stdout and "skipped" not in r.stdout, out
        assert not reports, out
