"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only) runs the pin suite cleanly: no out-of-bounds access, overflow or
other undefined behaviour in the reference the GPU path is checked against."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "libob_oracle_san.so")
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                               "-o", so, os.path.join(ROOT, "oracle", "ob_oracle.c"), "-lm"])
        log = os.path.join(tmp, "san")
        env = dict(os.environ, OB_ORACLE_LIB=so, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:log_path=" + log,
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:log_path=" + log)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        reports = "".join(open(os.path.join(tmp, f)).read()[:3000] for f in os.listdir(tmp)
                          if f.startswith("san"))
        out = r.stdout[-3000:] + r.stderr[-3000:] + reports
        assert r.returncode == 0, out
        assert not reports, out
