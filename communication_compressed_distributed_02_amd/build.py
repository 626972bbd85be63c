"""Compile the HIP library libob_adam.so in-tree for gfx950.

Flags that the arithmetic contract depends on: no FMA contraction
(-ffp-contract=off), correctly rounded fp32 division and square root, no
flush of denormals; packed fp32 instructions are disabled.
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libob_adam.so")
SOURCES = [os.path.join(CSRC, f) for f in ("ob_kernels.hip", "ob_adam.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fPIC", "-shared", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


PROBE_LIB = os.path.join(PKG, "libob_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "ob_probe.hip")]


def build(extra_flags=(), out=LIB):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra_flags) + SOURCES + ["-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build_probe(out=PROBE_LIB):
    """Streaming probes used by bench.py for ceilings and counter calibration."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC] + FLAGS + PROBE_SOURCES + ["-o", tmp])
    os.replace(tmp, out)
    return out


MATHCHECK_LIB = os.path.join(PKG, "libob_mathcheck.so")
MATHCHECK_SOURCES = [os.path.join(CSRC, "ob_mathcheck.hip")]


def build_mathcheck(out=MATHCHECK_LIB):
    """Elementwise checks of the step's floating-point environment (tests)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC] + FLAGS + MATHCHECK_SOURCES + ["-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    print(build_probe())
    print(build_mathcheck())
