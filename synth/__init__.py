"""Seeded synthetic gradients, bit-identical on the host and the GPU.

This module generates inputs only; it holds none of the optimizer's
arithmetic.  The counter-based generator is defined in philox.h; synth_cpu.c
and synth_gpu.hip are its host and device builds.  The GPU build is loaded
only when a GPU fill is requested.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

NORMAL = 0
STUDENT_T3 = 1
SEED = 1234

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
             "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fPIC", "-shared"]


def _atomic_build(cmd, out):
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(cmd + ["-o", tmp])
    os.replace(tmp, out)


def build_cpu():
    _atomic_build(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                   "-shared", "-Wall", os.path.join(_HERE, "synth_cpu.c"), "-lm"], CPU_LIB)


def build_gpu():
    _atomic_build([HIPCC] + HIP_FLAGS + [os.path.join(_HERE, "synth_gpu.hip")], GPU_LIB)


def build():
    build_cpu()
    build_gpu()


def normal_k(sigma):
    """fp32 factor that turns the centred Irwin-Hall integer into N(0, sigma)."""
    return np.float32(sigma * math.sqrt(3.0) / 2.0 ** 25)


def dist_params(dist, sigma):
    """(k, sigma) arguments of the generator for a distribution."""
    if dist == NORMAL:
        return normal_k(sigma), np.float32(1.0)
    return normal_k(1.0), np.float32(sigma)


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            build_cpu()
        L = ctypes.CDLL(CPU_LIB)
        L.synth_philox_block.argtypes = [ctypes.c_uint32] * 6 + [ctypes.POINTER(ctypes.c_uint32)]
        L.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                 ctypes.c_float, ctypes.c_float]
        L.synth_gather.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_float]
        _cpu = L
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        import torch  # noqa: F401  (the HIP runtime must be torch's, loaded first)
        if not os.path.exists(GPU_LIB):
            raise RuntimeError("synth GPU library not built: run __graft_entry__.build()")
        L = ctypes.CDLL(GPU_LIB)
        L.synth_fill_device.restype = ctypes.c_int
        L.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_void_p]
        _gpu = L
    return _gpu


def philox_block(c, k):
    out = (ctypes.c_uint32 * 4)()
    _cpu_lib().synth_philox_block(*(list(c) + list(k)), out)
    return list(out)


def fill_cpu(count, elem0, step, worker, dist=NORMAL, sigma=1e-2, bf16=False, seed=SEED):
    """Gradient of `worker` at `step` for elements [elem0, elem0+count)."""
    k, s = dist_params(dist, sigma)
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    _cpu_lib().synth_fill(out.ctypes.data, 1 if bf16 else 0, count, elem0, step, seed, worker,
                          dist, k, s)
    return out


def gather_cpu(elems, step, worker, dist=NORMAL, sigma=1e-2, bf16=False, seed=SEED):
    elems = np.ascontiguousarray(elems, dtype=np.uint64)
    k, s = dist_params(dist, sigma)
    out = np.empty(elems.size, dtype=np.uint16 if bf16 else np.float32)
    _cpu_lib().synth_gather(out.ctypes.data, 1 if bf16 else 0, elems.size, elems.ctypes.data,
                            step, seed, worker, dist, k, s)
    return out


def fill_gpu(tensor, elem0, step, worker, dist=NORMAL, sigma=1e-2, seed=SEED, stream=None):
    """Fill a contiguous device tensor (float32, or int16/bfloat16 for bf16)."""
    import torch
    if not tensor.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if tensor.dtype == torch.float32:
        dt = 0
    elif tensor.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        dt = 1
    else:
        raise TypeError("unsupported dtype %s" % tensor.dtype)
    k, s = dist_params(dist, sigma)
    if stream is None:
        stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _gpu_lib().synth_fill_device(tensor.data_ptr(), dt, tensor.numel(), elem0, step, seed,
                                      worker, dist, k, s, stream)
    if rc != 0:
        raise RuntimeError("synth_fill_device failed (%d)" % rc)
