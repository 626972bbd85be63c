"""The floating-point environment of the step's kernels: compiled with the
library's own flags, the device's fp32 square root and division, fp64 square
root and division, fp64 -> fp32 conversion and an uncontracted multiply-add
must equal the host's IEEE results bit for bit (NaN: both NaN), on random
bit patterns (all exponents, denormals included) and edge cases.  The
arithmetic contract of the step depends on each of them."""
import ctypes
import os

import numpy as np
import pytest

from gpu_common import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "communication_compressed_distributed_02_amd", "libob_mathcheck.so")

N32 = 1 << 25
N64 = 1 << 24

F32_EDGES = np.array([0.0, -0.0, 1.0, -1.0, 2.0, 4.0, 0.25, 1e-45, -1e-45, 1.17549421e-38,
                      1.17549435e-38, 3.4028235e38, -3.4028235e38, np.inf, -np.inf, np.nan,
                      1e-8, 1e-3, 0.999, 0.9, 0.1, 1.0000001, 16777216.0, 16777217.0],
                     dtype=np.float32)


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        raise RuntimeError("libob_mathcheck.so is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    L.ob_mathcheck_run.restype = ctypes.c_int
    L.ob_mathcheck_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return L


def run(L, op, a, b, out_dtype):
    import torch
    ta = torch.from_numpy(a).cuda()
    tb = torch.from_numpy(b).cuda() if b is not None else None
    out = torch.empty(a.size, dtype=out_dtype, device="cuda")
    rc = L.ob_mathcheck_run(op, ta.data_ptr(), tb.data_ptr() if tb is not None else None,
                            out.data_ptr(), a.size, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return out.cpu().numpy()


def same_bits(what, got, want):
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "%s: NaN pattern differs" % what
    ib = np.dtype("u%d" % got.dtype.itemsize)
    bad = np.flatnonzero(got[~nan].view(ib) != want[~nan].view(ib))
    assert bad.size == 0, "%s: %d of %d differ, first %r vs %r" % (
        what, bad.size, got.size, got[~nan][bad[0]], want[~nan][bad[0]])


def f32_inputs(rng, n):
    r = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([F32_EDGES, r])


def f64_inputs(rng, n):
    r = rng.integers(0, np.iinfo(np.uint64).max, size=n, dtype=np.uint64,
                     endpoint=True).view(np.float64)
    return np.concatenate([F32_EDGES.astype(np.float64), r])


def test_fp32_sqrt_and_division(lib):
    rng = np.random.default_rng(11)
    a = f32_inputs(rng, N32)
    with np.errstate(all="ignore"):
        same_bits("sqrtf", run(lib, 0, a, None, __import__("torch").float32), np.sqrt(a))
        b = f32_inputs(rng, N32)[::-1].copy()
        same_bits("fp32 a/b", run(lib, 1, a, b, __import__("torch").float32), a / b)
    log("fp32 sqrt and division: %d inputs each, bit-identical" % a.size)


def test_fp64_sqrt_division_and_conversion(lib):
    import torch
    rng = np.random.default_rng(12)
    a = f64_inputs(rng, N64)
    with np.errstate(all="ignore"):
        same_bits("sqrt", run(lib, 2, a, None, torch.float64), np.sqrt(a))
        b = f64_inputs(rng, N64)[::-1].copy()
        same_bits("fp64 a/b", run(lib, 3, a, b, torch.float64), a / b)
        # conversion: random doubles, and doubles inside the float range near
        # float values and halfway points (ties round to even)
        f = f32_inputs(rng, N64 // 2)
        f = f[np.isfinite(f)].astype(np.float64)
        near = f * (1.0 + rng.uniform(-2 ** -23, 2 ** -23, size=f.size))
        c = np.concatenate([a, near])
        same_bits("(float)double", run(lib, 4, c, None, torch.float32), c.astype(np.float32))
    log("fp64 sqrt, division and conversion: %d inputs, bit-identical" % a.size)


def test_multiply_add_is_not_contracted(lib):
    import torch
    rng = np.random.default_rng(13)
    a = np.concatenate([F32_EDGES, rng.standard_normal(N32).astype(np.float32)])
    b = np.concatenate([F32_EDGES[::-1], rng.standard_normal(N32).astype(np.float32)])
    with np.errstate(all="ignore"):
        want = (a * b) + a
        fused = (a.astype(np.float64) * b + a).astype(np.float32)
    assert np.count_nonzero(want != fused) > 1000  # the inputs tell the two apart
    same_bits("(a*b)+a", run(lib, 5, a, b, torch.float32), want)
