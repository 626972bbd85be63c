"""CPU oracle for the compression-phase step of 1-bit Adam (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use it; the product package never imports it.  The C
source (ob_oracle.c) states what the step computes and which passage of the
pages each part follows.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libob_oracle.so")
# The mutation test of the pins points this at deliberately broken builds.
_LOAD_PATH = os.environ.get("OB_ORACLE_LIB", LIB_PATH)

X, M, V, E_WORKER, E_SERVER, C_WORKER, U_SERVER, A_SERVER = range(8)
BITS_WORKER, BITS_SERVER, SCALE_WORKER, SCALE_SERVER = 8, 9, 10, 11
M_LOCAL, A_LOCAL, X_LOCAL = 12, 13, 14  # 0/1 Adam

_FLOAT_FIELDS = {X, M, V, E_WORKER, E_SERVER, C_WORKER, U_SERVER, A_SERVER,
                 SCALE_WORKER, SCALE_SERVER, M_LOCAL, A_LOCAL, X_LOCAL}


def build(force=True):
    """Compile the oracle: gcc -O2 -ffp-contract=off (no fast-math, no FTZ)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-Wall", "-o", tmp, os.path.join(_HERE, "ob_oracle.c"), "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LOAD_PATH == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(_LOAD_PATH)
        L.ob_oracle_create.restype = ctypes.c_void_p
        L.ob_oracle_create.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_int32]
        L.ob_oracle_destroy.argtypes = [ctypes.c_void_p]
        for f in (L.ob_oracle_warmup_step, L.ob_oracle_compressed_step):
            f.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                          ctypes.c_float]
        L.ob_oracle_zo_step.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
                                        ctypes.c_int32]
        L.ob_oracle_zo_gamma.restype = ctypes.c_float
        L.ob_oracle_zo_gamma.argtypes = [ctypes.c_void_p]
        L.ob_oracle_zo_open.restype = ctypes.c_int32
        L.ob_oracle_zo_open.argtypes = [ctypes.c_void_p]
        L.ob_oracle_field.restype = ctypes.c_void_p
        L.ob_oracle_field.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64)]
        L.ob_oracle_step.restype = ctypes.c_int64
        L.ob_oracle_step.argtypes = [ctypes.c_void_p]
        L.ob_oracle_held.restype = ctypes.c_int64
        L.ob_oracle_held.argtypes = [ctypes.c_void_p]
        L.ob_oracle_chunk_sumsq.restype = ctypes.c_double
        L.ob_oracle_chunk_sumsq.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.ob_oracle_chunk_scale.restype = ctypes.c_float
        L.ob_oracle_chunk_scale.argtypes = [ctypes.c_double, ctypes.c_int64]
        L.ob_oracle_pairwise_mean.restype = ctypes.c_float
        L.ob_oracle_pairwise_mean.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        _lib = L
    return _lib


def chunk_sumsq(c):
    c = np.ascontiguousarray(c, dtype=np.float32)
    return lib().ob_oracle_chunk_sumsq(c.ctypes.data, c.size)


def chunk_scale(sumsq, length):
    return np.float32(lib().ob_oracle_chunk_scale(sumsq, length))


def pairwise_mean(vals):
    v = np.ascontiguousarray(vals, dtype=np.float32)
    return np.float32(lib().ob_oracle_pairwise_mean(v.ctypes.data, v.size))


class Oracle:
    """One oracle instance holding chunks [j0, j1) of a d-vector, n workers."""

    def __init__(self, d, n, beta1=0.9, beta2=0.999, eps=1e-8, j0=0, j1=None, keep_debug=True):
        j1 = n if j1 is None else j1
        self.d, self.n, self.j0, self.j1 = d, n, j0, j1
        self.L = d // n
        self._h = lib().ob_oracle_create(d, n, j0, j1, beta1, beta2, eps, 1 if keep_debug else 0)
        if not self._h:
            raise ValueError("oracle: bad arguments (d=%d n=%d j0=%d j1=%d)" % (d, n, j0, j1))
        self.cnt = lib().ob_oracle_held(self._h)

    def close(self):
        if self._h:
            lib().ob_oracle_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _grad_ptrs(self, grads):
        arrs = []
        dtype = None
        for g in grads:
            g = np.ascontiguousarray(g)
            if g.dtype == np.float32:
                dt = 0
            elif g.dtype == np.uint16:
                dt = 1
            else:
                raise TypeError("grads must be float32 or uint16 (bf16 bits)")
            if dtype is not None and dt != dtype:
                raise TypeError("mixed gradient dtypes")
            if g.size != self.cnt:
                raise ValueError("gradient has %d elements, oracle holds %d" % (g.size, self.cnt))
            dtype = dt
            arrs.append(g)
        if len(arrs) != self.n:
            raise ValueError("need %d gradients" % self.n)
        ptrs = (ctypes.c_void_p * self.n)(*[a.ctypes.data for a in arrs])
        return arrs, ptrs, dtype

    def warmup_step(self, grads, lr):
        keep, ptrs, dt = self._grad_ptrs(grads)
        lib().ob_oracle_warmup_step(self._h, ptrs, dt, lr)
        del keep

    def compressed_step(self, grads, lr):
        keep, ptrs, dt = self._grad_ptrs(grads)
        lib().ob_oracle_compressed_step(self._h, ptrs, dt, lr)
        del keep

    def zo_step(self, grads, lr, sync, refresh=False):
        """One 0/1 Adam step (see ob_oracle_zo_step)."""
        if refresh and not sync:
            raise ValueError("the variance is refreshed only at a synchronizing step")
        keep, ptrs, dt = self._grad_ptrs(grads)
        lib().ob_oracle_zo_step(self._h, ptrs, dt, lr, 1 if sync else 0, 1 if refresh else 0)
        del keep

    @property
    def zo_gamma(self):
        """Sum of the step sizes of the open local period (fp32)."""
        return np.float32(lib().ob_oracle_zo_gamma(self._h))

    @property
    def zo_open(self):
        """Local steps taken in the open period (0 right after a synchronization)."""
        return lib().ob_oracle_zo_open(self._h)

    def _view(self, field, worker=0):
        cnt = ctypes.c_int64(0)
        p = lib().ob_oracle_field(self._h, field, worker, ctypes.byref(cnt))
        if not p:
            raise ValueError("field %d not kept (keep_debug=False?)" % field)
        if field in _FLOAT_FIELDS:
            ct = ctypes.c_float
            dt = np.float32
        else:
            ct = ctypes.c_uint64
            dt = np.uint64
        buf = (ct * cnt.value).from_address(p)
        return np.frombuffer(buf, dtype=dt)

    def get(self, field, worker=0):
        """Copy of a field (see the OBO_* list in ob_oracle.h)."""
        return self._view(field, worker).copy()

    def set(self, field, values, worker=0):
        """Overwrite a state field in place (tests use this to pose a state)."""
        view = self._view(field, worker)
        view[:] = np.asarray(values, dtype=view.dtype).reshape(view.shape)

    @property
    def step(self):
        return lib().ob_oracle_step(self._h)
