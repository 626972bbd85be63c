"""Python binding of libob_adam.so (argument marshalling only).

Functions carry the names of the C interface in include/ob_adam.h and raise
ObAdamError on a status other than OB_OK.  Every step of the computation runs
in the library's HIP kernels; PyTorch only provides device memory and the
stream.  There is no fallback: if the library is missing, importing this
module fails.
"""
import ctypes
import os

import torch  # loads the HIP runtime the library binds to

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libob_adam.so")

(OB_OK, OB_ERR_ARG, OB_ERR_SHAPE, OB_ERR_PHASE, OB_ERR_WORKSPACE, OB_ERR_HIP,
 OB_ERR_TOO_LARGE) = range(7)
OB_GRAD_F32, OB_GRAD_BF16 = 0, 1
(OB_X, OB_M, OB_V, OB_E_WORKER, OB_E_SERVER, OB_BITS_WORKER, OB_BITS_SERVER, OB_SCALE_WORKER,
 OB_SCALE_SERVER, OB_M_LOCAL, OB_A_LOCAL, OB_X_LOCAL) = range(12)
OB_METHOD_ONE_BIT, OB_METHOD_ZERO_ONE = 0, 1
OB_ZO_SYNC, OB_ZO_REFRESH = 1, 2

EXPORTED = ("ob_adam_workspace_bytes", "ob_adam_init", "ob_adam_warmup_step",
            "ob_adam_warmup_worker", "ob_adam_warmup_finish",
            "ob_adam_compressed_step", "ob_adam_compressed_step_static", "ob_adam_zero_one_step",
            "ob_adam_compress_worker", "ob_adam_compressed_finish",
            "ob_adam_get_state", "ob_adam_set_state", "ob_adam_params", "ob_adam_step_count",
            "ob_adam_get_counters", "ob_adam_attach", "ob_adam_check_guards", "ob_adam_set_debug",
            "ob_adam_set_timing",
            "ob_adam_kernel_times", "ob_adam_destroy", "ob_status_str")
KERNELS = ("warmup", "worker", "worker_scale", "server", "server_scale", "update", "zo_local",
           "zo_refresh")


class ObAdamError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, ob_status_str(status), status))


class ob_adam_config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("n_workers", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float), ("method", ctypes.c_int32)]


class ob_adam_counters(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("compressed_steps", ctypes.c_int64),
                ("warmup_steps", ctypes.c_int64)]


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError("libob_adam.so is not built (run __graft_entry__.build()): " + path)
    L = ctypes.CDLL(path)
    P, I32, I64, U64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    cfgp = ctypes.POINTER(ob_adam_config)
    sig = {
        "ob_adam_workspace_bytes": [cfgp, ctypes.POINTER(U64)],
        "ob_adam_init": [cfgp, P, U64, P, P, ctypes.POINTER(P)],
        "ob_adam_warmup_step": [P, ctypes.POINTER(P), F],
        "ob_adam_compressed_step": [P, ctypes.POINTER(P), F],
        "ob_adam_compressed_step_static": [P, ctypes.POINTER(P), F],
        "ob_adam_zero_one_step": [P, ctypes.POINTER(P), F, I32],
        "ob_adam_warmup_worker": [P, I32, P],
        "ob_adam_warmup_finish": [P, F],
        "ob_adam_compress_worker": [P, I32, P],
        "ob_adam_compressed_finish": [P, F],
        "ob_adam_get_state": [P, I32, I32, I64, I64, P],
        "ob_adam_set_state": [P, I32, I64, I64, P],
        "ob_adam_params": [P, ctypes.POINTER(P)],
        "ob_adam_get_counters": [P, ctypes.POINTER(ob_adam_counters)],
        "ob_adam_attach": [cfgp, P, U64, ctypes.POINTER(ob_adam_counters), P, ctypes.POINTER(P)],
        "ob_adam_check_guards": [P, ctypes.POINTER(I32)],
        "ob_adam_set_debug": [P, I32],
        "ob_adam_step_count": [P, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "ob_adam_set_timing": [P, I32],
        "ob_adam_kernel_times": [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64),
                                 ctypes.POINTER(I64)],
        "ob_adam_destroy": [P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.ob_status_str.argtypes = [ctypes.c_int]
    L.ob_status_str.restype = ctypes.c_char_p
    return L


_lib = _load()


def _check(status, where):
    if status != OB_OK:
        raise ObAdamError(status, where)


def ob_status_str(status):
    return _lib.ob_status_str(status).decode()


def make_config(d, n_workers, grad_dtype=OB_GRAD_F32, beta1=0.9, beta2=0.999, eps=1e-8,
                method=OB_METHOD_ONE_BIT):
    return ob_adam_config(d, n_workers, grad_dtype, beta1, beta2, eps, method)


def ob_adam_workspace_bytes(cfg):
    out = ctypes.c_uint64(0)
    _check(_lib.ob_adam_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)),
           "ob_adam_workspace_bytes")
    return out.value


def ob_adam_init(cfg, workspace_ptr, ws_bytes, x0_ptr, stream_ptr):
    h = ctypes.c_void_p(0)
    _check(_lib.ob_adam_init(ctypes.byref(cfg), workspace_ptr, ws_bytes, x0_ptr, stream_ptr,
                             ctypes.byref(h)), "ob_adam_init")
    return h.value


def _ptr_array(ptrs):
    if isinstance(ptrs, ctypes.Array):  # marshalled already (GradBatch)
        return ptrs
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def ob_adam_warmup_step(h, grad_ptrs, lr):
    _check(_lib.ob_adam_warmup_step(h, _ptr_array(grad_ptrs), lr), "ob_adam_warmup_step")


def ob_adam_warmup_worker(h, worker, grad_ptr):
    _check(_lib.ob_adam_warmup_worker(h, worker, grad_ptr), "ob_adam_warmup_worker")


def ob_adam_warmup_finish(h, lr):
    _check(_lib.ob_adam_warmup_finish(h, lr), "ob_adam_warmup_finish")


def ob_adam_compressed_step(h, grad_ptrs, lr):
    _check(_lib.ob_adam_compressed_step(h, _ptr_array(grad_ptrs), lr), "ob_adam_compressed_step")


def ob_adam_compressed_step_static(h, grad_ptrs, lr):
    _check(_lib.ob_adam_compressed_step_static(h, _ptr_array(grad_ptrs), lr),
           "ob_adam_compressed_step_static")


def ob_adam_zero_one_step(h, grad_ptrs, lr, flags):
    _check(_lib.ob_adam_zero_one_step(h, _ptr_array(grad_ptrs), lr, flags),
           "ob_adam_zero_one_step")


def ob_adam_compress_worker(h, worker, grad_ptr):
    _check(_lib.ob_adam_compress_worker(h, worker, grad_ptr), "ob_adam_compress_worker")


def ob_adam_compressed_finish(h, lr):
    _check(_lib.ob_adam_compressed_finish(h, lr), "ob_adam_compressed_finish")


def ob_adam_get_state(h, field, worker, offset, count, dst_ptr):
    _check(_lib.ob_adam_get_state(h, field, worker, offset, count, dst_ptr), "ob_adam_get_state")


def ob_adam_set_state(h, field, offset, count, src_ptr):
    _check(_lib.ob_adam_set_state(h, field, offset, count, src_ptr), "ob_adam_set_state")


def ob_adam_params(h):
    p = ctypes.c_void_p(0)
    _check(_lib.ob_adam_params(h, ctypes.byref(p)), "ob_adam_params")
    return p.value


def ob_adam_get_counters(h):
    c = ob_adam_counters()
    _check(_lib.ob_adam_get_counters(h, ctypes.byref(c)), "ob_adam_get_counters")
    return (c.steps, c.compressed_steps, c.warmup_steps)


def ob_adam_check_guards(h):
    """-1 if every workspace guard is intact, else the first changed one."""
    bad = ctypes.c_int32(0)
    _check(_lib.ob_adam_check_guards(h, ctypes.byref(bad)), "ob_adam_check_guards")
    return bad.value


(OB_DEBUG_SYNC, OB_DEBUG_GUARDS, OB_DEBUG_SEPARATE_SCALES, OB_DEBUG_UNSTAGED_SERVER,
 OB_DEBUG_SMALL_LAUNCHES) = 1, 2, 4, 8, 16


def ob_adam_set_debug(h, flags):
    _check(_lib.ob_adam_set_debug(h, flags), "ob_adam_set_debug")


def ob_adam_attach(cfg, workspace_ptr, ws_bytes, counters, stream_ptr):
    c = ob_adam_counters(*counters)
    h = ctypes.c_void_p(0)
    _check(_lib.ob_adam_attach(ctypes.byref(cfg), workspace_ptr, ws_bytes, ctypes.byref(c),
                               stream_ptr, ctypes.byref(h)), "ob_adam_attach")
    return h.value


def ob_adam_step_count(h):
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.ob_adam_step_count(h, ctypes.byref(a), ctypes.byref(b)), "ob_adam_step_count")
    return a.value, b.value


def ob_adam_set_timing(h, max_launches):
    _check(_lib.ob_adam_set_timing(h, max_launches), "ob_adam_set_timing")


def ob_adam_kernel_times(h):
    """{kernel name: (milliseconds, launches)} and the dropped-launch count."""
    ms = (ctypes.c_double * len(KERNELS))()
    cnt = (ctypes.c_int64 * len(KERNELS))()
    dropped = ctypes.c_int64(0)
    _check(_lib.ob_adam_kernel_times(h, ms, cnt, ctypes.byref(dropped)), "ob_adam_kernel_times")
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNELS)}, dropped.value


def ob_adam_destroy(h):
    _check(_lib.ob_adam_destroy(h), "ob_adam_destroy")


_FIELD_DTYPE = {OB_X: torch.float32, OB_M: torch.float32, OB_V: torch.float32,
                OB_E_WORKER: torch.float32, OB_E_SERVER: torch.float32,
                OB_BITS_WORKER: torch.int64, OB_BITS_SERVER: torch.int64,
                OB_SCALE_WORKER: torch.float32, OB_SCALE_SERVER: torch.float32,
                OB_M_LOCAL: torch.float32, OB_A_LOCAL: torch.float32, OB_X_LOCAL: torch.float32}


class GradBatch:
    """The n gradients of one step, checked and marshalled once
    (OneBitAdam.bind_grads); the step calls take it in place of the list and
    skip the per-call checks.  It holds the tensors, whose contents may change
    between steps; indexing gives worker i's tensor."""
    __slots__ = ("tensors", "ptrs")

    def __init__(self, tensors, ptrs):
        self.tensors = tuple(tensors)
        self.ptrs = _ptr_array(ptrs)

    def __len__(self):
        return len(self.tensors)

    def __getitem__(self, i):
        return self.tensors[i]

    def __iter__(self):
        return iter(self.tensors)


class OneBitAdam:
    """A handle plus the torch-allocated workspace it lives in."""

    def __init__(self, d, n_workers, grad_dtype=OB_GRAD_F32, beta1=0.9, beta2=0.999, eps=1e-8,
                 x0=None, device="cuda", stream=None, checkpoint=None,
                 method=OB_METHOD_ONE_BIT):
        """checkpoint: (workspace bytes as a uint8 tensor, counters) from
        checkpoint() of a handle with the same configuration; the state is
        copied into a fresh workspace and attached instead of initialized.
        method: OB_METHOD_ONE_BIT (compressed_step) or OB_METHOD_ZERO_ONE
        (zero_one_step)."""
        self.cfg = make_config(d, n_workers, grad_dtype, beta1, beta2, eps, method)
        self.d, self.n = d, n_workers
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self.ws_bytes = ob_adam_workspace_bytes(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        # the library works on self.stream: tensors it touches are recorded
        # on that stream so that torch does not hand their memory out again
        # before the stream has passed, and each call is ordered after the
        # caller's current stream (and the caller's stream after the call)
        self._order_after_caller(self.workspace)
        if checkpoint is not None:
            data, counters = checkpoint
            if data.numel() != self.ws_bytes:
                raise ValueError("checkpoint of %d bytes, workspace needs %d"
                                 % (data.numel(), self.ws_bytes))
            with torch.cuda.stream(self.stream):
                self.workspace.copy_(data)
            self.stream.synchronize()
            self.h = ob_adam_attach(self.cfg, self.workspace.data_ptr(), self.ws_bytes, counters,
                                    self.stream.cuda_stream)
            return
        x0p = None
        if x0 is not None:
            if x0.dtype != torch.float32 or x0.numel() != d or not x0.is_contiguous():
                raise ValueError("x0 must be a contiguous float32 tensor of d elements")
            x0p = x0.data_ptr()
        self.h = ob_adam_init(self.cfg, self.workspace.data_ptr(), self.ws_bytes, x0p,
                              self.stream.cuda_stream)

    def _separate(self):
        return torch.cuda.current_stream(self.device) != self.stream

    def _order_after_caller(self, *tensors):
        if self._separate():
            self.stream.wait_stream(torch.cuda.current_stream(self.device))
            for t in tensors:
                t.record_stream(self.stream)

    def _ordered(self, tensors, fn, *args):
        """fn(*args) on the library's stream, ordered after the caller's
        current stream and the caller's stream after it (tensors recorded on
        the library's stream when the two differ); one stream query."""
        cur = torch.cuda.current_stream(self.device)
        if cur == self.stream:
            fn(*args)
            return
        self.stream.wait_stream(cur)
        for t in tensors:
            t.record_stream(self.stream)
        fn(*args)
        cur.wait_stream(self.stream)

    def _grad_ptrs(self, grads, count=None):
        """Device pointers of `count` (default n) checked gradient tensors."""
        count = self.n if count is None else count
        if len(grads) != count:
            raise ValueError("%d gradients given, %d expected" % (len(grads), count))
        if isinstance(grads, GradBatch):
            return grads.ptrs
        want = torch.bfloat16 if self.cfg.grad_dtype == OB_GRAD_BF16 else torch.float32
        ptrs = []
        for g in grads:
            if g.dtype != want or g.numel() != self.d or not g.is_contiguous():
                raise ValueError("gradients must be contiguous %s tensors of d elements" % want)
            ptrs.append(g.data_ptr())
        return ptrs

    def bind_grads(self, grads):
        """A GradBatch of one step's n gradient tensors (checked here once)."""
        return GradBatch(grads, self._grad_ptrs(grads))

    def warmup_step(self, grads, lr):
        self._ordered(grads, ob_adam_warmup_step, self.h, self._grad_ptrs(grads), lr)

    def warmup_worker(self, worker, grad):
        self._ordered((grad,), ob_adam_warmup_worker, self.h, worker,
                      self._grad_ptrs([grad], 1)[0])

    def warmup_finish(self, lr):
        self._ordered((), ob_adam_warmup_finish, self.h, lr)

    def compressed_step(self, grads, lr):
        self._ordered(grads, ob_adam_compressed_step, self.h, self._grad_ptrs(grads), lr)

    def compressed_step_static(self, grads, lr):
        """compressed_step with the step's scratch in the library's static
        array (allocates nothing)."""
        self._ordered(grads, ob_adam_compressed_step_static, self.h, self._grad_ptrs(grads), lr)

    def zero_one_step(self, grads, lr, sync, refresh=False):
        """One 0/1 Adam step; `sync` closes the local period, `refresh` (only
        with sync) refreshes the stale variance."""
        self._ordered(grads, ob_adam_zero_one_step, self.h, self._grad_ptrs(grads), lr,
                      (OB_ZO_SYNC if sync else 0) | (OB_ZO_REFRESH if refresh else 0))

    def compress_worker(self, worker, grad):
        self._ordered((grad,), ob_adam_compress_worker, self.h, worker,
                      self._grad_ptrs([grad], 1)[0])

    def compressed_finish(self, lr):
        self._ordered((), ob_adam_compressed_finish, self.h, lr)

    def get(self, field, worker=0, offset=0, count=None):
        """Device tensor with `count` elements of a field (see include/ob_adam.h)."""
        size = {OB_BITS_WORKER: self.d // 64, OB_BITS_SERVER: self.d // 64,
                OB_SCALE_WORKER: self.n, OB_SCALE_SERVER: self.n}.get(field, self.d)
        if count is None:
            count = size - offset
        out = torch.empty(max(count, 0), dtype=_FIELD_DTYPE[field], device=self.device)
        self._ordered((out,), ob_adam_get_state, self.h, field, worker, offset, count,
                      out.data_ptr() if count else None)
        return out

    def set(self, field, src, offset=0):
        if src.dtype != torch.float32 or not src.is_contiguous():
            raise ValueError("source must be a contiguous float32 tensor")
        self._ordered((src,), ob_adam_set_state, self.h, field, offset, src.numel(),
                      src.data_ptr())

    def checkpoint(self, device="cpu"):
        """(copy of the workspace bytes, counters): the whole optimizer state."""
        counters = ob_adam_get_counters(self.h)
        self.stream.synchronize()
        return self.workspace.to(device, copy=True), counters

    def check_guards(self):
        """-1 if no kernel wrote past a workspace buffer (synchronizes)."""
        return ob_adam_check_guards(self.h)

    def params_view(self):
        """fp32[d] tensor aliasing the library's parameters x (no copy)."""
        off = ob_adam_params(self.h) - self.workspace.data_ptr()
        if off < 0 or off + 4 * self.d > self.ws_bytes:
            raise RuntimeError("parameter buffer outside the workspace")
        return self.workspace[off:off + 4 * self.d].view(torch.float32)

    @property
    def steps(self):
        return ob_adam_step_count(self.h)

    def close(self):
        if self.h:
            ob_adam_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
