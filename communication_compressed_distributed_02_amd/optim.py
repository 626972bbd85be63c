"""1-bit Adam over a list of ragged parameter tensors, n simulated workers.

The parameters are moved once into the library's flat fp32 parameter buffer
and rebound as views of it, and every worker gets one flat gradient buffer
whose per-parameter views can be bound as the parameters' .grad (autograd
then accumulates into them in place).  A step therefore copies nothing: it
is one library call over the flat buffers.  The first `warmup_steps` steps
are full-precision Adam ("1-bit Adam ..." Abstract: warm-up phase), the rest
compression-phase steps with the variance frozen; the learning rate may
follow a schedule (the LIT-278 record notes that the frozen variance meets
learning-rate annealing in the compression phase).

Layout: every tensor starts at a multiple of 64 elements and is followed by
zero padding up to the next multiple of 64; the flat length is padded to a
multiple of 64 * n_workers.  Padding elements keep zero gradients.

It is a torch.optim.Optimizer with one parameter group: the learning rate is
read from param_groups[0]["lr"] at every step, so torch's LR schedulers
drive it, and state_dict() / load_state_dict() carry the library's whole
state (workspace bytes and step counters), so a run resumes bit-identically.
"""
import torch

from . import ob_adam as ob


def flat_layout(numels, n_workers):
    """Start offset of every tensor and the padded flat length."""
    offsets = []
    off = 0
    for k in numels:
        offsets.append(off)
        off += -(-k // 64) * 64
    unit = 64 * n_workers
    d = max(unit, -(-off // unit) * unit)
    return offsets, d


class OneBitAdamOptimizer(torch.optim.Optimizer):
    def __init__(self, params, n_workers, lr=1e-3, betas=(0.9, 0.999), eps=1e-8,
                 warmup_steps=1, grad_dtype=torch.float32, lr_schedule=None):
        params = list(params)
        if not params:
            raise ValueError("no parameters")
        super().__init__(params, dict(lr=lr, betas=tuple(betas), eps=eps))
        if len(self.param_groups) != 1:
            raise ValueError("one parameter group")
        self.params = self.param_groups[0]["params"]
        dev = self.params[0].device
        for p in self.params:
            if p.dtype != torch.float32 or p.device != dev:
                raise ValueError("parameters must be float32 tensors on one device")
        if grad_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("gradients are float32 or bfloat16")
        if warmup_steps < 1:
            raise ValueError("the variance is frozen after at least one warm-up step")
        self.n = n_workers
        self.lr_schedule = lr_schedule
        self.warmup_steps = warmup_steps
        self.grad_dtype = grad_dtype
        self.numels = [p.numel() for p in self.params]
        self.offsets, self.d = flat_layout(self.numels, n_workers)
        self._gt = ob.OB_GRAD_BF16 if grad_dtype == torch.bfloat16 else ob.OB_GRAD_F32
        self.core = ob.OneBitAdam(self.d, n_workers, self._gt, betas[0], betas[1], eps,
                                  device=dev)
        x = self.core.params_view()
        with torch.no_grad():
            for p, off, k in zip(self.params, self.offsets, self.numels):
                x[off:off + k].copy_(p.detach().reshape(-1))
        self._bind_params()
        self.grads = torch.zeros((n_workers, self.d), dtype=grad_dtype, device=dev)
        self.t = 0

    def _bind_params(self):
        x = self.core.params_view()
        for p, off, k in zip(self.params, self.offsets, self.numels):
            p.data = x[off:off + k].view(p.shape)

    def worker_grads(self, w):
        """Views of worker w's gradient buffer, one per parameter (its shape)."""
        g = self.grads[w]
        return [g[off:off + k].view(p.shape)
                for p, off, k in zip(self.params, self.offsets, self.numels)]

    def bind_worker(self, w):
        """Make worker w's views the parameters' .grad, so that a backward pass
        accumulates straight into worker w's buffer (float32 gradients only)."""
        if self.grad_dtype != torch.float32:
            raise ValueError("binding .grad needs float32 gradients; write bf16 ones into "
                             "worker_grads(w)")
        for p, gv in zip(self.params, self.worker_grads(w)):
            p.grad = gv

    def zero_grad(self, set_to_none=False):
        """Zero every worker's gradient buffer (the bound .grad views stay)."""
        self.grads.zero_()

    def current_lr(self):
        if self.lr_schedule is not None:
            return float(self.lr_schedule(self.t))
        return float(self.param_groups[0]["lr"])

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        lr = self.current_lr()
        bufs = list(self.grads.unbind(0))
        if self.t < self.warmup_steps:
            self.core.warmup_step(bufs, lr)
        else:
            self.core.compressed_step(bufs, lr)
        self.t += 1
        return loss

    @property
    def compressing(self):
        return self.t >= self.warmup_steps

    def flat_params(self):
        return self.core.params_view()

    def state_dict(self):
        """The library's state (workspace bytes on the CPU, counters) and the
        optimizer's own step count and learning rate."""
        data, counters = self.core.checkpoint("cpu")
        return {"workspace": data, "counters": counters, "t": self.t,
                "lr": self.param_groups[0]["lr"], "d": self.d, "n": self.n}

    def load_state_dict(self, state):
        if state["d"] != self.d or state["n"] != self.n:
            raise ValueError("state of a different layout (d=%d, n=%d)" % (state["d"], state["n"]))
        g = self.param_groups[0]
        self.core = ob.OneBitAdam(self.d, self.n, self._gt, g["betas"][0], g["betas"][1],
                                  g["eps"], device=self.params[0].device,
                                  checkpoint=(state["workspace"], tuple(state["counters"])))
        self._bind_params()
        self.t = state["t"]
        g["lr"] = state["lr"]
