"""The synthetic workloads the steps are checked and measured on.

Each stands in for a training job of the kind the pages report on (BERT-Base,
BERT-Large and GPT-2 pre-training, "1-bit Adam ..." Abstract and the 0/1 Adam
abstract); no dataset or weights are needed, only the flat parameter count,
the tensor shapes of those architectures (public hyper-parameters) and seeded
gradients from synth.

Padding rule: every tensor is padded to a multiple of 64 elements and the
flat vector to a multiple of 64*n; padding elements get zero gradients and
otherwise take part like any other element.
"""
from dataclasses import dataclass, field

import numpy as np

from . import NORMAL, STUDENT_T3


@dataclass
class Workload:
    name: str
    d: int                      # padded flat length, multiple of 64*n
    n: int                      # simulated data-parallel workers
    warmup: int                 # full-precision Adam steps
    compressed: int             # compression-phase steps
    dist: int = NORMAL
    sigma: float = 1e-2
    bf16: bool = False
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    linear_decay: bool = False  # compressed steps use lr0*(T-t)/(T-Tw)
    staged: bool = False        # gradients produced one worker at a time
    pads: list = field(default_factory=list)  # [(start, end)) zero-gradient ranges
    tensors: int = 1
    raw: int = 0                # elements before padding
    method: str = "one_bit"     # or "zero_one": 0/1 Adam steps after the warm-up
    sync_every: int = 1         # 0/1 Adam: local steps per synchronization

    @property
    def L(self):
        return self.d // self.n

    @property
    def steps(self):
        return self.warmup + self.compressed

    def lr_at(self, t):
        """fp32 learning rate of 0-based step t (computed in fp64, rounded once)."""
        if not self.linear_decay or t < self.warmup:
            return np.float32(self.lr)
        T, Tw = self.steps, self.warmup
        return np.float32(self.lr * (T - t) / (T - Tw))

    def zo_flags(self, t):
        """(sync, refresh) of 0-based step t >= warmup of a 0/1 Adam workload:
        a synchronization every `sync_every` steps, and a variance refresh at
        the synchronizations whose count is a power of two (1st, 2nd, 4th,
        ...: intervals that double)."""
        k = t - self.warmup + 1
        sync = k % self.sync_every == 0
        syncs = k // self.sync_every
        return sync, sync and (syncs & (syncs - 1)) == 0

    def pad_mask(self, lo, hi):
        """Boolean mask over [lo, hi): True where the gradient is forced to 0."""
        m = np.zeros(hi - lo, dtype=bool)
        for a, b in self.pads:
            a2, b2 = max(a, lo), min(b, hi)
            if a2 < b2:
                m[a2 - lo:b2 - lo] = True
        return m


def _round_up(x, m):
    return (x + m - 1) // m * m


def _layout(sizes, n):
    """Per-tensor 64-padding, then tail padding to 64*n; returns (d, pads, raw)."""
    pads = []
    off = 0
    for s in sizes:
        p = _round_up(s, 64)
        if p > s:
            pads.append((off + s, off + p))
        off += p
    d = _round_up(off, 64 * n)
    if d > off:
        pads.append((off, d))
    return d, pads, sum(sizes)


def bert_large_sizes():
    """390 tensors of a 24-layer, hidden-1024, FFN-4096 BERT (vocab 30522)."""
    h, f, v = 1024, 4096, 30522
    sizes = [v * h, 512 * h, 2 * h, h, h]
    for _ in range(24):
        sizes += [h * h, h] * 4          # Q, K, V, attention output (+ biases)
        sizes += [h, h]                  # attention LayerNorm
        sizes += [h * f, f, f * h, h]    # FFN in / out (+ biases)
        sizes += [h, h]                  # output LayerNorm
    sizes += [v]                         # MLM decoder bias
    return sizes


def gpt2_xl_sizes():
    """580 tensors of a 48-layer, hidden-1600 GPT-2 (vocab 50257, context 1024)."""
    h, v = 1600, 50257
    sizes = [v * h, 1024 * h]
    for _ in range(48):
        sizes += [h, h, h * 3 * h, 3 * h, h * h, h, h, h, h * 4 * h, 4 * h, 4 * h * h, h]
    sizes += [h, h]
    return sizes


def _flat(raw, n):
    return _layout([raw], n)


def make(name):
    if name == "c1":
        return Workload("c1", d=1 << 20, n=4, warmup=3, compressed=7, sigma=1e-2, raw=1 << 20)
    if name == "c2":
        d, pads, raw = _flat(110_000_000, 8)
        return Workload("c2", d=d, n=8, warmup=2, compressed=20, sigma=1e-3, bf16=True,
                        pads=pads, raw=raw)
    if name == "c3":
        sizes = bert_large_sizes()
        d, pads, raw = _layout(sizes, 16)
        return Workload("c3", d=d, n=16, warmup=3, compressed=7, sigma=1e-3, pads=pads,
                        tensors=len(sizes), raw=raw)
    if name == "c4":
        sizes = gpt2_xl_sizes()
        d, pads, raw = _layout(sizes, 8)
        return Workload("c4", d=d, n=8, warmup=3, compressed=50, dist=STUDENT_T3, sigma=1e-3,
                        pads=pads, tensors=len(sizes), raw=raw)
    if name == "c5":
        d, pads, raw = _flat(340_000_000, 64)
        return Workload("c5", d=d, n=64, warmup=30, compressed=170, sigma=1e-3,
                        linear_decay=True, staged=True, pads=pads, raw=raw)
    # 0/1 Adam ("Maximizing Communication Efficiency for Large-scale Training
    # via 0/1 Adam", abstract: BERT-Base and BERT-Large pre-training among its
    # benchmarks; about half the communication rounds of 1-bit Adam): a
    # synchronization every 2 steps
    if name == "z2":
        d, pads, raw = _flat(110_000_000, 8)
        return Workload("z2", d=d, n=8, warmup=2, compressed=20, sigma=1e-3, bf16=True,
                        pads=pads, raw=raw, method="zero_one", sync_every=2)
    if name == "z3":
        sizes = bert_large_sizes()
        d, pads, raw = _layout(sizes, 16)
        return Workload("z3", d=d, n=16, warmup=3, compressed=12, sigma=1e-3, pads=pads,
                        tensors=len(sizes), raw=raw, method="zero_one", sync_every=2)
    if name == "idx64":
        # not a workload of the pages: the largest arrays of the tests, so
        # that element indices run past 2^31 (chunk 3 straddles it)
        d = (1 << 31) + (1 << 22)
        return Workload("idx64", d=d, n=4, warmup=1, compressed=2, sigma=1e-3, bf16=True, raw=d)
    raise KeyError(name)


NAMES = ("c1", "c2", "c3", "c4", "c5")
ZERO_ONE = ("z2", "z3")  # the 0/1 Adam workloads
EXTRA = ("idx64",)  # size edge case of the tests


def describe(w):
    return {"workload": w.name, "d": w.d, "n_workers": w.n, "chunk": w.L,
            "grads": ("bf16" if w.bf16 else "fp32") + (" student-t3" if w.dist else " normal"),
            "sigma": w.sigma, "warmup_steps": w.warmup, "compressed_steps": w.compressed,
            "tensors": w.tensors, "method": w.method,
            **({"sync_every": w.sync_every} if w.method == "zero_one" else {})}


def cpu_grad(w, worker, step, lo, hi):
    """Worker's gradient at 0-based step over [lo, hi) (numpy, pads zeroed)."""
    from . import fill_cpu
    g = fill_cpu(hi - lo, lo, step, worker, w.dist, w.sigma, w.bf16)
    mask = w.pad_mask(lo, hi)
    if mask.any():
        g[mask] = 0
    return g


