#!/usr/bin/env python3
"""Benchmark of the 1-bit Adam compression-phase step on one MI355X.

A step is one compressed step over one batch of n workers' synthetic
gradients (all of the compressed step: worker compress, worker scales,
server average/re-compress, server scales, decompress + frozen-variance
update).
Default workload: c5, the BERT-Large run on 64 data-parallel workers --
d = 340,000,768 fp32 parameters, n = 64 simulated workers, fp32 gradients
N(0, 1e-3), supplied one worker at a time (the staged entry points), 30
full-precision warm-up steps before the compressed ones.  All gradients are
generated on the GPU before the timed region.

Prints one JSON line with:
- params*workers/s of the whole step;
- the worker pass's roofline against MI355X's 8 TB/s HBM peak, timed live
  with HIP events the library records on its stream, next to the same
  figure from the committed kernel-trace average, plus the profiler's byte
  counters when they were taken on the current kernel code;
- the step's other kernels and streaming probes of the same access mix;
- the CPU oracle timed on a bounded sample (chunk 0), and, when the sample
  runs the same steps as the GPU, the comparison of the two states (parity).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "compressed-step params·workers/sec and achieved HBM GB/s (% of peak), 1 GPU"
# the 0/1 Adam workloads' line: the same units over their steps' mix
ZO_METRIC = "0/1 Adam step params·workers/sec and achieved HBM GB/s (% of peak), 1 GPU"
KERNEL_SRC = os.path.join(ROOT, "communication_compressed_distributed_02_amd", "csrc",
                          "ob_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "worker_pass_%s_counters.txt")  # % workload
TRACE_FILE = os.path.join(ROOT, "profiles", "compressed_step_%s_kernel_trace.txt")  # % workload
DEFAULT_WORKLOAD = "c5"
# CPU-baseline budget: (warm-up + timed) oracle steps x n x L element-workers
# (about 1e8 per second on one core)
CPU_BUDGET = 2.5e9


def alg_bytes(w):
    """Algorithmic HBM bytes per kernel launch of one steady-state compressed
    step (momentum held as server sign words + scales; every array touched
    once; partials of the fixed-order sums included)."""
    d, n = w.d, w.n
    gb = 2 if w.bf16 else 4
    nseg = -(-w.L // 1024)
    nquad = -(-nseg // 4)  # one fp64 partial per block of 4 segments
    part_w = 8 * n * n * nquad
    part_s = 8 * n * (nseg if n in (32, 64) else nquad)  # per segment at 32 and 64 workers
    # worker-pass launches per step: one for all workers, or one per worker
    # when the gradients come one worker at a time (each launch reads the
    # momentum's sign words)
    launches = n if w.staged else 1
    return {
        # grad in, compensated momentum in and out, sign words out, momentum words in
        "worker": n * d * (gb + 4 + 4) + n * d // 8 + launches * (d // 8) + part_w,
        "worker_scale": part_w + 4 * n * n,
        # worker sign words in, server u in and out, server words out
        "server": n * d // 8 + 8 * d + d // 8 + part_s + 4 * n * n,
        "server_scale": part_s + 4 * n,
        # server words in, x in and out, v in
        "update": d // 8 + 12 * d + 4 * n,
    }


# elements per dispatch of a streaming pass; the 32- and 64-worker server pass
# uses 16 times that
DISPATCH_ELEMS = 1 << 26


def pass_dispatches(rows, nbx, row_elems, elems=DISPATCH_ELEMS):
    """Dispatches the library issues for a pass over `rows` grid rows of
    `nbx` blocks, each row `row_elems` elements: whole rows grouped into
    launches of about `elems` elements, or a longer row cut into ranges of
    its blocks."""
    total = rows * row_elems
    cuts, per_rows = 1, rows
    if total > elems:
        if row_elems >= elems:
            cuts, per_rows = min(nbx, -(-row_elems // elems)), 1
        else:
            per_rows = -(-rows // -(-total // elems))
    bx_per = -(-nbx // cuts)
    return -(-rows // per_rows) * -(-nbx // bx_per)


def dispatches_per_pass(w):
    """Dispatches of one worker pass, server pass and update of workload w."""
    nseg = -(-w.L // 1024)
    nquad = -(-nseg // 4)
    groups = -(-(w.d // 64) // 16)  # the update's waves: 16 rows each
    return {
        "worker": pass_dispatches((1 if w.staged else w.n) * w.n, nquad, w.L),
        "server": (pass_dispatches(w.n, nseg, w.L, 16 * DISPATCH_ELEMS) if w.n in (32, 64)
                   else pass_dispatches(w.n, nquad, w.L)),
        "update": -(-groups // -(-groups // max(1, -(-groups * 1024 // DISPATCH_ELEMS)))),
    }


def zo_alg_bytes(w):
    """The 0/1 Adam workloads: algorithmic bytes per launch of each kernel, a
    schedule with `sync_every` = 2 (every local step opens a period, every
    synchronizing step closes it).  Local step: gradient in, local momentum
    and mean momentum out, shared momentum's words in.  Synchronizing worker
    pass: gradient, local momentum, mean momentum and compensated momentum
    in, compensated momentum and sign words out, partials.  Refresh: all
    workers' gradients in, v in and out.  Scales, server pass and update as
    in the compressed step."""
    d, n = w.d, w.n
    gb = 2 if w.bf16 else 4
    b = alg_bytes(w)
    nseg = -(-w.L // 1024)
    part_w = 8 * n * n * -(-nseg // 4)
    return {
        "zo_local": n * d * (gb + 8) + d // 8,
        "worker": n * d * (gb + 4 + 4 + 4 + 4) + n * d // 8 + part_w,
        "worker_scale": b["worker_scale"],
        "server": b["server"],
        "server_scale": b["server_scale"],
        "update": b["update"],
        "zo_refresh": n * d * gb + 8 * d,
    }


def fp32_momentum_step_bytes(w):
    """Bytes per step with the momentum kept in fp32 (read and written each
    step) and the server-bit read counted per worker: d*[n*(gb+8.25)+28.125]."""
    gb = 2 if w.bf16 else 4
    return w.d * (w.n * (gb + 8.25) + 28.125)


def kernel_sha():
    """sha256[:16] of the kernel source's code: // comments, indentation and
    blank lines removed, so that only a change of code voids the counters."""
    code = []
    for line in open(KERNEL_SRC, encoding="utf-8"):
        line = re.sub(r"//.*$", "", line).strip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _load_record(path, key, workload):
    """The `key: {json}` record of a profile summary, if it was taken on the
    current kernel source for this workload (else None)."""
    t = None
    try:
        for line in open(path % workload):
            if line.startswith(key + ": "):
                t = json.loads(line[len(key) + 2:])
    except (OSError, ValueError):
        return None
    if t is None:
        return None
    if t.get("kernel_source_sha") != kernel_sha() or t.get("workload") != workload:
        return None
    return t


def load_traffic(workload):
    """Counter-measured HBM bytes per worker pass (the summed counters of its
    dispatches), if they were taken on the current kernel source (else
    None)."""
    return _load_record(TRAFFIC_FILE, "traffic_record", workload)


def load_trace(workload):
    """rocprofv3's average duration of a steady-state worker pass (the summed
    durations of its dispatches), if the trace was taken on the current
    kernel source (else None)."""
    return _load_record(TRACE_FILE, "trace_record", workload)


def host_cpu():
    """The host's CPU model and the cores this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_plan(w, steps):
    """(warm-up steps, compressed steps) of the CPU baseline on chunk 0.  The
    workload's own warm-up and `steps` compressed steps when the sample fits
    CPU_BUDGET (then its state can be compared with the GPU's); else one
    warm-up step and as many compressed steps as fit, at least one.  The
    oracle's time per compressed step does not depend on the state it starts
    from, so the shortened sample still times the same work per step."""
    unit = w.n * w.L
    if (w.warmup + steps) * unit <= CPU_BUDGET:
        return w.warmup, steps
    return 1, max(1, min(steps, int(CPU_BUDGET // unit) - 1))


def cpu_baseline(w, steps=1, snap=None):
    """The CPU oracle on chunk 0 (all n workers, 1/n of the step's work),
    timed over the compressed steps of cpu_plan(), scaled by n.  The calling thread is pinned to one core while the
    oracle runs.  With `snap` (the GPU's chunk-0 state after the same steps on
    the same gradients) the two are compared: returns (baseline, parity)."""
    import oracle
    from synth import workloads as W
    L = w.L
    warm, steps = cpu_plan(w, steps)
    model, usable = host_cpu()
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        per_step, o = _oracle_step_seconds(oracle, W, w, L, warm, steps)
    finally:
        os.sched_setaffinity(0, allowed)
    parity = compare_chunk0(oracle, o, snap, w) if snap is not None else None
    o.close()
    short = "" if warm == w.warmup else (
        " (the workload has %d warm-up steps; the sample starts its compressed steps after %d "
        "to bound its run)" % (w.warmup, warm))
    return {"value": w.n * w.d / per_step, "unit": "params*workers/s", "cores": 1,
            "kind": "oracle",
            "sample": "chunk 0 of %d (%d elements x %d workers), %d %s step(s) after "
                      "%d warm-up step(s)%s, single thread pinned to core %d, time x%d for the "
                      "whole step" % (w.n, L, w.n, steps,
                                      "0/1 Adam" if w.method == "zero_one" else "compressed",
                                      warm, short, core, w.n),
            "host_cpu": model, "host_cores_usable": usable,
            "s_per_step_extrapolated": per_step}, parity


REL_TOL, ABS_TOL = 1e-5, 1e-6


def snapshot_chunk0(opt, w):
    """The GPU's state of chunk 0 (host copies) for compare_chunk0."""
    from communication_compressed_distributed_02_amd import ob_adam as ob
    L, n = w.L, w.n

    def get(field, worker=0, count=L):
        return opt.get(field, worker, 0, count).cpu().numpy()
    return {"step": opt.steps[0],
            "x": get(ob.OB_X), "e_srv": get(ob.OB_E_SERVER),
            "e_w": [get(ob.OB_E_WORKER, i) for i in range(n)],
            "bits_w": [get(ob.OB_BITS_WORKER, i, L // 64).view(np.uint64) for i in range(n)],
            "bits_s": get(ob.OB_BITS_SERVER, 0, L // 64).view(np.uint64),
            "scale_w": [get(ob.OB_SCALE_WORKER, i, 1).view(np.uint32)[0] for i in range(n)],
            "scale_s": get(ob.OB_SCALE_SERVER, 0, 1).view(np.uint32)[0]}


def replica_snapshot(w, warm, steps):
    """The GPU's chunk-0 state after the CPU sample's own schedule -- `warm`
    warm-up steps, then `steps` compressed (or 0/1 Adam) steps, on the same
    gradients, step sizes and 0/1 flags -- run on a fresh full-size handle
    (for a workload whose sample does not follow the timed run's steps, such
    as c5's: its 30 warm-up steps would not fit the sample's budget)."""
    import torch

    import synth
    from communication_compressed_distributed_02_amd import ob_adam as ob
    dev = torch.device("cuda:0")
    gdt = torch.bfloat16 if w.bf16 else torch.float32
    zero_one = w.method == "zero_one"
    opt = ob.OneBitAdam(w.d, w.n, ob.OB_GRAD_BF16 if w.bf16 else ob.OB_GRAD_F32, w.beta1,
                        w.beta2, w.eps, device=dev,
                        method=ob.OB_METHOD_ZERO_ONE if zero_one else ob.OB_METHOD_ONE_BIT)

    def fill(buf, i, t):
        synth.fill_gpu(buf, 0, t, i, w.dist, w.sigma)
        for lo, hi in w.pads:
            buf[lo:hi].zero_()
    if w.staged:  # one gradient buffer, regenerated per worker
        one = torch.empty(w.d, dtype=gdt, device=dev)
        for t in range(warm + steps):
            for i in range(w.n):
                fill(one, i, t)
                (opt.warmup_worker if t < warm else opt.compress_worker)(i, one)
            (opt.warmup_finish if t < warm else opt.compressed_finish)(w.lr_at(t))
    else:
        full = torch.empty((w.n, w.d), dtype=gdt, device=dev)
        for t in range(warm + steps):
            for i in range(w.n):
                fill(full[i], i, t)
            g = list(full.unbind(0))
            if t < warm:
                opt.warmup_step(g, w.lr_at(t))
            elif zero_one:  # the flags of the step after the workload's own warm-up
                opt.zero_one_step(g, w.lr_at(t), *w.zo_flags(w.warmup + t - warm))
            else:
                opt.compressed_step(g, w.lr_at(t))
    torch.cuda.synchronize()
    snap = snapshot_chunk0(opt, w)
    snap["gpu_run"] = ("a fresh full-size handle running the sample's %d warm-up + %d %s "
                       "steps" % (warm, steps, "0/1 Adam" if zero_one else "compressed"))
    del opt
    torch.cuda.empty_cache()
    return snap


def compare_chunk0(oracle, o, snap, w):
    """Sign words, scales and the step counter bit-exact; x and the errors
    within 1e-5 relative or 1e-6 absolute (worst ratio of error to the
    allowed error reported; <= 1 passes)."""
    n = w.n
    bits = all(np.array_equal(snap["bits_w"][i], o._view(oracle.BITS_WORKER, i))
               for i in range(n)) and np.array_equal(snap["bits_s"], o._view(oracle.BITS_SERVER))
    scales = (all(snap["scale_w"][i] == o._view(oracle.SCALE_WORKER, i)[:1].view(np.uint32)[0]
                  for i in range(n))
              and snap["scale_s"] == o._view(oracle.SCALE_SERVER)[:1].view(np.uint32)[0])
    worst = {}
    fields = [("x", snap["x"], o._view(oracle.X)), ("e_srv", snap["e_srv"], o._view(oracle.E_SERVER))]
    fields += [("e_w%d" % i, snap["e_w"][i], o._view(oracle.E_WORKER, i)) for i in range(n)]
    for name, g, r in fields:
        g64 = g.astype(np.float64)
        r64 = r.astype(np.float64)
        allowed = np.maximum(REL_TOL * np.abs(r64), ABS_TOL)
        worst[name] = float(np.max(np.abs(g64 - r64) / allowed))
    ratio = max(worst.values())
    return {"against": "oracle", "sample": "chunk 0 (%d elements x %d workers), state after "
            "step %d" % (w.L, n, o.step),
            "gpu_run": snap.get("gpu_run", "the timed run's own untimed steps"),
            "step_equal": snap["step"] == o.step,
            "sign_words_equal": bool(bits), "scales_equal": bool(scales),
            "fp32_worst_error_over_tolerance": ratio,
            "fp32_worst_field": max(worst, key=worst.get),
            "pass": bool(bits and scales and snap["step"] == o.step and ratio <= 1.0)}


def _oracle_step_seconds(oracle, W, w, L, warm, steps):
    o = oracle.Oracle(w.d, w.n, w.beta1, w.beta2, w.eps, j0=0, j1=1, keep_debug=False)
    secs = []
    for t in range(warm + steps):
        g = [W.cpu_grad(w, i, t, 0, L) for i in range(w.n)]
        if t < warm:
            o.warmup_step(g, w.lr_at(t))
            continue
        t0 = time.perf_counter()
        if w.method == "zero_one":
            sync, refresh = w.zo_flags(w.warmup + t - warm)
            o.zo_step(g, w.lr_at(t), sync, refresh)
        else:
            o.compressed_step(g, w.lr_at(t))
        secs.append(time.perf_counter() - t0)
        del g
    return sum(secs) / len(secs) * w.n, o


PROBE_LIB = os.path.join(ROOT, "communication_compressed_distributed_02_amd", "libob_probe.so")
PROBE_KINDS = {"mix": 0, "copy": 1, "read": 2, "write": 3, "mix32": 4}


def probe_lib():
    import ctypes
    import torch  # noqa: F401  (torch's HIP runtime first)
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("libob_probe.so is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.ob_probe_run_sync.restype = ctypes.c_int
    lib.ob_probe_run_sync.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int64,
                                                                                ctypes.c_void_p]
    lib.ob_probe_run.restype = ctypes.c_int
    lib.ob_probe_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p]
    return lib


def run_probe(lib, kind, a, b, n):
    import torch
    rc = lib.ob_probe_run(PROBE_KINDS[kind], a.data_ptr() if a is not None else None,
                          b.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError("ob_probe_run(%s) failed: %d" % (kind, rc))


def copy_calibration(mib):
    """Plain streaming kernels of known size (mib MiB each): copy, read-only and
    write-only, three dispatches each, for scaling profiler byte counters."""
    import torch
    lib = probe_lib()
    n = mib * 1024 * 1024 // 4
    n -= n % 4096
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for kind, a in (("copy", x), ("read", x), ("write", None)):
        for _ in range(3):
            run_probe(lib, kind, a, y, n)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_bytes": 4 * n, "copy": "reads and writes 4n",
                      "read": "reads 4n", "write": "writes 4n", "dispatches_each": 3}), flush=True)


def stream_ceilings(n, bf16=True, reps=5, sync=False):
    """GB/s of the probes over n elements on this device, issued as the
    library issues a pass: dispatches of about DISPATCH_ELEMS elements.  The
    worker pass's access mix (bf16 gradients: 6 B read + 4 B written per
    element; fp32: 8 + 4), copy, read-only and write-only, with the step's own
    wave-row mapping and non-temporal hints; with `sync`, the 0/1 Adam
    synchronizing worker pass's mix too (gradient + 12 B read, 4 B written);
    and, for reference, the same mix as a torch elementwise kernel and a
    runtime device-to-device copy (one dispatch each)."""
    import torch
    lib = probe_lib()
    parts = max(1, -(-n // DISPATCH_ELEMS))
    per = max(4096, (n // parts) // 4096 * 4096)
    n = per * parts
    g = torch.zeros(n, dtype=torch.int16 if bf16 else torch.float32, device="cuda:0")
    c = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    c2 = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    out = {"elements": n, "dispatches": parts}
    mix = ("mix", g, c, 10 * n) if bf16 else ("mix32", g, c, 12 * n)

    def sliced(kind, a, b):
        for i in range(parts):
            run_probe(lib, kind, a[i * per:(i + 1) * per] if a is not None else None,
                      b[i * per:(i + 1) * per], per)
    for kind, a, b, nbytes in (mix, ("copy", c, c2, 8 * n),
                               ("read", c, c2, 4 * n), ("write", None, c2, 4 * n)):
        for _ in range(2):
            sliced(kind, a, b)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sliced(kind, a, b)
        e1.record()
        torch.cuda.synchronize()
        out[("mix" if kind == "mix32" else kind) + "_GB_s"] = round(
            nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    if sync:
        m = torch.zeros(n, dtype=torch.float32, device="cuda:0")
        a = torch.zeros(n, dtype=torch.float32, device="cuda:0")
        st = torch.cuda.current_stream().cuda_stream

        def sync_pass():
            for i in range(parts):
                sl = slice(i * per, (i + 1) * per)
                rc = lib.ob_probe_run_sync(1 if bf16 else 0, g[sl].data_ptr(), m[sl].data_ptr(),
                                           a[sl].data_ptr(), c[sl].data_ptr(), per, st)
                if rc != 0:
                    raise RuntimeError("ob_probe_run_sync failed: %d" % rc)
        for _ in range(2):
            sync_pass()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sync_pass()
        e1.record()
        torch.cuda.synchronize()
        nbytes = ((2 if bf16 else 4) + 16) * n
        out["sync_mix_GB_s"] = round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del m, a
    # the same access mix and a copy as the vendor stack implements them:
    # torch's elementwise c += g (the gradient widened to fp32 on the fly),
    # and the runtime's device-to-device copy
    gt = g.view(torch.bfloat16) if bf16 else g
    for name, fn, nbytes in (("torch_mix", lambda: c.add_(gt), (6 if bf16 else 8) * n + 4 * n),
                             ("runtime_copy", lambda: c2.copy_(c), 8 * n)):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_GB_s"] = round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del g, c, c2
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3, help="untimed compressed steps")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=None,
                    help="compressed steps of the CPU baseline (default: --warmup, so that "
                         "its state can be compared with the GPU's after the untimed steps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's device copy of MIB MiB five times (a kernel of "
                         "known traffic for scaling profiler byte counters) and exit")
    a = ap.parse_args()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: the simulated workers live on one MI355X; "
              "--gpus %d is not supported" % a.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from communication_compressed_distributed_02_amd import ob_adam as ob
    from synth import workloads as W

    w = W.make(a.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gdt = torch.bfloat16 if w.bf16 else torch.float32
    batch_bytes = w.n * w.d * (2 if w.bf16 else 4)
    batches = w.warmup + a.warmup + a.steps
    # distinct gradients for every step when they fit in about 120 GB, else a
    # ring of as many batches as fit (at least one; reuse does not help the
    # caches: one batch is many times their size)
    ring = max(1, min(batches, int(120e9 // batch_bytes)))
    print("# generating %d gradient batch(es) of %d x %d %s on the GPU"
          % (ring, w.n, w.d, "bf16" if w.bf16 else "fp32"), file=sys.stderr, flush=True)
    ring_grads = []
    for t in range(ring):
        g = torch.empty((w.n, w.d), dtype=gdt, device=dev)
        for i in range(w.n):
            synth.fill_gpu(g[i], 0, t, i, w.dist, w.sigma)
            for lo, hi in w.pads:
                g[i, lo:hi].zero_()
        ring_grads.append(list(g.unbind(0)))
    grads = [ring_grads[t % ring] for t in range(batches)]

    zero_one = w.method == "zero_one"

    def step(opt, t):
        if zero_one:
            sync, refresh = w.zo_flags(t)
            opt.zero_one_step(grads[t], w.lr_at(t), sync, refresh)
        elif w.staged:
            for i in range(w.n):
                opt.compress_worker(i, grads[t][i])
            opt.compressed_finish(w.lr_at(t))
        else:
            opt.compressed_step(grads[t], w.lr_at(t))
    opt = ob.OneBitAdam(w.d, w.n, ob.OB_GRAD_BF16 if w.bf16 else ob.OB_GRAD_F32, w.beta1,
                        w.beta2, w.eps, device=dev,
                        method=ob.OB_METHOD_ZERO_ONE if zero_one else ob.OB_METHOD_ONE_BIT)
    # each batch checked and marshalled once, as a training loop with fixed
    # gradient buffers would: a step call then costs the C call and its
    # launches only (on 1M x 4 the per-call checks took longer than the step)
    bound = [opt.bind_grads(r) for r in ring_grads]
    grads = [bound[t % ring] for t in range(batches)]
    for t in range(w.warmup):
        if w.staged:
            for i in range(w.n):
                opt.warmup_worker(i, grads[t][i])
            opt.warmup_finish(w.lr_at(t))
        else:
            opt.warmup_step(grads[t], w.lr_at(t))
    for t in range(w.warmup, w.warmup + a.warmup):
        step(opt, t)
    torch.cuda.synchronize()
    cpu_steps = a.warmup if a.cpu_steps is None else a.cpu_steps
    snap = None
    if (not a.no_cpu_baseline and cpu_steps == a.warmup and ring >= w.warmup + a.warmup
            and cpu_plan(w, cpu_steps) == (w.warmup, cpu_steps)):
        # the untimed steps ran on each step's own gradients: keep chunk 0's
        # state for the comparison with the oracle after the same steps
        snap = snapshot_chunk0(opt, w)
        torch.cuda.synchronize()
    print("# timing %d compressed steps" % a.steps, file=sys.stderr, flush=True)

    # Region 1 (the headline): K steps with nothing but the step on the stream.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for i in range(a.steps):
        step(opt, w.warmup + a.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / a.steps
    # Region 2: the same K steps again (the next steps of the run) with the
    # library's per-kernel HIP events, taken from the dispatch packets on its
    # stream; they add ~1.5 % to a step, so they stay out of region 1.
    ob.ob_adam_set_timing(opt.h, (w.n + 4) * a.steps + 8)  # passes per step: n + 4 at most
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record()
    for i in range(a.steps):
        step(opt, w.warmup + a.warmup + i)
    f1.record()
    torch.cuda.synchronize()
    ms_step_timed = f0.elapsed_time(f1) / a.steps
    kt, dropped = ob.ob_adam_kernel_times(opt.h)
    ob.ob_adam_set_timing(opt.h, 0)

    ab = zo_alg_bytes(w) if zero_one else alg_bytes(w)
    kernels = {}
    for k in ab:
        ms, cnt = kt[k]
        if cnt:
            avg = ms / cnt
            kernels[k] = {"avg_ms": round(avg, 5), "launches": cnt, "alg_bytes": ab[k],
                          "GB_s": round(ab[k] / (avg * 1e-3) / 1e9, 1)}
    if w.staged:  # one worker-pass launch per worker: report the per-step sum
        k = kernels["worker"]
        per = w.n
        k["avg_ms"] = round(k["avg_ms"] * per, 5)
        k["launches"] //= per
        k["GB_s"] = round(ab["worker"] / (k["avg_ms"] * 1e-3) / 1e9, 1)
        k["note"] = "staged: %d launches (one per worker) per step, summed" % per
    wk = kernels["worker"]
    traffic = load_traffic(w.name)
    trace = load_trace(w.name)
    # the same roofline from rocprofv3's kernel trace of this kernel code,
    # committed: a pass's algorithmic bytes over the summed durations of its
    # dispatches, averaged over the run's steady-state passes
    per_pass = ab["worker"] // (w.n if w.staged else 1)
    trace_gbs = per_pass / (trace["avg_ns"] * 1e-9) / 1e9 if trace else None
    if zero_one:
        # mean bytes per step over the timed steps' schedule (local steps,
        # synchronizing steps with their finalizes, server pass and update,
        # refreshes where flagged)
        tot = 0
        for t in range(w.warmup + a.warmup, w.warmup + a.warmup + a.steps):
            sync, refresh = w.zo_flags(t)
            if not sync:
                tot += ab["zo_local"]
                continue
            tot += sum(ab[k] for k in ("worker", "worker_scale", "server", "server_scale",
                                       "update"))
            tot += ab["zo_refresh"] if refresh else 0
        step_bytes = tot / a.steps
    else:
        step_bytes = sum(ab.values())
    result = {
        "metric": ZO_METRIC if zero_one else METRIC,
        "value": w.n * w.d / (ms_step * 1e-3),
        "unit": "params*workers/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(W.describe(w), parallelism="n simulated data-parallel workers on 1 GPU",
                       gradient_batches=ring, entry_point="staged per-worker" if w.staged
                       else ("0/1 Adam steps, all workers" if zero_one else "all workers")),
        "roofline": {"bound": "hbm",
                     "kernel": "synchronizing worker pass" if zero_one else "worker pass",
                     "achieved": round(wk["GB_s"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(wk["GB_s"] / HBM_PEAK_GBS, 4),
                     "frac_source": "HIP events from the start of the first to the end of "
                                    "the last dispatch of every worker pass of timing region 2 "
                                    "(live, this run)",
                     "achieved_from_trace": round(trace_gbs, 1) if trace else None,
                     "frac_from_trace": round(trace_gbs / HBM_PEAK_GBS, 4) if trace else None,
                     "trace_avg_us_per_pass": round(trace["avg_ns"] / 1e3, 2) if trace else None,
                     "trace_dispatches_per_pass": trace.get("dispatches_per_pass") if trace
                     else None,
                     "trace_kernel": trace["kernel"] if trace else None,
                     "trace_file": os.path.relpath(TRACE_FILE % w.name, ROOT) if trace else None,
                     "traffic": traffic["bytes_per_pass"] if traffic else None,
                     "traffic_unit": "HBM bytes per worker pass (rocprofv3 FETCH_SIZE + "
                                     "WRITE_SIZE of its dispatches, copy-calibrated)",
                     "traffic_fetch": traffic["fetch_bytes_per_pass"] if traffic else None,
                     "traffic_write": traffic["write_bytes_per_pass"] if traffic else None,
                     "alg_bytes_per_pass": per_pass,
                     "passes_per_step": w.n if w.staged else 1,
                     "dispatches_per_pass": dispatches_per_pass(w)["worker"]},
        "step": {"alg_bytes": step_bytes, "GB_s": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                 "frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "fp32_momentum_bytes": None if zero_one else fp32_momentum_step_bytes(w),
                 "fp32_momentum_frac_of_peak": None if zero_one else round(
                     fp32_momentum_step_bytes(w) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "traffic": traffic.get("step_bytes") if traffic else None,
                 "traffic_GB_s": round(traffic["step_bytes"] / (ms_step * 1e-3) / 1e9, 1)
                 if traffic and traffic.get("step_bytes") else None,
                 "traffic_unit": "HBM bytes per steady-state step (rocprofv3 FETCH_SIZE + "
                                 "WRITE_SIZE of each kernel, copy-calibrated)",
                 "wall_s": round(wall, 4),
                 "ms_per_step_with_kernel_events": round(ms_step_timed, 4),
                 "timing_launches_dropped": dropped},
        "kernels": kernels,
    }
    del grads, bound, ring_grads, opt
    torch.cuda.empty_cache()
    ceil = stream_ceilings(min(w.n * w.d if not w.staged else w.d, 1 << 31), w.bf16,
                           sync=zero_one)
    ceil["note"] = ("probe kernels with the worker pass's mapping over as many elements as one "
                    "pass of it (at most 2^31), in dispatches of about 2^26 elements as the "
                    "library issues a pass; mix = its %d B read + 4 B written per element; "
                    "torch_mix = the same mix as torch's c += g, runtime_copy = a device-to-"
                    "device copy" % (6 if w.bf16 else 8))
    if zero_one:
        ceil["note"] += ("; sync_mix = the synchronizing worker pass's %d B read + 4 B written "
                         "per element, against which worker_frac_of_mix is taken"
                         % (14 if w.bf16 else 16))
    ceil["worker_frac_of_mix"] = round(wk["GB_s"] / ceil["sync_mix_GB_s" if zero_one
                                                          else "mix_GB_s"], 4)
    result["ceilings"] = ceil
    if not a.no_cpu_baseline:
        print("# timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if snap is None:
            # the sample does not follow the timed run: replay its schedule on
            # the GPU (the timed run's memory is free by now)
            snap = replica_snapshot(w, *cpu_plan(w, cpu_steps))
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, cpu_steps, snap)
    else:
        result["cpu_baseline"] = None
        result["parity"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
