"""Write the stored expected values of the large workloads from the CPU oracle.

Only the oracle (oracle/) and the seeded input generator (synth/) are used;
nothing here touches the GPU path.  Every chunk of the method is independent
of the others, so the oracle runs on whole sampled chunks (all n workers,
every step) and records, for each:
 - per compressed step: the bit patterns of the chunk's n worker scales and
   server scale, and xxh64 digests of all workers' sign words and of the
   server's sign words over the chunk; for the 0/1 Adam workloads the same
   at every synchronizing step, and at every local step digests of all
   workers' local momenta and step-weighted mean momenta over the chunk;
 - after the warm-up: x, m, v at the sampled elements;
 - after the middle compressed step ("mid") and after the last step
   ("final"): xxh64 digests of the whole chunk's x, m, v, server error and
   every worker's error (fp32 bit patterns), and the values of x, m, v and
   the server error at the sampled elements, and of the errors of the first
   and the last worker (a 0/1 Adam workload's mid checkpoint falls inside a
   local period and adds digests of every worker's local model).
The sampled elements of a chunk are its first and last segments (1024
elements each) and 2048 more drawn with a seeded generator (for a chunk that
holds element 2^31, also the four around it and 60 past it).

    python tests/golden/make_golden.py c2 --jobs 4
writes tests/golden/c2/chunk_<j>.json (scales, digests) and chunk_<j>.npz
(the sampled elements' offsets in the chunk, and their values as uint32 bit
patterns) for the chunks listed in SAMPLED.
"""
import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import xxhash  # noqa: E402

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SAMPLED = {"c1": [0, 1, 2, 3], "c2": list(range(8)), "c3": list(range(16)), "c4": [0, 2, 5, 7],
           "c5": [0, 7, 15, 23, 31, 39, 47, 55, 63], "idx64": [3],
           "z2": list(range(8)), "z3": list(range(16))}
N_RANDOM = 2048
SEG = 1024


def sample_indices(w, j):
    """Sorted global indices of the sampled elements of chunk j."""
    L = w.L
    rng = np.random.default_rng(1000 + j)
    ends = np.concatenate([np.arange(min(SEG, L)), np.arange(max(0, L - SEG), L)])
    mid_lo, mid_hi = min(SEG, L), max(min(SEG, L), L - SEG)
    pool = mid_hi - mid_lo
    mid = mid_lo + rng.choice(pool, min(N_RANDOM, pool), replace=False) if pool > 0 else []
    loc = [ends, np.asarray(mid, dtype=np.int64)]
    b = (1 << 31) - j * L
    if 2 <= b < L - 2:
        loc.append(np.arange(b - 2, b + 2))
        loc.append(b + rng.choice(L - b, 60, replace=False))
    loc = np.unique(np.concatenate(loc).astype(np.int64))
    return j * L + loc


def error_workers(n):
    return sorted({0, n - 1})


def mid_step(w):
    """0-based step after which the mid checkpoint is taken (for a 0/1 Adam
    workload the local step before it if that is a synchronization, so that
    the checkpoint sees an open local period)."""
    t = w.warmup + max(1, w.compressed // 2) - 1
    if w.method == "zero_one" and w.zo_flags(t)[0] and t > w.warmup:
        t -= 1
    return t


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def digest(a):
    return xxhash.xxh64(np.ascontiguousarray(a).tobytes()).hexdigest()


def chunk_digest(views):
    h = xxhash.xxh64()
    for v in views:
        h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


def checkpoint(o, n, loc, ew, zero_one=False):
    """(digests of whole-chunk fp32 fields, sampled bit patterns); inside an
    open 0/1 Adam local period also every worker's local model."""
    fields = {"x": o._view(oracle.X), "m": o._view(oracle.M), "v": o._view(oracle.V),
              "es": o._view(oracle.E_SERVER)}
    dig = {k: digest(bits32(v)) for k, v in fields.items()}
    dig["e"] = [digest(bits32(o._view(oracle.E_WORKER, i))) for i in range(n)]
    if zero_one and o.zo_open > 0:
        dig["xl"] = [digest(bits32(o.get(oracle.X_LOCAL, i))) for i in range(n)]
    samp = {k: bits32(v[loc]) for k, v in fields.items()}
    samp["e"] = np.stack([bits32(o._view(oracle.E_WORKER, i)[loc]) for i in ew])
    return dig, samp


def run_chunk(name, j, gen_threads=1, log=None):
    w = W.make(name)
    L = w.L
    lo, hi = j * L, (j + 1) * L
    o = oracle.Oracle(w.d, w.n, w.beta1, w.beta2, w.eps, j0=j, j1=j + 1, keep_debug=False)
    idx = sample_indices(w, j)
    loc = idx - lo
    ew = error_workers(w.n)
    tmid = mid_step(w)
    rec = {"workload": name, "chunk": j, "d": w.d, "n": w.n, "L": L,
           "samples": int(idx.size), "idx_digest": digest(idx), "error_workers": ew,
           "mid_t": tmid, "steps": []}
    arrays = {"loc": loc.astype(np.uint32), "ew": np.asarray(ew, dtype=np.int32)}
    pool = cf.ThreadPoolExecutor(gen_threads) if gen_threads > 1 else None
    t0 = time.time()
    for t in range(w.steps):
        if pool:
            g = list(pool.map(lambda i: W.cpu_grad(w, i, t, lo, hi), range(w.n)))
        else:
            g = [W.cpu_grad(w, i, t, lo, hi) for i in range(w.n)]
        lr = w.lr_at(t)
        zo = w.method == "zero_one" and t >= w.warmup
        sync, refresh = w.zo_flags(t) if zo else (True, False)
        if t < w.warmup:
            o.warmup_step(g, lr)
        elif zo:
            o.zo_step(g, lr, sync, refresh)
        else:
            o.compressed_step(g, lr)
        del g
        if t == w.warmup - 1:
            for k, f in (("x", oracle.X), ("m", oracle.M), ("v", oracle.V)):
                arrays["aw_" + k] = bits32(o._view(f)[loc])
        if zo and not sync:  # a 0/1 local step: every worker's momenta over the chunk
            rec["steps"].append({
                "t": t, "lr_bits": int(np.float32(lr).view(np.uint32)), "sync": False,
                "mh": chunk_digest([bits32(o._view(oracle.M_LOCAL, i)) for i in range(w.n)]),
                "ah": chunk_digest([bits32(o._view(oracle.A_LOCAL, i)) for i in range(w.n)])})
        elif t >= w.warmup:
            ws = [int(np.float32(o._view(oracle.SCALE_WORKER, i)[0]).view(np.uint32))
                  for i in range(w.n)]
            ss = int(np.float32(o._view(oracle.SCALE_SERVER)[0]).view(np.uint32))
            rec["steps"].append({
                "t": t, "lr_bits": int(np.float32(lr).view(np.uint32)), "ws": ws, "ss": ss,
                "wh": chunk_digest([o._view(oracle.BITS_WORKER, i) for i in range(w.n)]),
                "sh": chunk_digest([o._view(oracle.BITS_SERVER)])})
            if zo:
                rec["steps"][-1].update(sync=True, refresh=bool(refresh))
        for tag, at in (("mid", tmid), ("fin", w.steps - 1)):
            if t == at:
                dig, samp = checkpoint(o, w.n, loc, ew, w.method == "zero_one")
                rec[tag + "_digest"] = dig
                for k, v in samp.items():
                    arrays["%s_%s" % (tag, k)] = v
        if log:
            log("%s chunk %d step %d/%d  %.0fs" % (name, j, t + 1, w.steps, time.time() - t0))
    rec["t"] = int(o.step)
    o.close()
    if pool:
        pool.shutdown()
    return rec, arrays


def out_path(name, j, ext="json"):
    return os.path.join(HERE, name, "chunk_%d.%s" % (j, ext))


def _job(args):
    name, j, gen_threads = args

    def log(msg):
        print(msg, flush=True)

    rec, arrays = run_chunk(name, j, gen_threads, log)
    os.makedirs(os.path.join(HERE, name), exist_ok=True)
    tmp = out_path(name, j, "npz") + ".tmp.npz"
    np.savez_compressed(tmp, **arrays)
    os.replace(tmp, out_path(name, j, "npz"))
    tmp = out_path(name, j) + ".tmp"
    with open(tmp, "w") as f:
        json.dump(rec, f, separators=(",", ":"))
    os.replace(tmp, out_path(name, j))
    return name, j


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--jobs", type=int, default=1, help="chunks run in parallel processes")
    ap.add_argument("--gen-threads", type=int, default=1,
                    help="threads generating inputs inside each process")
    ap.add_argument("--chunks", default=None, help="comma list overriding the sampled chunks")
    ap.add_argument("--force", action="store_true")
    a = ap.parse_args()
    work = []
    for name in a.workloads:
        chunks = [int(x) for x in a.chunks.split(",")] if a.chunks else SAMPLED[name]
        for j in chunks:
            if a.force or not os.path.exists(out_path(name, j, "npz")):
                work.append((name, j, a.gen_threads))
    with cf.ProcessPoolExecutor(a.jobs) as ex:
        for name, j in ex.map(_job, work):
            print("wrote", out_path(name, j), flush=True)


if __name__ == "__main__":
    main()
