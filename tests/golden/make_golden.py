"""Write the stored expected values of the large workloads from the CPU oracle.

Only the oracle (oracle/) and the seeded input generator (synth/) are used;
nothing here touches the GPU path.  Every chunk of the method is independent
of the others, so the oracle runs on whole sampled chunks (all n workers,
every step) and records, per compressed step, the bit patterns of the worker
and server scales of that chunk and xxh64 digests of the worker and server
sign words over that chunk; after the last step it records the state at 256
sampled elements of the chunk (fp32 bit patterns).

    python tests/golden/make_golden.py c2 --jobs 4
writes tests/golden/c2/chunk_<j>.json for the chunks listed in SAMPLED.
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
SAMPLED = {"c1": [0, 1, 2, 3], "c2": list(range(8)), "c3": list(range(16)), "c4": list(range(8)),
           "c5": [0, 3, 7, 11, 15, 19, 23, 27, 31, 35, 39, 43, 47, 51, 55, 59, 63], "idx64": [3]}
N_SAMPLES = 256


def sample_indices(w, j):
    """Sorted global indices of the sampled elements of chunk j (first and last
    included; for a chunk that holds element 2^31, also the elements around it
    and 60 past it)."""
    rng = np.random.default_rng(1000 + j)
    loc = rng.choice(w.L, N_SAMPLES, replace=False)
    loc[0], loc[1] = 0, w.L - 1
    b = (1 << 31) - j * w.L
    if 2 <= b < w.L - 2:
        extra = np.concatenate([np.arange(b - 2, b + 2),
                                b + rng.choice(w.L - b, 60, replace=False)])
        loc = np.unique(np.concatenate([loc, extra]))
    loc.sort()
    return j * w.L + loc


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).tolist()


def chunk_digest(views):
    h = xxhash.xxh64()
    for v in views:
        h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()


def run_chunk(name, j, gen_threads=1, log=None):
    w = W.make(name)
    L = w.L
    lo, hi = j * L, (j + 1) * L
    o = oracle.Oracle(w.d, w.n, w.beta1, w.beta2, w.eps, j0=j, j1=j + 1, keep_debug=False)
    idx = sample_indices(w, j)
    loc = idx - lo
    rec = {"workload": name, "chunk": j, "d": w.d, "n": w.n, "L": L, "idx": idx.tolist(),
           "steps": []}
    pool = cf.ThreadPoolExecutor(gen_threads) if gen_threads > 1 else None
    t0 = time.time()
    for t in range(w.steps):
        if pool:
            g = list(pool.map(lambda i: W.cpu_grad(w, i, t, lo, hi), range(w.n)))
        else:
            g = [W.cpu_grad(w, i, t, lo, hi) for i in range(w.n)]
        lr = w.lr_at(t)
        if t < w.warmup:
            o.warmup_step(g, lr)
        else:
            o.compressed_step(g, lr)
        del g
        if t == w.warmup - 1:
            rec["after_warmup"] = {k: f32_bits(o._view(f)[loc]) for k, f in
                                   (("x", oracle.X), ("m", oracle.M), ("v", oracle.V))}
        if t >= w.warmup:
            ws = [int(np.float32(o._view(oracle.SCALE_WORKER, i)[0]).view(np.uint32))
                  for i in range(w.n)]
            ss = int(np.float32(o._view(oracle.SCALE_SERVER)[0]).view(np.uint32))
            rec["steps"].append({
                "t": t, "lr_bits": int(np.float32(lr).view(np.uint32)), "ws": ws, "ss": ss,
                "wh": chunk_digest([o._view(oracle.BITS_WORKER, i) for i in range(w.n)]),
                "sh": chunk_digest([o._view(oracle.BITS_SERVER)])})
        if log:
            log("%s chunk %d step %d/%d  %.0fs" % (name, j, t + 1, w.steps, time.time() - t0))
    rec["final"] = {"x": f32_bits(o._view(oracle.X)[loc]), "m": f32_bits(o._view(oracle.M)[loc]),
                    "v": f32_bits(o._view(oracle.V)[loc]),
                    "es": f32_bits(o._view(oracle.E_SERVER)[loc]),
                    "e": [f32_bits(o._view(oracle.E_WORKER, i)[loc]) for i in range(w.n)]}
    rec["t"] = int(o.step)
    o.close()
    if pool:
        pool.shutdown()
    return rec


def out_path(name, j):
    return os.path.join(HERE, name, "chunk_%d.json" % j)


def _job(args):
    name, j, gen_threads = args

    def log(msg):
        print(msg, flush=True)

    rec = run_chunk(name, j, gen_threads, log)
    os.makedirs(os.path.join(HERE, name), exist_ok=True)
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
            if a.force or not os.path.exists(out_path(name, j)):
                work.append((name, j, a.gen_threads))
    with cf.ProcessPoolExecutor(a.jobs) as ex:
        for name, j in ex.map(_job, work):
            print("wrote", out_path(name, j), flush=True)


if __name__ == "__main__":
    main()
