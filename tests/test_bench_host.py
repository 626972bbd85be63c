"""Host logic of the benchmark, on the CPU: the algorithmic byte counts the
roofline is priced with, the selection of counter records, and the refusal
of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import workloads as W  # noqa: E402

NAMES = ["c1", "c2", "c3", "c4", "c5"]


@pytest.mark.parametrize("name", NAMES)
def test_step_bytes_follow_the_per_element_terms(name):
    """Per (element, worker): gradient, compensated momentum in and out, sign
    word out and read back by the server (gb + 8.25); per element: momentum
    words read by each worker-pass launch, server u in and out and its words
    out, update words, x in and out and v in (20.375 with one launch).  The
    step must equal d*[n*(gb + 8.25) + 20.375] + (launches - 1)*d/8 plus the
    segment partials and scales (momentum held as server sign words); the
    fp32-momentum count is d*[n*(gb + 8.25) + 28.125]."""
    w = W.make(name)
    d, n = w.d, w.n
    gb = 2 if w.bf16 else 4
    nseg = -(-w.L // 1024)
    ab = bench.alg_bytes(w)
    assert set(ab) == {"worker", "worker_scale", "server", "server_scale", "update"}
    nquad = -(-nseg // 4)  # partials per block of 4 segments...
    sparts = nseg if n in (32, 64) else nquad  # ...but per segment in the 32/64-worker server
    partials = 2 * 8 * n * n * nquad + 2 * 8 * n * sparts  # written once, read once
    small = 4 * n * n + 4 * n + 4 * n * n + 4 * n       # scales
    launches = n if w.staged else 1
    # exact in eighths: scale everything by 8
    want8 = d * (n * (8 * gb + 66) + 163) + (launches - 1) * d + 8 * (partials + small)
    assert 8 * sum(ab.values()) == want8
    assert bench.fp32_momentum_step_bytes(w) == d * (n * (gb + 8.25) + 28.125)
    # with one worker-pass launch, the compact layout moves fewer bytes than
    # the fp32-momentum count (per-worker launches re-read the momentum words)
    if not w.staged:
        assert sum(ab.values()) < bench.fp32_momentum_step_bytes(w)


def test_bytes_match_the_stated_c2_figures():
    ab = bench.alg_bytes(W.make("c2"))
    assert ab["worker"] == 8925479168
    assert sum(ab.values()) == 11265130944


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("steps", [1, 3, 5, 20])
def test_cpu_baseline_sample_is_bounded(name, steps):
    """The CPU leg's oracle work stays within its budget (or is the least
    sample there is: one warm-up and one compressed step), and keeps the
    workload's own warm-up and the requested steps (so that its state can be
    compared with the GPU's) wherever they fit."""
    w = W.make(name)
    warm, k = bench.cpu_plan(w, steps)
    unit = w.n * w.L
    assert 1 <= k <= steps
    assert (warm + k) * unit <= bench.CPU_BUDGET or (warm, k) == (1, 1)
    if (w.warmup + steps) * unit <= bench.CPU_BUDGET:
        assert (warm, k) == (w.warmup, steps)
    else:
        assert warm == 1


def test_default_workload_is_the_largest_config():
    """The headline runs the 64-worker BERT-Large workload: the most
    params x workers and the most bytes per step of all workloads."""
    def size(nm):
        w = W.make(nm)
        return w.n * w.d, sum(bench.alg_bytes(w).values())
    assert bench.DEFAULT_WORKLOAD == "c5"
    for nm in NAMES:
        assert size(nm) <= size("c5")


def test_traffic_records_are_per_workload_and_kernel_code(tmp_path, monkeypatch):
    sha = bench.kernel_sha()
    rec = {"workload": "c3", "kernel_source_sha": sha, "kernel": "worker pass",
           "bytes_per_pass": 123, "step_bytes": 456}
    (tmp_path / "worker_pass_c3_counters.txt").write_text(
        "summary\ntraffic_record: " + json.dumps(rec) + "\n")
    stale = dict(rec, workload="c4", kernel_source_sha="0" * 16)
    (tmp_path / "worker_pass_c4_counters.txt").write_text(
        "traffic_record: " + json.dumps(stale) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "worker_pass_%s_counters.txt"))
    assert bench.load_traffic("c3")["bytes_per_pass"] == 123
    assert bench.load_traffic("c4") is None   # taken on other kernel code
    assert bench.load_traffic("c2") is None   # no record


def test_committed_records_name_their_workload():
    for name in NAMES:
        path = bench.TRAFFIC_FILE % name
        if not os.path.exists(path):
            continue
        lines = [ln for ln in open(path) if ln.startswith("traffic_record: ")]
        assert len(lines) == 1
        rec = json.loads(lines[0][len("traffic_record: "):])
        assert rec["workload"] == name
        assert rec["bytes_per_pass"] > 0 and rec["step_bytes"] >= rec["bytes_per_pass"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", ["z2", "z3"])
def test_zero_one_schedule_and_bytes(name):
    """0/1 workloads: a synchronization every second step, refreshes at the
    1st, 2nd, 4th, 8th ... synchronization; the synchronizing worker pass
    moves gradient + local, mean and compensated momentum in and the
    compensated momentum out (16 B + gb per element and worker), the local
    step gradient in and both momenta out (8 B + gb)."""
    w = W.make(name)
    flags = [w.zo_flags(t) for t in range(w.warmup, w.warmup + 20)]
    assert [s for s, _ in flags] == [False, True] * 10
    refreshed = [k + 1 for k, (s, r) in enumerate([f for f in flags if f[0]]) if r]
    assert refreshed == [1, 2, 4, 8]
    gb = 2 if w.bf16 else 4
    ab = bench.zo_alg_bytes(w)
    assert ab["zo_local"] == w.n * w.d * (gb + 8) + w.d // 8
    nquad = -(-(-(-w.L // 1024)) // 4)
    assert ab["worker"] == w.n * w.d * (gb + 16) + w.n * w.d // 8 + 8 * w.n * w.n * nquad
    assert ab["zo_refresh"] == w.n * w.d * gb + 8 * w.d


def test_profiled_dispatch_counts_follow_the_launch_partition():
    """The committed kernel traces (rocprofv3 dispatch counts) against
    bench.dispatches_per_pass, the library's rule for cutting a pass into
    launches: over a traced run of W + 2S compressed steps (--warmup W,
    --steps S, both timing regions), the steady worker kernel dispatches
    (W + 2S - 1) passes (the first step runs worker_first_kernel), the
    server pass and the update W + 2S each."""
    import re
    for name in ("c1", "c2", "c3", "c4", "c5"):
        path = bench.TRACE_FILE % name
        if not os.path.exists(path):
            continue
        text = open(path).read()
        steps = int(re.search(r"--steps (\d+)", text).group(1))
        warm = int(re.search(r"--warmup (\d+)", text).group(1))
        calls = {}
        for line in text.splitlines():
            m = re.match(r"(\w+_kernel(?:<[^>]*>)?)\s+(\d+)\s+[\d.]+\s+[\d.]+\s+[\d.]+", line)
            if m:
                calls[m.group(1)] = int(m.group(2))
        w = W.make(name)
        dpp = bench.dispatches_per_pass(w)
        per = w.n if w.staged else 1
        comp = warm + 2 * steps
        worker = [k for k in calls if k.startswith("worker_kernel")]
        server = [k for k in calls if k.startswith("server")]
        update = [k for k in calls if k.startswith("update_kernel")]
        assert len(worker) == len(server) == len(update) == 1, (name, sorted(calls))
        assert calls[worker[0]] == (comp - 1) * per * dpp["worker"], name
        assert calls[server[0]] == comp * dpp["server"], name
        assert calls[update[0]] == comp * dpp["update"], name
