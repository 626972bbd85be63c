"""Parity of the 0/1 Adam step's HIP path (ob_adam_zero_one_step, through
the C interface) with the CPU oracle's ob_oracle_zo_step, and its reduction
to the 1-bit Adam step.

Every field is compared with the oracle after every step, bit for bit: the
shared x, m and v, the worker and server errors, sign words and scales, and
while a local period is open every worker's local momentum, step-weighted
mean momentum and local model.  Schedules mix local steps, synchronizations
and variance refreshes with changing step sizes; worker counts cover every
server form (1, 3, 4, 5, 8, 16, 64), bf16 and fp32 gradients, chunks with a
ragged last segment.  With a synchronization at every step and no refresh
the HIP 0/1 step must equal the HIP 1-bit compressed step bit for bit."""
import numpy as np
import pytest

import oracle
from gpu_common import compare_full, gpu_np, host_grads, log, to_device_grad

pytestmark = pytest.mark.gpu

ob = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global ob
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_compressed_distributed_02_amd import ob_adam
    ob = ob_adam


L, S, R = "local", "sync", "sync+refresh"

SCHEDULES = {
    "every_step": [S] * 5,
    "pairs_refresh_doubling": [L, R, L, R, L, S, L, R],
    "triples": [L, L, S, L, L, R, L, L, S],
    "irregular": [L, L, L, R, S, L, S, L, L, L, L, S],
    "one_period": [L, L, R],
}

CASES = [
    # (name, d, n, bf16, warm, schedule)
    ("n4_ragged_pairs", 4 * 3392, 4, False, 2, "pairs_refresh_doubling"),
    ("n3_generic_triples", 3 * 1472, 3, False, 1, "triples"),
    ("n1_irregular", 2112, 1, False, 1, "irregular"),
    ("n8_bf16_irregular", 8 * 2112, 8, True, 2, "irregular"),
    ("n5_generic_pairs", 5 * 1088, 5, False, 1, "pairs_refresh_doubling"),
    ("n16_triples", 16 * 1152, 16, False, 1, "triples"),
    ("n64_pairs", 64 * 1088, 64, False, 1, "pairs_refresh_doubling"),
    ("n8_every_step", 8 * 2112, 8, True, 2, "every_step"),
    # chunks of 1025 blocks of segments (4 x 1025 >= 4096 blocks): the first
    # local step shares each segment of the fp32 momentum among a block's
    # workers; a ragged last segment of one row
    ("n4_first_local_shared_m", 4 * 4194368, 4, False, 1, "one_period"),
]


def lr_at(t):
    return np.float32(1e-3 * (1.0 + 0.3 * ((7 * t) % 5)))  # changes every step


def compare_local(opt, orc, n, where):
    for w in range(n):
        for name, gf, of in (("m_local", ob.OB_M_LOCAL, oracle.M_LOCAL),
                             ("a_local", ob.OB_A_LOCAL, oracle.A_LOCAL),
                             ("x_local", ob.OB_X_LOCAL, oracle.X_LOCAL)):
            g = gpu_np(opt, gf, w).view(np.uint32)
            r = orc.get(of, w).view(np.uint32)
            if not np.array_equal(g, r):
                i = int(np.flatnonzero(g != r)[0])
                raise AssertionError("%s worker %d %s differs at %d: %r vs %r" % (
                    where, w, name, i, g[i:i + 1].view(np.float32)[0],
                    r[i:i + 1].view(np.float32)[0]))


@pytest.mark.parametrize("name,d,n,bf16,warm,sched", CASES, ids=[c[0] for c in CASES])
def test_zero_one_matches_oracle(name, d, n, bf16, warm, sched, debug=0):
    run_zero_one(name, d, n, bf16, warm, SCHEDULES[sched], debug)


def test_zero_one_random_shapes_match_oracle():
    """Seeded random shapes and schedules: n in 1..64, 1 to 40 rows of 64 per
    chunk, bf16 or fp32, 1 or 2 warm-up steps, then 3 to 7 steps each a local
    step, a synchronization or a synchronization with a variance refresh (so
    a schedule may also open with a synchronization, or synchronize every
    step); every field bit-identical to the oracle after every step."""
    import os
    # OB_ZO_RANDOM_CASES / OB_ZO_RANDOM_SEED widen the sweep for a one-off run
    rng = np.random.default_rng(int(os.environ.get("OB_ZO_RANDOM_SEED", "2025")))
    for case in range(int(os.environ.get("OB_ZO_RANDOM_CASES", "24"))):
        n = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 31, 32, 33, 48, 63, 64]))
        rows = int(rng.integers(1, 41))
        bf16 = bool(rng.integers(0, 2))
        plan = [[L, S, R][int(k)] for k in rng.choice(3, size=int(rng.integers(3, 8)),
                                                      p=[0.5, 0.3, 0.2])]
        run_zero_one("random shape %d" % case, n * 64 * rows, n, bf16, 1 + case % 2, plan)


def run_zero_one(name, d, n, bf16, warm, plan, debug=0):
    import torch
    log("case %s: d=%d n=%d bf16=%s warm=%d schedule=%s debug=%d"
        % (name, d, n, bf16, warm, plan, debug))
    opt = ob.OneBitAdam(d, n, ob.OB_GRAD_BF16 if bf16 else ob.OB_GRAD_F32,
                        method=ob.OB_METHOD_ZERO_ONE)
    if debug:
        ob.ob_adam_set_debug(opt.h, debug)
    orc = oracle.Oracle(d, n)
    sigma = 1e-3 if bf16 else 1e-2
    for t in range(warm + len(plan)):
        hg = host_grads(d, n, t, sigma=sigma, bf16=bf16)
        dg = [to_device_grad(g) for g in hg]
        lr = lr_at(t)
        if t < warm:
            opt.warmup_step(dg, lr)
            orc.warmup_step(hg, lr)
            continue
        kind = plan[t - warm]
        opt.zero_one_step(dg, lr, sync=kind != L, refresh=kind == R)
        orc.zo_step(hg, lr, sync=kind != L, refresh=kind == R)
        torch.cuda.synchronize()
        where = "%s step %d (%s)" % (name, t, kind)
        compare_full(opt, orc, True, exact=True, where=where)
        if kind == L:
            assert orc.zo_open > 0
            compare_local(opt, orc, n, where)
        else:
            with pytest.raises(ob.ObAdamError) as e:
                opt.get(ob.OB_M_LOCAL, 0)
            assert e.value.status == ob.OB_ERR_PHASE
            np.testing.assert_array_equal(gpu_np(opt, ob.OB_X_LOCAL, n - 1), gpu_np(opt, ob.OB_X))
    assert opt.check_guards() == -1, "a kernel wrote past the end of a workspace buffer"


@pytest.mark.parametrize("name", ["n4_ragged_pairs", "n8_bf16_irregular", "n64_pairs",
                                  "n4_first_local_shared_m"])
def test_zero_one_small_launches(name):
    """The local and synchronizing passes cut into launches of one block
    (OB_DEBUG_SMALL_LAUNCHES), against the oracle at every step."""
    d, n, bf16, warm, sched = {c[0]: c[1:] for c in CASES}[name]
    run_zero_one(name, d, n, bf16, warm, SCHEDULES[sched], debug=ob.OB_DEBUG_SMALL_LAUNCHES)


@pytest.mark.parametrize("n,bf16", [(4, False), (8, True), (3, False)])
def test_sync_every_step_equals_the_compressed_step_on_the_gpu(n, bf16):
    """Two GPU handles fed the same gradients: 0/1 steps with a
    synchronization every step and no refresh, and 1-bit compressed steps.
    Every field identical after every step."""
    import torch
    d = n * 3392
    a = ob.OneBitAdam(d, n, ob.OB_GRAD_BF16 if bf16 else ob.OB_GRAD_F32)
    b = ob.OneBitAdam(d, n, ob.OB_GRAD_BF16 if bf16 else ob.OB_GRAD_F32,
                      method=ob.OB_METHOD_ZERO_ONE)
    for t in range(2 + 6):
        dg = [to_device_grad(g) for g in host_grads(d, n, t, sigma=1e-3 if bf16 else 1e-2,
                                                    bf16=bf16)]
        lr = lr_at(t)
        if t < 2:
            a.warmup_step(dg, lr)
            b.warmup_step(dg, lr)
            continue
        a.compressed_step(dg, lr)
        b.zero_one_step(dg, lr, sync=True)
        torch.cuda.synchronize()
        fields = [(ob.OB_X, 0), (ob.OB_M, 0), (ob.OB_V, 0), (ob.OB_E_SERVER, 0),
                  (ob.OB_BITS_SERVER, 0), (ob.OB_SCALE_SERVER, 0)]
        fields += [(f, w) for w in range(n)
                   for f in (ob.OB_E_WORKER, ob.OB_BITS_WORKER, ob.OB_SCALE_WORKER)]
        for f, w in fields:
            assert torch.equal(a.get(f, w), b.get(f, w)), (t, f, w)


def test_phase_and_flag_rules():
    """A 1-bit handle refuses 0/1 steps and a 0/1 handle compressed steps;
    refresh needs a sync; counters only between local periods; the local
    fields belong to 0/1 handles."""
    d, n = 4 * 1088, 4
    dg = [to_device_grad(g) for g in host_grads(d, n, 0)]
    one = ob.OneBitAdam(d, n)
    zo = ob.OneBitAdam(d, n, method=ob.OB_METHOD_ZERO_ONE)
    with pytest.raises(ob.ObAdamError) as e:  # before any warm-up step
        zo.zero_one_step(dg, 1e-3, sync=True)
    assert e.value.status == ob.OB_ERR_PHASE
    with pytest.raises(ob.ObAdamError) as e:
        one.compressed_step(dg, 1e-3)
    assert e.value.status == ob.OB_ERR_PHASE
    one.warmup_step(dg, 1e-3)
    zo.warmup_step(dg, 1e-3)
    with pytest.raises(ob.ObAdamError) as e:
        one.zero_one_step(dg, 1e-3, sync=True)
    assert e.value.status == ob.OB_ERR_PHASE
    with pytest.raises(ob.ObAdamError) as e:
        zo.compressed_step(dg, 1e-3)
    assert e.value.status == ob.OB_ERR_PHASE
    with pytest.raises(ob.ObAdamError) as e:
        zo.compressed_step_static(dg, 1e-3)
    assert e.value.status == ob.OB_ERR_PHASE
    with pytest.raises(ob.ObAdamError) as e:
        zo.zero_one_step(dg, 1e-3, sync=False, refresh=True)
    assert e.value.status == ob.OB_ERR_ARG
    with pytest.raises(ob.ObAdamError) as e:
        ob.ob_adam_zero_one_step(zo.h, [g.data_ptr() for g in dg], 1e-3, 4)
    assert e.value.status == ob.OB_ERR_ARG
    with pytest.raises(ob.ObAdamError) as e:
        one.get(ob.OB_X_LOCAL, 0)
    assert e.value.status == ob.OB_ERR_ARG
    zo.zero_one_step(dg, 1e-3, sync=False)
    with pytest.raises(ob.ObAdamError) as e:
        ob.ob_adam_get_counters(zo.h)
    assert e.value.status == ob.OB_ERR_PHASE
    zo.zero_one_step(dg, 1e-3, sync=True)
    assert ob.ob_adam_get_counters(zo.h) == (3, 2, 1)


def test_checkpoint_resume_between_periods():
    """A 0/1 run checkpointed right after a synchronization and resumed in a
    fresh handle continues bit-identically to the uninterrupted run."""
    import torch
    d, n = 8 * 1088, 8
    plan = [L, S, L, L, R, L, S]
    a = ob.OneBitAdam(d, n, method=ob.OB_METHOD_ZERO_ONE)
    grads = [[to_device_grad(g) for g in host_grads(d, n, t)] for t in range(1 + len(plan))]
    a.warmup_step(grads[0], 1e-3)
    for t, kind in enumerate(plan[:2]):
        a.zero_one_step(grads[1 + t], lr_at(t), sync=kind != L, refresh=kind == R)
    ck = a.checkpoint()
    b = ob.OneBitAdam(d, n, method=ob.OB_METHOD_ZERO_ONE, checkpoint=ck)
    for t, kind in enumerate(plan[2:], start=2):
        for h in (a, b):
            h.zero_one_step(grads[1 + t], lr_at(t), sync=kind != L, refresh=kind == R)
    torch.cuda.synchronize()
    for f, w in [(ob.OB_X, 0), (ob.OB_M, 0), (ob.OB_V, 0), (ob.OB_E_SERVER, 0)] + \
            [(ob.OB_E_WORKER, w) for w in range(n)]:
        assert torch.equal(a.get(f, w), b.get(f, w)), (f, w)
    assert a.steps == b.steps
