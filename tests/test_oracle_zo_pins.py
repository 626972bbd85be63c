"""Pins of the oracle's 0/1 Adam step ("Maximizing Communication Efficiency
for Large-scale Training via 0/1 Adam", abstract) against what the page and
the mathematics fix, independent of the oracle's own code:

 - the step is linear in the gradients while the state is stale: inside a
   local period a worker's model is the sum of its Adam-like steps taken
   with the frozen variance (checked against a float64 re-derivation of the
   sequential local steps, with step sizes that change every step, so that a
   wrongly weighted mean momentum fails), and the local model and mean
   momentum are affine in the gradients (difference checks);
 - 1-bit compression with error feedback is the compressed step's codec:
   with a synchronization at every step and no variance refresh the 0/1
   step equals the 1-bit Adam compressed step bit for bit, over many steps;
 - a synchronization averages the workers' local models through the
   communicated mean momenta: in exact dyadic cases (where the 1-bit codec
   loses nothing) the new shared model is the mean of the local models and
   the shared momentum the mean of the mean momenta, bitwise;
 - the variance refresh is Adam's second-moment step on the full-precision
   worker average, taken after the model update of its synchronizing step
   (exact dyadic case);
 - a synchronization closes the local period and the next step starts from
   the shared momentum and model.

What the abstract leaves open -- the refresh and synchronization schedules
(the caller's flags), the placement of the refresh after the update, the
incremental form of the step-weighted mean -- is recorded as readings; the
trajectories of the 0/1 workloads are parity unpinned beyond these
invariants."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def grads(d, n, t, sigma=1e-2, bf16=False, seed=1234):
    return [synth.fill_cpu(d, 0, t, w, sigma=sigma, bf16=bf16, seed=seed) for w in range(n)]


def f32(x):
    return np.float32(x)


@pytest.mark.parametrize("d,n,bf16", [(4 * 3392, 4, False), (3 * 1472, 3, True),
                                      (8 * 1088, 8, False), (1024, 1, False)])
def test_sync_every_step_without_refresh_is_the_compressed_step(d, n, bf16):
    """0/1 Adam with no local steps and a stale (never refreshed) variance is
    1-bit Adam's compression phase, bit for bit, field by field."""
    a = oracle.Oracle(d, n)
    b = oracle.Oracle(d, n)
    warm, steps = 2, 7
    for t in range(warm + steps):
        g = grads(d, n, t, 1e-3 if bf16 else 1e-2, bf16)
        lr = f32(1e-3 * (1.0 + 0.25 * t))  # a schedule: the sum of one step size is that step size
        if t < warm:
            a.warmup_step(g, lr)
            b.warmup_step(g, lr)
            continue
        a.compressed_step(g, lr)
        b.zo_step(g, lr, sync=True)
        assert b.zo_open == 0
        for f in (oracle.X, oracle.M, oracle.V, oracle.E_SERVER, oracle.BITS_SERVER,
                  oracle.SCALE_SERVER):
            assert a.get(f).tobytes() == b.get(f).tobytes(), (t, f)
        for w in range(n):
            for f in (oracle.E_WORKER, oracle.BITS_WORKER, oracle.SCALE_WORKER):
                assert a.get(f, w).tobytes() == b.get(f, w).tobytes(), (t, f, w)
    assert a.step == b.step


def _posed(d, n, seed):
    """An oracle after one warm-up step (a positive variance, a momentum)."""
    o = oracle.Oracle(d, n)
    o.warmup_step(grads(d, n, 0, seed=seed), f32(1e-3))
    return o


@pytest.mark.parametrize("k", [2, 3, 5])
def test_local_models_are_the_sequential_local_steps(k):
    """Inside a local period (no synchronization) each worker's model equals
    x_sync minus its Adam-like steps with the frozen variance, taken one
    after another (float64 re-derivation), and its mean momentum is the
    step-size-weighted mean of its momenta: the linearization of the page.
    Step sizes change every step, so an unweighted mean fails."""
    d, n = 2 * 1088, 2
    b1 = np.float64(np.float32(0.9))
    o = _posed(d, n, 7)
    x0 = o.get(oracle.X).astype(np.float64)
    m0 = o.get(oracle.M).astype(np.float64)
    v = o.get(oracle.V).astype(np.float64)
    eps = np.float64(np.float32(1e-8))
    lrs = [f32(1e-3 * (1 + 0.7 * j)) for j in range(k)]
    gs = [grads(d, n, 10 + j, seed=99) for j in range(k)]
    for j in range(k):
        o.zo_step(gs[j], lrs[j], sync=False)
    assert o.zo_open == k
    gsum = sum(np.float64(l) for l in lrs)
    assert abs(np.float64(o.zo_gamma) - gsum) <= 4 * k * np.finfo(np.float32).eps * gsum
    assert o.get(oracle.X).tobytes() == np.float32(x0).tobytes()  # the shared model waits
    u = 2.0 ** -24  # fp32 unit roundoff
    for w in range(n):
        m = m0.copy()
        x = x0.copy()
        num = np.zeros(d)
        mags = np.abs(m0)  # elementwise sum of the magnitudes that enter m
        for j in range(k):
            gj = gs[j][w].astype(np.float64)
            m = b1 * m + (1 - b1) * gj
            x = x - np.float64(lrs[j]) * m / (np.sqrt(v) + eps)
            num += np.float64(lrs[j]) * m
            mags = mags + np.abs(m) + np.abs(gj)
        mloc = o.get(oracle.M_LOCAL, w).astype(np.float64)
        aloc = o.get(oracle.A_LOCAL, w).astype(np.float64)
        xloc = o.get(oracle.X_LOCAL, w).astype(np.float64)
        # each fp32 operation rounds by at most u relative to its operands, so
        # the errors are bounded by the magnitudes that enter (cancellation
        # in the mean momentum is allowed for)
        tol_m = 8 * u * mags
        tol_a = (8 + 16 * k) * u * mags
        assert np.all(np.abs(mloc - m) <= tol_m), w
        assert np.all(np.abs(aloc - num / gsum) <= tol_a), w
        tol_x = gsum * tol_a / (np.sqrt(v) + eps) + 8 * u * (np.abs(x0) + np.abs(x - x0))
        assert np.all(np.abs(xloc - x) <= tol_x), w
        # the unweighted mean of the momenta misses by far more than that
        plain = np.zeros(d)
        mm = m0.copy()
        for j in range(k):
            mm = b1 * mm + (1 - b1) * gs[j][w].astype(np.float64)
            plain += mm / k
        assert np.mean(np.abs(aloc - plain) > tol_a) > 0.5


def test_local_period_is_affine_in_the_gradients():
    """With the state stale, a period's mean momentum is affine in the
    gradients: mean(g + h) - mean(g) = mean(h) - mean(0), to rounding."""
    d, n, k = 1088, 1, 3
    lrs = [f32(2e-3), f32(1e-3), f32(3e-3)]
    gs = [grads(d, n, 20 + j, seed=5) for j in range(k)]
    hs = [grads(d, n, 30 + j, seed=6) for j in range(k)]
    zs = [[np.zeros(d, dtype=np.float32)] for _ in range(k)]

    def run(seq):
        o = _posed(d, n, 3)
        for j in range(k):
            o.zo_step(seq[j], lrs[j], sync=False)
        return o.get(oracle.A_LOCAL, 0).astype(np.float64)
    a_g = run(gs)
    a_h = run(hs)
    a_gh = run([[gs[j][0] + hs[j][0]] for j in range(k)])
    a_0 = run(zs)
    lhs = a_gh - a_g
    rhs = a_h - a_0
    tol = 64 * 2.0 ** -24 * (np.abs(a_gh) + np.abs(a_g) + np.abs(a_h) + np.abs(a_0))
    assert np.all(np.abs(lhs - rhs) <= tol)


def _dyadic(o, n, L, vals_m, vals_v):
    """Pose chunks of constant m and v (exact dyadic values), x = 0."""
    d = n * L
    o.set(oracle.X, np.zeros(d, dtype=np.float32))
    o.set(oracle.M, np.repeat(np.float32(vals_m), L))
    o.set(oracle.V, np.repeat(np.float32(vals_v), L))


def test_sync_averages_the_local_models_exactly():
    """beta1 = 1/2, eps = 0, v = 1, constant gradients per (worker, chunk),
    step sizes 1/2 and 1/2 (weights 1 and 1/2 in the mean momentum), chunks
    of 64 so every scale is exact: after a local step the workers' models
    are x_sync minus their own steps; after the synchronizing second step
    the shared momentum is the mean of the workers' step-weighted mean
    momenta and the shared model the mean of their local models, bitwise,
    with every error 0 (the codec loses nothing here)."""
    n, L = 4, 64
    d = n * L
    o = oracle.Oracle(d, n, beta1=0.5, beta2=0.75, eps=0.0)
    _dyadic(o, n, L, [1.0, -2.0, 0.5, 4.0], [1.0, 1.0, 1.0, 1.0])
    # worker w, chunk j: gradient gv[w][j] at both steps
    gv = np.array([[2.0, 4.0, -1.0, 8.0], [6.0, 0.0, 1.0, 0.0],
                   [-2.0, -4.0, 3.0, 8.0], [2.0, 8.0, -3.0, 0.0]], dtype=np.float64)
    g = [np.repeat(np.float32(gv[w]), L) for w in range(n)]
    lrs = [Fraction(1, 2), Fraction(1, 2)]
    m0 = [Fraction(1), Fraction(-2), Fraction(1, 2), Fraction(4)]

    def local(w, steps):
        """(mean momentum, local model) of worker w after `steps` local steps,
        exactly: x = -sum(lr_k m_k) (v = 1, eps = 0), a = sum(lr_k m_k)/sum(lr_k)."""
        mw, num, x = list(m0), [Fraction(0)] * n, [Fraction(0)] * n
        for lr in lrs[:steps]:
            mw = [Fraction(1, 2) * mw[j] + Fraction(1, 2) * Fraction(gv[w][j]) for j in range(n)]
            num = [num[j] + lr * mw[j] for j in range(n)]
            x = [x[j] - lr * mw[j] for j in range(n)]
        return [num[j] / sum(lrs[:steps]) for j in range(n)], x

    def rep(vals):
        return np.repeat(np.float32([float(v) for v in vals]), L).tobytes()

    o.zo_step(g, f32(0.5), sync=False)
    for w in range(n):
        a1, x1 = local(w, 1)
        assert o.get(oracle.A_LOCAL, w).tobytes() == rep(a1), w
        assert o.get(oracle.X_LOCAL, w).tobytes() == rep(x1), w
    o.zo_step(g, f32(0.5), sync=True)
    ends = [local(w, 2) for w in range(n)]
    mean_a = [sum(ends[w][0][j] for w in range(n)) / n for j in range(n)]
    mean_x = [sum(ends[w][1][j] for w in range(n)) / n for j in range(n)]
    assert o.get(oracle.M).tobytes() == rep(mean_a)
    assert o.get(oracle.X).tobytes() == rep(mean_x)
    assert not np.any(o.get(oracle.E_SERVER))
    for w in range(n):
        assert not np.any(o.get(oracle.E_WORKER, w))
    assert o.zo_open == 0
    # after the synchronization every local model is the shared model again
    for w in range(n):
        assert o.get(oracle.X_LOCAL, w).tobytes() == o.get(oracle.X).tobytes()


def test_refresh_is_adam_second_moment_after_the_update():
    """beta2 = 3/4: v = (3/4)v + (1/4)gbar^2 on the pairwise worker average of
    the synchronizing step's gradients, and the model update of that step
    uses the old variance (v = 1 -> step m/1; the new v = 4 would halve it)."""
    n, L = 2, 64
    d = n * L
    o = oracle.Oracle(d, n, beta1=0.5, beta2=0.75, eps=0.0)
    _dyadic(o, n, L, [2.0, 2.0], [1.0, 1.0])
    # gradients 2 and 6: gbar 4, v = (3/4)*1 + (1/4)*16 = 4.75; momenta
    # (1/2)*2 + (1/2)*2 = 2 and (1/2)*2 + (1/2)*6 = 4, mean 3 (exact through
    # the codec), so x = 0 - (1/2)*(3/sqrt(1)) with the old variance
    g = [np.full(d, 2.0, dtype=np.float32), np.full(d, 6.0, dtype=np.float32)]
    o.zo_step(g, f32(0.5), sync=True, refresh=True)
    assert np.all(o.get(oracle.V) == np.float32(4.75))
    assert np.all(o.get(oracle.M) == np.float32(3.0))
    assert np.all(o.get(oracle.X) == np.float32(-1.5))
    # without the refresh flag the variance stays
    o.zo_step(g, f32(0.5), sync=True)
    assert np.all(o.get(oracle.V) == np.float32(4.75))


def test_refresh_only_at_a_synchronization():
    o = oracle.Oracle(128, 2)
    with pytest.raises(ValueError):
        o.zo_step([np.zeros(128, np.float32)] * 2, f32(1e-3), sync=False, refresh=True)


def test_period_restarts_from_the_shared_momentum():
    """After a synchronization the next local step starts from the shared
    (decompressed) momentum, not from the worker's own: two workers whose
    local momenta differed leave the first step of the next period with
    momenta that differ only by their gradients."""
    d, n = 1088, 2
    o = _posed(d, n, 11)
    g = grads(d, n, 40)
    o.zo_step(g, f32(1e-3), sync=False)
    o.zo_step(g, f32(1e-3), sync=True)
    shared = o.get(oracle.M)
    z = [np.zeros(d, np.float32)] * n
    o.zo_step(z, f32(1e-3), sync=False)
    want = np.float32(0.9) * shared  # (b1 * m) + ((1 - b1) * 0)
    for w in range(n):
        assert o.get(oracle.M_LOCAL, w).tobytes() == want.tobytes()
        assert o.get(oracle.A_LOCAL, w).tobytes() == want.tobytes()
