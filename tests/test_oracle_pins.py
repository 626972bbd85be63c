"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test names what fixes the expected value: textbook Adam (the "Adam: A
Method for Stochastic Optimization" entry the 1-bit Adam page builds on),
exact rational arithmetic, closed forms of 1-bit compression with per-chunk
scaling, error-feedback conservation, and structural identities (n identical
workers, chunk independence).  The method itself is the one of "1-bit Adam:
Communication Efficient Large-Scale Training with Adam's Convergence Speed"
(Abstract) and the LIT-278 record (Key takeaways; tag lines SOTA-214/215).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

F32 = np.float32


def decode_bits(words, count):
    """Sign bits of elements 0..count-1: bit k%64 of little-endian word k//64."""
    b = np.unpackbits(np.ascontiguousarray(words, dtype="<u8").view(np.uint8), bitorder="little")
    return b[:count].astype(bool)


def decompress(words, scales, L):
    bits = decode_bits(words, L * len(scales))
    s = np.repeat(np.asarray(scales, dtype=np.float32), L)
    return np.where(bits, s, -s)


def f32_neighbours(f):
    f = np.float32(f)
    return np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))


def exact_scale_f32(c):
    """Correctly rounded fp32 of sqrt(sum(c^2)/L), from exact rationals."""
    X = sum((Fraction(float(v)) ** 2 for v in c), Fraction(0)) / len(c)
    guess = np.float32(math.sqrt(float(X)))
    for _ in range(4):
        lo, f, hi = f32_neighbours(guess)
        lo_mid = (Fraction(float(lo)) + Fraction(float(f))) / 2
        hi_mid = (Fraction(float(f)) + Fraction(float(hi))) / 2
        if X < lo_mid * lo_mid:
            guess = lo
        elif X > hi_mid * hi_mid:
            guess = hi
        else:
            return f, X
    return guess, X


def ulp_distance(a, b):
    ia = np.array([a], dtype=np.float32).view(np.int32)[0]
    ib = np.array([b], dtype=np.float32).view(np.int32)[0]
    return abs(int(ia) - int(ib))


# ---------------------------------------------------------------- scale ----

@pytest.mark.parametrize("L", [1, 7, 63, 64, 1000, 1023, 1024, 1025, 4096, 5000, 70000])
def test_scale_within_one_ulp_of_exact_norm(L):
    """scale = ||c||_2 / sqrt(L): the oracle's fixed-order fp64 sum and its
    single rounding land within 1 fp32 ulp of the exact rational value."""
    rng = np.random.default_rng(L)
    c = (rng.standard_normal(L) * rng.choice([1e-3, 1.0, 30.0], L)).astype(np.float32)
    S = oracle.chunk_sumsq(c)
    want, X = exact_scale_f32(c)
    exact_S = X * L
    assert abs(Fraction(S) - exact_S) <= exact_S * Fraction(L, 2 ** 52)
    s = oracle.chunk_scale(S, L)
    assert ulp_distance(s, want) <= 1


@pytest.mark.parametrize("j,k", [(0, 0), (1, 3), (3, 7), (5, 10)])
def test_constant_chunk_scale_is_exact(j, k):
    """A chunk of 4^j copies of 2^-k has norm 2^j * 2^-k, so the scale is 2^-k exactly."""
    L = 4 ** j
    c = np.full(L, 2.0 ** -k, dtype=np.float32)
    assert oracle.chunk_scale(oracle.chunk_sumsq(c), L) == np.float32(2.0 ** -k)


def test_sumsq_counts_every_element_once():
    """Indicator chunks: the square of exactly one element reaches the sum."""
    for L in (1, 64, 1000, 1024, 3000, 9000):
        for pos in sorted({0, L // 2, L - 1}):
            c = np.zeros(L, dtype=np.float32)
            c[pos] = 3.0
            assert oracle.chunk_sumsq(c) == 9.0


# -------------------------------------------------------------- average ----

def test_pairwise_mean_of_identical_values_is_exact():
    for n in (1, 2, 4, 8, 16, 64):
        v = np.full(n, np.float32(0.3), dtype=np.float32)
        assert oracle.pairwise_mean(v) == np.float32(0.3)


def test_pairwise_mean_tree_shape():
    """Pairs (2i, 2i+1) level by level, an odd tail passes up: with one large
    value and tiny ones the grouping decides whether the tiny ones survive."""
    big, tiny = np.float32(1.0), np.float32(2.0 ** -24)
    # n = 3: (big + tiny) + tiny -> both tiny values are absorbed one at a time
    assert oracle.pairwise_mean(np.array([big, tiny, tiny], np.float32)) == np.float32(1.0) / np.float32(3)
    # n = 3 with the big one last: (tiny + tiny) + big keeps 2^-23
    r = oracle.pairwise_mean(np.array([tiny, tiny, big], np.float32))
    assert r == (np.float32(1.0) + np.float32(2.0 ** -23)) / np.float32(3)
    # n = 4: (1 + t) + (-1 + t): the first tiny is absorbed, the second kept
    r = oracle.pairwise_mean(np.array([big, tiny, -big, tiny], np.float32))
    assert r == np.float32(2.0 ** -24) / np.float32(4)
    # n = 5: ((t+t) + (t+t)) + big keeps 4*tiny = 2^-22
    r = oracle.pairwise_mean(np.array([tiny] * 4 + [big], np.float32))
    assert r == (np.float32(1.0) + np.float32(2.0 ** -22)) / np.float32(5)


# ------------------------------------------------------------- warm-up -----

def textbook_adam(grads_per_step, lr, b1, b2, eps, d):
    """Adam with bias correction in float64 (Kingma and Ba, Algorithm 1)."""
    m = np.zeros(d)
    v = np.zeros(d)
    x = np.zeros(d)
    for t, g in enumerate(grads_per_step, start=1):
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        x = x - lr * mh / (np.sqrt(vh) + eps)
    return x, m, v


def test_warmup_equals_textbook_adam():
    d, n, steps, lr = 4096, 4, 6, 1e-3
    o = oracle.Oracle(d, n)
    gbar = []
    for t in range(steps):
        g = [synth.fill_cpu(d, 0, t, w, sigma=1e-2) for w in range(n)]
        o.warmup_step(g, lr)
        gbar.append(np.mean(np.stack(g).astype(np.float64), axis=0))
    b1, b2 = float(F32(0.9)), float(F32(0.999))
    x, m, v = textbook_adam(gbar, lr, b1, b2, 1e-8, d)
    # m is a signed sum and may cancel: bound its error by the sum of the
    # magnitudes that went into it (fp32 rounding, a few ulps per step)
    mag = np.zeros(d)
    for g in gbar:
        mag = b1 * mag + (1 - b1) * np.abs(g)
    assert np.all(np.abs(o.get(oracle.M) - m) <= 8 * steps * 2.0 ** -24 * mag)
    np.testing.assert_allclose(o.get(oracle.V), v, rtol=2e-5, atol=1e-16)
    # x accumulates `steps` updates of size ~lr each
    np.testing.assert_allclose(o.get(oracle.X), x, rtol=0, atol=steps * lr * 2e-5)
    assert o.step == steps


def test_first_warmup_step_closed_form():
    """After one bias-corrected step m_hat = g and v_hat = g^2, so
    x1 = x0 - lr * g / (|g| + eps)."""
    d, n, lr = 2048, 2, 1e-3
    o = oracle.Oracle(d, n)
    g = [synth.fill_cpu(d, 0, 0, w, sigma=1e-2) for w in range(n)]
    o.warmup_step(g, lr)
    gbar = (g[0].astype(np.float64) + g[1]) / 2
    want = -lr * gbar / (np.abs(gbar) + 1e-8)
    np.testing.assert_allclose(o.get(oracle.X), want, rtol=1e-5, atol=1e-11)


# ----------------------------------------------- exact compression cases ---

def _exact_oracle(d, n):
    """beta1 = 1/2 and eps = 0 keep every fp32 operation of these cases exact."""
    o = oracle.Oracle(d, n, beta1=0.5, beta2=0.999, eps=0.0)
    return o


def test_codec_round_trip_single_worker():
    """n = 1: compress then decompress returns scale * sign(c), sign(0) = +1,
    with scale = ||c||_2/sqrt(L) (L = 4^6 so the server keeps it exactly)."""
    d = 4096
    o = oracle.Oracle(d, 1)
    rng = np.random.default_rng(7)
    o.set(oracle.M, rng.standard_normal(d).astype(np.float32) * F32(0.01))
    o.set(oracle.V, np.full(d, 1e-4, np.float32))
    g = rng.standard_normal(d).astype(np.float32) * F32(0.01)
    g[::97] = 0
    o.compressed_step([g], 1e-3)
    c = o.get(oracle.C_WORKER)
    s = o.get(oracle.SCALE_WORKER)[0]
    want, _ = exact_scale_f32(c)
    assert ulp_distance(s, want) <= 1
    sign = np.where(c >= 0, F32(1), F32(-1))
    np.testing.assert_array_equal(o.get(oracle.M), s * sign)
    assert o.get(oracle.SCALE_SERVER)[0] == s
    np.testing.assert_array_equal(o.get(oracle.E_SERVER), np.zeros(d, np.float32))
    np.testing.assert_array_equal(o.get(oracle.E_WORKER), c - s * sign)


def test_error_feedback_exact_pattern():
    """Chunk [11,5,5,5]: norm 14, scale 7, error [4,-2,-2,-2]; next step the
    error is added back to the momentum (error feedback on the momentum)."""
    o = _exact_oracle(4, 1)
    g1 = np.array([22, 10, 10, 10], np.float32)            # c = g/2
    o.compressed_step([g1], 2.0 ** -10)
    np.testing.assert_array_equal(o.get(oracle.C_WORKER), [11, 5, 5, 5])
    assert o.get(oracle.SCALE_WORKER)[0] == 7
    np.testing.assert_array_equal(o.get(oracle.E_WORKER), [4, -2, -2, -2])
    np.testing.assert_array_equal(o.get(oracle.M), [7, 7, 7, 7])
    # m = 7: c2 = m/2 + g/2 + e = 3.5 + 3.5 + e = [11, 5, 5, 5] again
    o.compressed_step([np.full(4, 7, np.float32)], 2.0 ** -10)
    np.testing.assert_array_equal(o.get(oracle.C_WORKER), [11, 5, 5, 5])
    np.testing.assert_array_equal(o.get(oracle.E_WORKER), [4, -2, -2, -2])
    assert o.step == 2


def test_server_average_error_feedback_and_update_exact():
    """Two workers, two chunks of 4, every value dyadic so nothing rounds.
    Step 1: worker scales (16, 6) on chunk 0 and (6, 2) on chunk 1; server
    average [11,5,5,5] -> server scale 7, server error [4,-2,-2,-2].
    Step 2: the average is 7 everywhere on chunk 0 and the server error turns
    it into [11,5,5,5] again; chunk 1 averages to 0 (scale 0, sign(0) = +1).
    Update with frozen v = 4 and eps = 0: x -= lr * m / 2."""
    o = _exact_oracle(8, 2)
    o.set(oracle.V, np.full(8, 4, np.float32))
    lr = 2.0 ** -10
    g0 = np.array([64, 0, 0, 0, 12, 12, 12, 12], np.float32)
    g1 = np.array([12, -12, -12, -12, 4, 4, 4, 4], np.float32)
    o.compressed_step([g0, g1], lr)
    np.testing.assert_array_equal(o.get(oracle.SCALE_WORKER, 0), [16, 6])
    np.testing.assert_array_equal(o.get(oracle.SCALE_WORKER, 1), [6, 2])
    np.testing.assert_array_equal(o.get(oracle.E_WORKER, 0), [16, -16, -16, -16, 0, 0, 0, 0])
    np.testing.assert_array_equal(o.get(oracle.E_WORKER, 1), np.zeros(8))
    assert int(o.get(oracle.BITS_WORKER, 0)[0]) == 0xFF
    assert int(o.get(oracle.BITS_WORKER, 1)[0]) == 0xF1
    np.testing.assert_array_equal(o.get(oracle.A_SERVER), [11, 5, 5, 5, 4, 4, 4, 4])
    np.testing.assert_array_equal(o.get(oracle.SCALE_SERVER), [7, 4])
    np.testing.assert_array_equal(o.get(oracle.E_SERVER), [4, -2, -2, -2, 0, 0, 0, 0])
    np.testing.assert_array_equal(o.get(oracle.M), [7, 7, 7, 7, 4, 4, 4, 4])
    np.testing.assert_array_equal(o.get(oracle.X), np.array([-7] * 4 + [-4] * 4) / 2048.0)
    assert int(o.get(oracle.BITS_SERVER)[0]) == 0xFF

    g0 = np.array([-23, 41, 41, 41, 0, 0, 0, 0], np.float32)
    g1 = np.array([5, 5, 5, 5, -8, -8, -8, -8], np.float32)
    o.compressed_step([g0, g1], lr)
    np.testing.assert_array_equal(o.get(oracle.C_WORKER, 0), [8, 8, 8, 8, 2, 2, 2, 2])
    np.testing.assert_array_equal(o.get(oracle.C_WORKER, 1), [6, 6, 6, 6, -2, -2, -2, -2])
    assert int(o.get(oracle.BITS_WORKER, 1)[0]) == 0x0F
    np.testing.assert_array_equal(o.get(oracle.A_SERVER), [7, 7, 7, 7, 0, 0, 0, 0])
    np.testing.assert_array_equal(o.get(oracle.U_SERVER), [11, 5, 5, 5, 0, 0, 0, 0])
    np.testing.assert_array_equal(o.get(oracle.SCALE_SERVER), [7, 0])
    np.testing.assert_array_equal(o.get(oracle.E_SERVER), [4, -2, -2, -2, 0, 0, 0, 0])
    np.testing.assert_array_equal(o.get(oracle.M), [7, 7, 7, 7, 0, 0, 0, 0])
    assert int(o.get(oracle.BITS_SERVER)[0]) == 0xFF
    np.testing.assert_array_equal(o.get(oracle.X), np.array([-14] * 4 + [-4] * 4) / 2048.0)
    np.testing.assert_array_equal(o.get(oracle.V), np.full(8, 4, np.float32))


def test_zero_chunk():
    """c = 0: scale 0, every sign bit +1, zero errors, x unchanged."""
    o = oracle.Oracle(2048, 2)
    o.set(oracle.V, np.full(2048, 1e-4, np.float32))
    o.compressed_step([np.zeros(2048, np.float32)] * 2, 1e-3)
    for w in range(2):
        np.testing.assert_array_equal(o.get(oracle.SCALE_WORKER, w), [0, 0])
        assert np.all(o.get(oracle.BITS_WORKER, w) == np.uint64(0xFFFFFFFFFFFFFFFF))
        np.testing.assert_array_equal(o.get(oracle.E_WORKER, w), np.zeros(2048))
    np.testing.assert_array_equal(o.get(oracle.X), np.zeros(2048))
    np.testing.assert_array_equal(o.get(oracle.M), np.zeros(2048))


def test_bit_layout_and_sign_of_zero():
    """Element k -> bit k%64 of word k//64; +1 for c >= 0 (including 0), -1
    for c < 0 and for NaN."""
    d = 320
    o = _exact_oracle(d, 1)
    rng = np.random.default_rng(3)
    pattern = rng.choice([-1.0, 0.0, 1.0], d).astype(np.float32)
    pattern[17] = np.nan
    o.compressed_step([2 * pattern], 2.0 ** -10)
    words = o.get(oracle.BITS_WORKER)
    for wi in range(d // 64):
        want = 0
        for b in range(64):
            v = pattern[64 * wi + b]
            if v >= 0:          # False for NaN
                want |= 1 << b
        assert int(words[wi]) == want


def test_all_sign_patterns_of_16():
    """All 2^16 sign patterns of 16 elements, packed four per word."""
    P = 1 << 16
    d = 16 * P
    idx = np.arange(d)
    signs = ((idx // 16)[:, None] >> (idx % 16)[:, None]).ravel() & 1
    c = np.where(signs == 1, 1.0, -1.0).astype(np.float32)
    o = _exact_oracle(d, 1)
    o.compressed_step([2 * c], 2.0 ** -10)
    words = o.get(oracle.BITS_WORKER)
    p = np.arange(P, dtype=np.uint64).reshape(-1, 4)
    want = p[:, 0] | (p[:, 1] << np.uint64(16)) | (p[:, 2] << np.uint64(32)) | (p[:, 3] << np.uint64(48))
    np.testing.assert_array_equal(words, want)
    assert o.get(oracle.SCALE_WORKER)[0] == 1.0
    np.testing.assert_array_equal(o.get(oracle.E_WORKER), np.zeros(d))


# ------------------------------------------ conservation over many steps ---

def _run_recorded(d, n, warm, comp, seed_step0=0):
    o = oracle.Oracle(d, n)
    rec = []
    for t in range(warm + comp):
        g = [synth.fill_cpu(d, 0, seed_step0 + t, w, sigma=1e-2) for w in range(n)]
        if t < warm:
            o.warmup_step(g, 1e-3)
            continue
        prev = {"m": o.get(oracle.M), "x": o.get(oracle.X), "v": o.get(oracle.V),
                "e": [o.get(oracle.E_WORKER, w) for w in range(n)], "es": o.get(oracle.E_SERVER)}
        o.compressed_step(g, 1e-3)
        cur = {"g": g, "c": [o.get(oracle.C_WORKER, w) for w in range(n)],
               "e": [o.get(oracle.E_WORKER, w) for w in range(n)],
               "bits": [o.get(oracle.BITS_WORKER, w) for w in range(n)],
               "s": [o.get(oracle.SCALE_WORKER, w) for w in range(n)],
               "a": o.get(oracle.A_SERVER), "u": o.get(oracle.U_SERVER),
               "es": o.get(oracle.E_SERVER), "sbits": o.get(oracle.BITS_SERVER),
               "ss": o.get(oracle.SCALE_SERVER), "m": o.get(oracle.M), "x": o.get(oracle.X),
               "v": o.get(oracle.V)}
        rec.append((prev, cur))
    return o, rec


@pytest.fixture(scope="module")
def recorded():
    return _run_recorded(d=16384, n=4, warm=3, comp=6)


def test_variance_frozen_in_compression_phase(recorded):
    _, rec = recorded
    v0 = rec[0][0]["v"]
    for _, cur in rec:
        np.testing.assert_array_equal(cur["v"], v0)


def test_bits_are_signs_of_compensated_momentum(recorded):
    o, rec = recorded
    for _, cur in rec:
        for w in range(o.n):
            np.testing.assert_array_equal(decode_bits(cur["bits"][w], o.d), cur["c"][w] >= 0)
        np.testing.assert_array_equal(decode_bits(cur["sbits"], o.d), cur["u"] >= 0)


def test_worker_error_feedback_conservation(recorded):
    """sum(transmitted + new error) == sum(compensated input), 1e-6 relative."""
    o, rec = recorded
    for _, cur in rec:
        for w in range(o.n):
            t = decompress(cur["bits"][w], cur["s"][w], o.L).astype(np.float64)
            c = cur["c"][w].astype(np.float64)
            for j in range(o.n):
                sl = slice(j * o.L, (j + 1) * o.L)
                lhs = np.sum(t[sl] + cur["e"][w][sl])
                assert abs(lhs - np.sum(c[sl])) <= 1e-6 * np.sum(np.abs(c[sl]))


def test_worker_telescoping_per_element(recorded):
    """Per element: sum over steps of what a worker transmits equals the sum
    of its uncompensated momenta (beta1*m + (1-beta1)*g) minus its final
    error -- up to fp32 rounding."""
    o, rec = recorded
    b1 = float(F32(0.9))
    ob1 = float(F32(1) - F32(0.9))
    for w in range(o.n):
        sent = np.zeros(o.d)
        fed = np.zeros(o.d)
        mag = np.zeros(o.d)
        for prev, cur in rec:
            y = b1 * prev["m"].astype(np.float64) + ob1 * cur["g"][w].astype(np.float64)
            sent += decompress(cur["bits"][w], cur["s"][w], o.L)
            fed += y
            mag += np.abs(y) + np.abs(prev["e"][w]) + np.abs(cur["c"][w]) + np.abs(cur["e"][w])
        resid = sent - (fed - rec[-1][1]["e"][w])
        assert np.all(np.abs(resid) <= 4 * 2.0 ** -24 * mag + 1e-30)


def test_server_average_and_telescoping(recorded):
    """The server averages what the workers transmitted; per element the sum
    of what it transmits equals the sum of those averages minus its final
    error (server error feedback)."""
    o, rec = recorded
    sent = np.zeros(o.d)
    fed = np.zeros(o.d)
    mag = np.zeros(o.d)
    for prev, cur in rec:
        sent_w = np.array([decompress(cur["bits"][w], cur["s"][w], o.L) for w in range(o.n)],
                          dtype=np.float64)
        avg = sent_w.mean(axis=0)
        # the fp32 pairwise sum may cancel: its error is bounded by the magnitudes
        assert np.all(np.abs(cur["a"] - avg) <= 4 * 2.0 ** -24 * np.abs(sent_w).mean(axis=0))
        sent += decompress(cur["sbits"], cur["ss"], o.L)
        fed += avg
        mag += np.abs(avg) + np.abs(prev["es"]) + np.abs(cur["u"]) + np.abs(cur["es"])
    resid = sent - (fed - rec[-1][1]["es"])
    assert np.all(np.abs(resid) <= 4 * 2.0 ** -24 * mag)


def test_momentum_is_decompressed_server_output_and_update(recorded):
    o, rec = recorded
    for prev, cur in rec:
        m = decompress(cur["sbits"], cur["ss"], o.L)
        np.testing.assert_array_equal(cur["m"], m)
        step = 1e-3 * m.astype(np.float64) / (np.sqrt(cur["v"].astype(np.float64)) + 1e-8)
        want = prev["x"].astype(np.float64) - step
        assert np.all(np.abs(cur["x"] - want) <= 1e-6 * np.abs(step) + 2.0 ** -23 * np.abs(want))


# ------------------------------------------------ structural identities ----

def test_identical_workers_equal_per_chunk_single_worker():
    """n identical workers: every chunk behaves as a one-worker run on that
    chunk alone, bit for bit (the average of n equal values is exact)."""
    d, n, L = 8192, 4, 2048
    big = oracle.Oracle(d, n)
    small = [oracle.Oracle(L, 1) for _ in range(n)]
    for t in range(5):
        g = synth.fill_cpu(d, 0, t, 0, sigma=1e-2)
        if t < 2:
            big.warmup_step([g] * n, 1e-3)
        else:
            big.compressed_step([g] * n, 1e-3)
        for j in range(n):
            gs = g[j * L:(j + 1) * L]
            (small[j].warmup_step if t < 2 else small[j].compressed_step)([gs], 1e-3)
    for j in range(n):
        sl = slice(j * L, (j + 1) * L)
        for f in (oracle.X, oracle.M, oracle.V, oracle.E_SERVER):
            np.testing.assert_array_equal(big.get(f)[sl], small[j].get(f))
        for w in range(n):
            np.testing.assert_array_equal(big.get(oracle.E_WORKER, w)[sl],
                                          small[j].get(oracle.E_WORKER))
            assert big.get(oracle.SCALE_WORKER, w)[j] == small[j].get(oracle.SCALE_WORKER)[0]
            np.testing.assert_array_equal(big.get(oracle.BITS_WORKER, w)[j * L // 64:(j + 1) * L // 64],
                                          small[j].get(oracle.BITS_WORKER))
        assert big.get(oracle.SCALE_SERVER)[j] == small[j].get(oracle.SCALE_SERVER)[0]


def test_chunk_subset_equals_full_run():
    d, n = 4 * 2048, 4
    L = d // n
    full = oracle.Oracle(d, n)
    part = oracle.Oracle(d, n, j0=1, j1=3)
    for t in range(5):
        g = [synth.fill_cpu(d, 0, t, w, sigma=1e-2) for w in range(n)]
        gp = [x[L:3 * L] for x in g]
        if t < 2:
            full.warmup_step(g, 1e-3)
            part.warmup_step(gp, 1e-3)
        else:
            full.compressed_step(g, 1e-3)
            part.compressed_step(gp, 1e-3)
    sl = slice(L, 3 * L)
    for f in (oracle.X, oracle.M, oracle.V, oracle.E_SERVER):
        np.testing.assert_array_equal(full.get(f)[sl], part.get(f))
    for w in range(n):
        np.testing.assert_array_equal(full.get(oracle.E_WORKER, w)[sl], part.get(oracle.E_WORKER, w))
        np.testing.assert_array_equal(full.get(oracle.SCALE_WORKER, w)[1:3],
                                      part.get(oracle.SCALE_WORKER, w))
    np.testing.assert_array_equal(full.get(oracle.SCALE_SERVER)[1:3], part.get(oracle.SCALE_SERVER))
