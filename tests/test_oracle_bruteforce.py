"""Brute force on tiny vectors (d <= 64): every step of the oracle is redone
in exact rational arithmetic and compared with what the oracle produced.

Each quantity is recomputed exactly (Python fractions; square roots to 50
significant digits) from the oracle's own fp32 values of its inputs, so a
comparison only has to allow for the rounding of the few fp32 operations
that form that one quantity, and a mistake anywhere -- a dropped term, a
wrong coefficient, sign or index, the wrong norm, epsilon or bias correction
in the wrong place, feedback taken from the wrong value -- shows up at the
step where it happens.  Worker counts 1 to 4 (an odd count included),
chunks shorter than one sign word, fp32 and bf16 gradients.

What each check follows: full-precision Adam for the warm-up, then 1-bit
compressed momentum with error feedback and per-chunk scaling, preconditioned
by the frozen variance ("1-bit Adam: Communication Efficient Large-Scale
Training with Adam's Convergence Speed", Abstract; "LIT-278: 1-bit Adam ...",
Key takeaways and tag lines SOTA-214, SOTA-215); the per-chunk scale is the
chunk's L2 norm over sqrt(chunk length), the sign of 0 is +1, the server
re-compresses the worker average with its own error feedback, and the
momentum after a compressed step is the decompressed server output.
"""
from decimal import Decimal, localcontext
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle

U = Fr(1, 2 ** 24)  # unit roundoff of fp32


def fr(x):
    """Exact value of an fp32 number."""
    return Fr(float(np.float32(x)))


def sqrt_fr(q):
    with localcontext() as ctx:
        ctx.prec = 50
        return Fr((Decimal(q.numerator) / Decimal(q.denominator)).sqrt())


def bits_of(words, count):
    w = [int(x) for x in np.asarray(words, dtype=np.uint64)]
    return [(w[k >> 6] >> (k & 63)) & 1 for k in range(count)]


def assert_close(got, want, bound, what):
    got = fr(got)
    assert abs(got - want) <= bound, "%s: oracle %r, exact %r (bound %r)" % (
        what, float(got), float(want), float(bound))


def state(o):
    s = {"x": o.get(oracle.X), "m": o.get(oracle.M), "v": o.get(oracle.V),
         "es": o.get(oracle.E_SERVER)}
    s["e"] = [o.get(oracle.E_WORKER, w) for w in range(o.n)]
    return s


def grad_values(g):
    """Exact values of the gradients as the oracle reads them."""
    if g.dtype == np.uint16:
        g = (g.astype(np.uint32) << 16).view(np.float32)
    return [fr(v) for v in g]


def check_warmup(o, pre, grads, lr, t, b1, b2, eps):
    d, n = o.d, o.n
    post = state(o)
    B1, B2, EPS, LR = fr(b1), fr(b2), fr(eps), fr(lr)
    gv = [grad_values(g) for g in grads]
    for k in range(d):
        gbar = sum(gv[w][k] for w in range(n)) / n
        gabs = sum(abs(gv[w][k]) for w in range(n)) / n
        mk, vk = fr(pre["m"][k]), fr(pre["v"][k])
        m_exact = B1 * mk + (1 - B1) * gbar
        # the average rounds about log2(n) + 1 times, then two products and a sum
        assert_close(post["m"][k], m_exact, (n + 4) * U * (B1 * abs(mk) + (1 - B1) * gabs),
                     "warm-up m[%d]" % k)
        v_exact = B2 * vk + (1 - B2) * gbar * gbar
        assert_close(post["v"][k], v_exact, (2 * n + 6) * U * (B2 * vk + (1 - B2) * gabs * gabs),
                     "warm-up v[%d]" % k)
        # the update from the oracle's own m and v, bias-corrected, eps outside the root
        bc1, bc2 = 1 - B1 ** t, 1 - B2 ** t
        m_o, v_o = fr(post["m"][k]), fr(post["v"][k])
        q = (m_o / bc1) / (sqrt_fr(v_o / bc2) + EPS)
        xk = fr(pre["x"][k])
        x_exact = xk - LR * q
        assert_close(post["x"][k], x_exact, 12 * U * abs(LR * q) + U * abs(x_exact),
                     "warm-up x[%d]" % k)
        for w in range(n):
            assert post["e"][w][k] == 0.0
        assert post["es"][k] == 0.0


def check_compressed(o, pre, grads, lr, b1, eps):
    d, n, L = o.d, o.n, o.L
    post = state(o)
    B1, EPS, LR = fr(b1), fr(eps), fr(lr)
    gv = [grad_values(g) for g in grads]
    c = [o.get(oracle.C_WORKER, w) for w in range(n)]
    wbits = [bits_of(o.get(oracle.BITS_WORKER, w), d) for w in range(n)]
    ws = [o.get(oracle.SCALE_WORKER, w) for w in range(n)]
    a = o.get(oracle.A_SERVER)
    u = o.get(oracle.U_SERVER)
    sbits = bits_of(o.get(oracle.BITS_SERVER), d)
    ss = o.get(oracle.SCALE_SERVER)

    # worker i: compensated momentum, its sign, per-chunk scale and new error
    for w in range(n):
        for k in range(d):
            mk, gk, ek = fr(pre["m"][k]), gv[w][k], fr(pre["e"][w][k])
            c_exact = B1 * mk + (1 - B1) * gk + ek
            bound = 4 * U * (B1 * abs(mk) + (1 - B1) * abs(gk) + abs(ek))
            assert_close(c[w][k], c_exact, bound, "c[%d][%d]" % (w, k))
            if abs(c_exact) > bound or c_exact == 0:
                # sign(0) = +1
                assert wbits[w][k] == (1 if c_exact >= 0 else 0), "sign bit of c[%d][%d]" % (w, k)
            assert wbits[w][k] == (1 if c[w][k] >= 0 else 0)
        for j in range(n):
            seg = [fr(x) for x in c[w][j * L:(j + 1) * L]]
            s_exact = sqrt_fr(sum(x * x for x in seg) / L)
            assert_close(ws[w][j], s_exact, 2 * U * s_exact, "worker %d scale of chunk %d" % (w, j))
            sw = fr(ws[w][j])
            for k in range(j * L, (j + 1) * L):
                e_exact = fr(c[w][k]) - (sw if wbits[w][k] else -sw)
                assert_close(post["e"][w][k], e_exact, U * abs(e_exact), "e[%d][%d]" % (w, k))

    # server j: average of the decompressed workers, its own error feedback,
    # re-compression, new server error; the momentum becomes the server output
    for j in range(n):
        for k in range(j * L, (j + 1) * L):
            vals = [fr(ws[w][j]) if wbits[w][k] else -fr(ws[w][j]) for w in range(n)]
            a_exact = sum(vals) / n
            assert_close(a[k], a_exact, (n + 1) * U * sum(abs(x) for x in vals) / n,
                         "server average a[%d]" % k)
            u_exact = fr(a[k]) + fr(pre["es"][k])
            assert_close(u[k], u_exact, U * abs(u_exact), "u[%d]" % k)
            assert sbits[k] == (1 if u[k] >= 0 else 0)
            if u_exact == 0:
                assert sbits[k] == 1, "sign of a zero server value"
        seg = [fr(x) for x in u[j * L:(j + 1) * L]]
        s_exact = sqrt_fr(sum(x * x for x in seg) / L)
        assert_close(ss[j], s_exact, 2 * U * s_exact, "server scale of chunk %d" % j)
        sj = fr(ss[j])
        for k in range(j * L, (j + 1) * L):
            t = sj if sbits[k] else -sj
            es_exact = fr(u[k]) - t
            assert_close(post["es"][k], es_exact, U * abs(es_exact), "server error[%d]" % k)
            assert fr(post["m"][k]) == t, "m[%d] is not the decompressed server output" % k
            # frozen variance, no bias correction, eps outside the root
            assert post["v"][k] == pre["v"][k]
            q = t / (sqrt_fr(fr(post["v"][k])) + EPS)
            x_exact = fr(pre["x"][k]) - LR * q
            assert_close(post["x"][k], x_exact, 6 * U * abs(LR * q) + U * abs(x_exact),
                         "x[%d]" % k)


CASES = [  # d, n, bf16, elements whose gradient is always 0 (like padding)
    (64, 1, False, 0),
    (64, 2, False, 0),
    (48, 3, False, 0),
    (63, 3, True, 0),
    (64, 4, False, 4),
    (16, 4, True, 2),
]


@pytest.mark.parametrize("d,n,bf16,zeros", CASES)
def test_every_step_matches_exact_arithmetic(d, n, bf16, zeros):
    """With zero gradients on the last elements, m stays 0 there through the
    warm-up and the first compressed step sees c = 0 exactly (sign +1)."""
    b1, b2, eps = 0.9, 0.999, 1e-8
    rng = np.random.default_rng(97 + 7 * d + n)
    o = oracle.Oracle(d, n, b1, b2, eps, keep_debug=True)
    o.set(oracle.X, rng.normal(0, 1, d).astype(np.float32))
    warm, comp = 3, 5
    for t in range(warm + comp):
        grads = []
        for _ in range(n):
            g = rng.normal(0, 1e-2, d).astype(np.float32)
            g[d - zeros:] = 0.0
            if bf16:
                g = (g.view(np.uint32) >> 16).astype(np.uint16)
            grads.append(g)
        lr = np.float32(1e-3 * (1 + 0.25 * t))
        pre = state(o)
        if t < warm:
            o.warmup_step(grads, lr)
            check_warmup(o, pre, grads, lr, t + 1, b1, b2, eps)
        else:
            o.compressed_step(grads, lr)
            check_compressed(o, pre, grads, lr, b1, eps)
        assert o.step == t + 1
    o.close()
