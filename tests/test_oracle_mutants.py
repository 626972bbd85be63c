"""The pins must catch plausible mistakes: each mutant below is the oracle
with one deliberate error (a dropped term, a wrong sign, a transposed index,
a misplaced feedback; for the 0/1 Adam step a wrongly weighted mean, a lost
step-size sum, a dropped refresh), built on the CPU into a temporary
library; the pins, the exact-arithmetic brute force and the 0/1 pins run
against it have to fail."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ob_oracle.c")

MUTANTS = {
    "worker_error_dropped": ("c[q] = ((o->beta1 * o->m[k]) + (ob1 * g)) + e[k];",
                             "c[q] = ((o->beta1 * o->m[k]) + (ob1 * g));"),
    "beta_swapped": ("c[q] = ((o->beta1 * o->m[k]) + (ob1 * g)) + e[k];",
                     "c[q] = ((ob1 * o->m[k]) + (o->beta1 * g)) + e[k];"),
    "scale_index_transposed": ("float sw = o->wscale[(size_t)w * (size_t)o->nch + jj];",
                               "float sw = o->wscale[(size_t)jj * (size_t)o->n + w];"),
    "server_error_dropped": ("u[q] = a[q] + o->e_srv[k];", "u[q] = a[q];"),
    "sign_of_zero_negative": ("int bit = c[q] >= 0.0f;", "int bit = c[q] > 0.0f;"),
    "eps_inside_sqrt": ("o->x[k] = o->x[k] - step * (o->m[k] / (sqrtf(o->v[k]) + o->eps));",
                        "o->x[k] = o->x[k] - step * (o->m[k] / sqrtf(o->v[k] + o->eps));"),
    "scale_divided_by_L": ("return (float)(sqrt(sumsq) / sqrt((double)len));",
                           "return (float)(sqrt(sumsq) / (double)len);"),
    "butterfly_doubles": ("nxt[k] = acc[k] + acc[k ^ o];", "nxt[k] = acc[k] + acc[k];"),
    "warmup_no_bias_correction": ("float mh = o->m[k] / bc1;", "float mh = o->m[k];"),
    "momentum_not_decompressed": ("o->m[k] = t;", "(void)t;"),
    "bit_order_reversed": ("if (bit) words[k >> 6] |= (uint64_t)1 << (k & 63);",
                           "if (bit) words[k >> 6] |= (uint64_t)1 << (63 - (k & 63));"),
    "average_tree_reordered": ("t[i] = t[2 * i] + t[2 * i + 1];", "t[i] = t[i] + t[i + half];"),
    "server_error_keeps_average": ("o->e_srv[k] = u[q] - t;", "o->e_srv[k] = a[q] - t;"),
    # the 0/1 Adam step
    "zo_mean_unweighted": ("al[k] = first ? mi : al[k] + (wk * (mi - al[k]));",
                           "al[k] = first ? mi : al[k] + ((1.0f / (float)(o->zk + 1)) * "
                           "(mi - al[k]));"),
    "zo_step_sizes_not_summed": ("o->zgamma = first ? lr : o->zgamma + lr;", "o->zgamma = lr;"),
    "zo_momentum_always_shared": ("float msrc = first ? o->m[k] : ml[k];",
                                  "float msrc = o->m[k];"),
    "zo_refresh_dropped": ("if (refresh) {", "if (0) {"),
    "zo_update_by_last_step_size": ("server_round(o, o->zgamma);", "server_round(o, lr);"),
    "zo_error_dropped": ("c[q] = al[base + q] + e[base + q];", "c[q] = al[base + q];"),
    "zo_local_model_without_step_sizes": (
        "out[k] = o->x[k] - o->zgamma * (al[k] / (sqrtf(o->v[k]) + o->eps));",
        "out[k] = o->x[k] - (al[k] / (sqrtf(o->v[k]) + o->eps));"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + name
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "ob_oracle.c")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        with open(os.path.join(tmp, "ob_oracle.h"), "w") as f:
            f.write(open(os.path.join(ROOT, "oracle", "ob_oracle.h")).read())
        so = os.path.join(tmp, "libmut.so")
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", so, c, "-lm"])
        env = dict(os.environ, OB_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                            os.path.join(ROOT, "tests", "test_oracle_bruteforce.py"),
                            os.path.join(ROOT, "tests", "test_oracle_zo_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
