"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/sinkhorn_oracle.c
(a dropped term, a wrong sign or index, a transposed weight, a halved
gradient, a wrong threshold, a biased sum), builds it, and runs the pin suite
(tests/test_oracle_pins.py) against that build in a fresh process: at least
one pin must fail.  The unmutated copy, built the same way, must pass them all.
The mistakes live only in the temporary copies; the oracle itself is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sinkhorn_oracle.c")

# (name, text in the oracle, its replacement); each text occurs exactly once
MUTATIONS = [
    ("log weight dropped from the half-update",
     "z[j] = (pot[j] - sq_dist(p, Q + (size_t)j * d, d)) / eps + logw[j];",
     "z[j] = (pot[j] - sq_dist(p, Q + (size_t)j * d, d)) / eps;"),
    ("sign of the cost flipped in the half-update",
     "z[j] = (pot[j] - sq_dist(p, Q + (size_t)j * d, d)) / eps + logw[j];",
     "z[j] = (pot[j] + sq_dist(p, Q + (size_t)j * d, d)) / eps + logw[j];"),
    ("sign of the update flipped",
     "out[t] = -eps * log_sum_exp(z, nq);",
     "out[t] = eps * log_sum_exp(z, nq);"),
    ("g-update takes the old g's weights",
     "oracle_half_update(Yp, m, Xp, n, d, fp, la, eps[s], NULL, 0, gp);",
     "oracle_half_update(Yp, m, Xp, n, d, gp, la, eps[s], NULL, 0, gp);"),
    ("attention form without eps in the bias",
     "ga[i] = eps[s] * la[i];",
     "ga[i] = la[i];"),
    ("plan without the g potential",
     "return (fi + gj - sq_dist(x, y, d)) / eps + (lai + lbj);",
     "return (fi - sq_dist(x, y, d)) / eps + (lai + lbj);"),
    ("plan without log b",
     "return (fi + gj - sq_dist(x, y, d)) / eps + (lai + lbj);",
     "return (fi + gj - sq_dist(x, y, d)) / eps + lai;"),
    ("sum of exponentials biased",
     "        s += exp(z[k] - M);\n    return M + log(s);",
     "        s += exp(z[k] - M) * (1.0 + 1e-9);\n    return M + log(s);"),
    ("threshold taken as its square root",
     "double log_thr = log(rel_thr);",
     "double log_thr = 0.5 * log(rel_thr);"),
    ("gradient on the stored support halved",
     "dXp[(size_t)i * d + c] += 2.0 * vals[k] * (x[c] - y[c]);",
     "dXp[(size_t)i * d + c] += vals[k] * (x[c] - y[c]);"),
    ("dense gradient with x and y exchanged",
     "acc_add(&G[c], 2.0 * P * (x[c] - y[c]));",
     "acc_add(&G[c], 2.0 * P * (y[c] - x[c]));"),
    ("compensated sum loses its correction",
     "static double acc_get(const acc_t *a) { return a->s + a->c; }",
     "static double acc_get(const acc_t *a) { return a->s + 2.0 * a->c + 1e-12; }"),
    ("COO normalisation without the row weight",
     "al[i] = mx_r[i] > -INFINITY ? log(ap[i]) - (mx_r[i] + log(sm_r[i])) : 0.0;",
     "al[i] = mx_r[i] > -INFINITY ? -(mx_r[i] + log(sm_r[i])) : 0.0;"),
    ("Hessian-vector product with a halved row term",
     "r[i] += pij * 2.0 * dot;",
     "r[i] += pij * dot;"),
    ("Hessian-vector product with columns of no mass kept in the solve",
     "            if (mb[j] > 0.0) {\n                if (pin < 0)",
     "            if (mb[j] >= 0.0) {\n                if (pin < 0)"),
]


def _build(src_text, out_dir):
    c = os.path.join(out_dir, "oracle_copy.c")
    so = os.path.join(out_dir, "liboracle_copy.so")
    with open(c, "w") as fh:
        fh.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", c, "-o",
                           so, "-lm"])
    return so


def _run_pins(so):
    env = dict(os.environ, SK_ORACLE_LIB=so, OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.mark.slow
def test_unmutated_copy_passes_every_pin(tmp_path):
    so = _build(open(SRC).read(), str(tmp_path))
    r = _run_pins(so)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_every_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {old!r}"
    so = _build(src.replace(old, new), str(tmp_path))
    r = _run_pins(so)
    assert r.returncode != 0, f"no pin caught: {name}"
