"""Pins of the CPU oracle to facts it does not compute itself.

Each test checks the fp64 oracle against something fixed by the mathematics
of entropic optimal transport or by an independent library routine, never
against a retyped copy of its own formula.  The mistakes these are chosen to
catch: a dropped log-weight term (non-uniform weights everywhere), a sign or
scale error in the cost (brute-force assignment, closed forms), a transposed
operand (n != m, swap symmetry), a wrong half-update order (marginals), and a
wrong plan/threshold formula (2x2 closed form, dense enumeration, duality).

Pages: FlashSinkhorn technical summary, Methodologie 1 (Propositie 1) for the
log-domain updates; CUDA-APML page, Abstract / Innovation for the thresholded
sparse plan and the loss/gradient on the stored support.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment
from scipy.special import logsumexp

import oracle
import workloads


def _case(seed, n, m, d=3, weights="dirichlet", spread=1.0):
    # weights renormalised in float64: float32-rounded weights need not have
    # equal sums, and then no plan can match both marginals exactly
    c = workloads.random_case(seed, 1, n, m, d, weights=weights, spread=spread)
    a, b = c["a"][0].astype(np.float64), c["b"][0].astype(np.float64)
    return (c["X"][0].astype(np.float64), c["Y"][0].astype(np.float64),
            a / a.sum(), b / b.sum())


def _cost_matrix(X, Y):
    return ((X[:, None, :] - Y[None, :, :]) ** 2).sum(-1)


def _converge(X, Y, a, b, eps, iters):
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[iters])
    return f, g


# ---------------------------------------------------------------- half-update
@pytest.mark.parametrize("n,m,d", [(17, 29, 3), (64, 5, 7), (1, 40, 2)])
def test_half_update_matches_scipy_weighted_logsumexp(n, m, d):
    rng = np.random.default_rng(n * 100 + m)
    X, Y = rng.random((n, d)), rng.random((m, d))
    g = rng.normal(size=m)
    b = rng.dirichlet(np.ones(m))
    eps = 0.07
    f = oracle.half_update(X, Y, g, b, eps)
    C = _cost_matrix(X, Y)
    ref = -eps * logsumexp((g[None, :] - C) / eps, b=b[None, :], axis=1)
    np.testing.assert_allclose(f, ref, rtol=1e-13, atol=1e-13)
    rows = [n - 1, 0]
    np.testing.assert_array_equal(oracle.half_update(X, Y, g, b, eps, rows=rows), f[rows])


# ------------------------------------------------------- attention vs direct
@pytest.mark.parametrize("d", [3, 64])
@pytest.mark.parametrize("k", [1, 10, 100])
def test_attention_form_agrees_with_direct_form(d, k):
    X, Y, a, b = _case(11 + d, 37, 23, d=d)
    eps = 0.05 if d == 3 else 0.5
    f1, g1 = oracle.potentials(X, Y, a, b, eps=[eps], iters=[k], form="direct")
    f2, g2 = oracle.potentials(X, Y, a, b, eps=[eps], iters=[k], form="attention")
    scale = max(np.abs(f1).max(), np.abs(g1).max(), eps)
    assert np.abs(f1 - f2).max() / scale < 1e-10
    assert np.abs(g1 - g2).max() / scale < 1e-10


def test_attention_form_agrees_on_a_schedule_with_warm_start():
    X, Y, a, b = _case(5, 41, 31)
    eps = workloads.geometric_schedule(1.0, 0.01, 4).astype(np.float64)
    f1, g1 = oracle.potentials(X, Y, a, b, eps=eps, iters=[5] * 4, form="direct")
    f2, g2 = oracle.potentials(X, Y, a, b, eps=eps, iters=[5] * 4, form="attention")
    np.testing.assert_allclose(f1, f2, rtol=0, atol=1e-10 * np.abs(f1).max())
    np.testing.assert_allclose(g1, g2, rtol=0, atol=1e-10 * np.abs(g1).max())
    # split run == full run (potentials are the complete state)
    fa, ga = oracle.potentials(X, Y, a, b, eps=eps[:2], iters=[5] * 2)
    fb, gb = oracle.potentials(X, Y, a, b, eps=eps[2:], iters=[5] * 2, f0=fa, g0=ga)
    np.testing.assert_array_equal(fb, f1)
    np.testing.assert_array_equal(gb, g1)


# ----------------------------------------------------------- fixed point
def test_marginals_hold_at_convergence():
    X, Y, a, b = _case(3, 200, 150)
    eps = 0.05
    f, g = _converge(X, Y, a, b, eps, 600)
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert st["col_err"][0] <= 1e-12     # exact after the g-update
    assert st["row_err"][0] <= 1e-6      # the pages' convergence tolerance
    # one more f-update barely moves f (fixed point)
    f_next = oracle.half_update(X, Y, g, b, eps)
    assert np.abs(f_next - f).max() < 1e-9


def test_marginals_fail_before_convergence():
    # guards the test above against a trivially-satisfied statistic
    X, Y, a, b = _case(3, 200, 150)
    f, g = _converge(X, Y, a, b, 0.05, 2)
    st = oracle.plan_stats(X, Y, a, b, f, g, 0.05)
    assert st["row_err"][0] > 1e-4


def test_strong_duality_at_convergence():
    # dual value = primal entropic objective <P,C> + eps KL(P || a b^T)
    X, Y, a, b = _case(8, 60, 45)
    eps = 0.1
    f, g = _converge(X, Y, a, b, eps, 3000)
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert st["row_err"][0] < 1e-12
    primal = st["cost"][0] + eps * st["kl"][0]
    assert abs(st["dual"][0] - primal) <= 1e-10 * abs(primal)
    # primal cost and dual differ by eps*KL, a strictly positive amount here
    assert st["dual"][0] - st["cost"][0] > 1e-3


# ----------------------------------------------------- closed forms / limits
def _two_by_two_plan(C, a1, b1, eps):
    """Entropic plan of a 2x2 problem from the cross-ratio invariant
    P11 P22 / (P12 P21) = K11 K22 / (K12 K21), K = exp(-C/eps)."""
    kappa = math.exp(-(C[0, 0] + C[1, 1] - C[0, 1] - C[1, 0]) / eps)
    A, Bq, Cq = 1.0 - kappa, 1.0 - a1 - b1 + kappa * (a1 + b1), -kappa * a1 * b1
    lo, hi = max(0.0, a1 + b1 - 1.0), min(a1, b1)
    if abs(A) < 1e-15:
        roots = [-Cq / Bq]
    else:
        disc = math.sqrt(Bq * Bq - 4 * A * Cq)
        roots = [(-Bq + disc) / (2 * A), (-Bq - disc) / (2 * A)]
    p = [r for r in roots if lo - 1e-15 <= r <= hi + 1e-15]
    assert len(p) == 1
    p = p[0]
    return np.array([[p, a1 - p], [b1 - p, 1.0 - a1 - b1 + p]])


@pytest.mark.parametrize("eps", [0.5, 0.1, 0.03])
def test_two_by_two_closed_form(eps):
    X = np.array([[0.1, 0.2, 0.0], [0.9, 0.4, 0.3]])
    Y = np.array([[0.8, 0.5, 0.2], [0.0, 0.1, 0.4]])
    a = np.array([0.3, 0.7])
    b = np.array([0.55, 0.45])
    C = _cost_matrix(X, Y)
    Pref = _two_by_two_plan(C, a[0], b[0], eps)
    f, g = _converge(X, Y, a, b, eps, 3000)
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-300)
    P = np.zeros((2, 2))
    P[rows, cols] = vals
    np.testing.assert_allclose(P, Pref, rtol=1e-10, atol=1e-14)
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert abs(st["cost"][0] - (Pref * C).sum()) <= 1e-10


def test_single_point_pair():
    X = np.array([[0.3, -1.0, 2.0]])
    Y = np.array([[1.5, 0.5, -0.5]])
    C11 = float(((X - Y) ** 2).sum())
    f, g = oracle.potentials(X, Y, [1.0], [1.0], eps=[0.01], iters=[3])
    assert abs(f[0] + g[0] - C11) <= 1e-15 * C11
    st = oracle.plan_stats(X, Y, [1.0], [1.0], f, g, 0.01)
    assert abs(st["cost"][0] - C11) <= 1e-15 * C11


def test_large_eps_limit_is_independent_coupling():
    X, Y, a, b = _case(21, 30, 40)
    eps = 1e4
    f, g = _converge(X, Y, a, b, eps, 20)
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    ma, mb = a @ X, b @ Y
    indep = a @ (X ** 2).sum(1) + b @ (Y ** 2).sum(1) - 2 * ma @ mb
    assert abs(st["cost"][0] - indep) / indep < 1e-3


# ------------------------------------------- entropic -> exact assignment
def _best_permutation_cost(C):
    n = C.shape[0]
    best = min(sum(C[i, s[i]] for i in range(n)) for s in itertools.permutations(range(n)))
    return best / n


@pytest.mark.parametrize("n", [1, 2, 4, 6, 7])
@pytest.mark.parametrize("eps", [1e-2, 1e-3])
def test_small_eps_approaches_brute_force_assignment(n, eps):
    # <C,P_eps> - OT_0 <= eps (H(P_eps) - H(P*)) <= eps (2 ln n - ln n): P_eps minimises
    # <C,P> - eps H(P) over the coupling polytope and a permutation plan has H = ln n
    X, Y, a, b = _case(40 + n, n, n, weights="uniform")
    C = _cost_matrix(X, Y)
    ot0 = _best_permutation_cost(C)
    sched = list(np.geomspace(1.0, eps, 12)) + [eps]      # annealed, to reach the fixed point
    f, g = oracle.potentials(X, Y, a, b, eps=sched, iters=[500] * 12 + [100000])
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert st["row_err"][0] < 1e-6
    slack = st["row_err"][0] * C.max() + 1e-12            # plan off the polytope by row_err
    assert ot0 - slack <= st["cost"][0] <= ot0 + eps * math.log(max(n, 1)) + slack


def test_small_eps_approaches_linear_sum_assignment_n64():
    X, Y, a, b = _case(77, 64, 64, weights="uniform")
    C = _cost_matrix(X, Y)
    r, c = linear_sum_assignment(C)
    ot0 = C[r, c].sum() / 64
    eps = 2e-3
    sched = list(np.geomspace(1.0, eps, 12)) + [eps]
    f, g = oracle.potentials(X, Y, a, b, eps=sched, iters=[300] * 12 + [20000])
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert st["row_err"][0] < 1e-5
    slack = st["row_err"][0] * C.max() + 1e-12
    assert ot0 - slack <= st["cost"][0] <= ot0 + eps * math.log(64) + slack


# ---------------------------------------------------------- invariances
@pytest.mark.parametrize("t", [(3.0, -2.0, 5.0), (100.0, 100.0, 100.0)])
def test_translation_invariance(t):
    X, Y, a, b = _case(9, 50, 70)
    eps = 0.05
    f1, g1 = oracle.potentials(X, Y, a, b, eps=[eps], iters=[50])
    f2, g2 = oracle.potentials(X + np.array(t), Y + np.array(t), a, b, eps=[eps], iters=[50])
    sc = max(np.abs(f1).max(), np.abs(g1).max())
    assert np.abs(f1 - f2).max() / sc < 1e-9
    assert np.abs(g1 - g2).max() / sc < 1e-9
    c1 = oracle.plan_stats(X, Y, a, b, f1, g1, eps)["cost"][0]
    c2 = oracle.plan_stats(X + np.array(t), Y + np.array(t), a, b, f2, g2, eps)["cost"][0]
    assert abs(c1 - c2) / c1 < 1e-9


def test_swap_symmetry_at_convergence():
    X, Y, a, b = _case(13, 40, 25)
    eps = 0.1
    f, g = _converge(X, Y, a, b, eps, 500)
    g2, f2 = _converge(Y, X, b, a, eps, 500)   # roles swapped: potentials swap too
    s1 = oracle.plan_stats(X, Y, a, b, f, g, eps)
    s2 = oracle.plan_stats(Y, X, b, a, g2, f2, eps)
    assert abs(s1["cost"][0] - s2["cost"][0]) < 1e-9
    assert abs(s1["dual"][0] - s2["dual"][0]) < 1e-9


def test_zero_weight_points_drop_out():
    c = workloads.random_case(4, 1, 30, 20, 3, weights="dirichlet", zero_weights=3)
    X, Y = c["X"][0].astype(float), c["Y"][0].astype(float)
    a, b = c["a"][0].astype(float), c["b"][0].astype(float)
    eps = 0.05
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[30])
    fr, gr = oracle.potentials(X[3:], Y[3:], a[3:], b[3:], eps=[eps], iters=[30])
    np.testing.assert_allclose(f[3:], fr, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g[3:], gr, rtol=1e-13, atol=1e-13)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))


# ------------------------------------------------------- sparse plan / loss
def test_coo_matches_dense_enumeration():
    X, Y, a, b = _case(31, 33, 47)
    eps = 0.02
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[7])
    for thr in (1e-8, 1e-3, 1.0):
        rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=thr)
        logP = (f[:, None] + g[None, :] - _cost_matrix(X, Y)) / eps \
            + np.log(a)[:, None] + np.log(b)[None, :]
        keep = np.argwhere(logP >= logP.max() + np.log(thr))     # row-major order
        np.testing.assert_array_equal(rows, keep[:, 0])
        np.testing.assert_array_equal(cols, keep[:, 1])
        np.testing.assert_allclose(vals, np.exp(logP[keep[:, 0], keep[:, 1]]), rtol=1e-13)
        assert offs.tolist() == [0, len(rows)]
        if thr == 1.0:
            assert len(rows) >= 1


def test_coo_batch_offsets_and_pair_independence():
    c = workloads.random_case(2, 3, 12, 9, 3, weights="dirichlet")
    X, Y, a, b = (c[k].astype(float) for k in ("X", "Y", "a", "b"))
    eps = 0.05
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[10])
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-4)
    for p in range(3):
        r1, c1, v1, o1 = oracle.plan_coo(X[p], Y[p], a[p], b[p], f[p], g[p], eps, rel_thr=1e-4)
        s = slice(offs[p], offs[p + 1])
        np.testing.assert_array_equal(rows[s], r1)
        np.testing.assert_array_equal(cols[s], c1)
        np.testing.assert_array_equal(vals[s], v1)


def test_gradient_is_envelope_derivative_of_ot_value():
    # at convergence, d OT_eps / d x_i = sum_j 2 P_ij (x_i - y_j)
    X, Y, a, b = _case(17, 12, 9)
    eps, iters = 0.1, 3000

    def ot_value(Xv):
        f, g = oracle.potentials(Xv, Y, a, b, eps=[eps], iters=[iters])
        return float(a @ f + b @ g)

    f, g = _converge(X, Y, a, b, eps, iters)
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-300)
    assert len(rows) == 12 * 9
    loss, dX = oracle.loss_grad(X, Y, rows, cols, vals, offs)
    h = 1e-5
    fd = np.zeros_like(X)
    for i in range(X.shape[0]):
        for k in range(3):
            Xp, Xm = X.copy(), X.copy()
            Xp[i, k] += h
            Xm[i, k] -= h
            fd[i, k] = (ot_value(Xp) - ot_value(Xm)) / (2 * h)
    np.testing.assert_allclose(dX[0], fd, rtol=1e-6, atol=1e-8)
    # with the full support the loss is the transport cost
    st = oracle.plan_stats(X, Y, a, b, f, g, eps)
    assert abs(loss[0] - st["cost"][0]) <= 1e-12 * st["cost"][0]


def test_loss_grad_any_order_and_truncated_support():
    X, Y, a, b = _case(19, 20, 15)
    eps = 0.03
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[20])
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-2)
    loss, dX = oracle.loss_grad(X, Y, rows, cols, vals, offs)
    perm = np.random.default_rng(0).permutation(len(rows))
    loss2, dX2 = oracle.loss_grad(X, Y, rows[perm], cols[perm], vals[perm], offs)
    np.testing.assert_allclose(loss2, loss, rtol=1e-13)
    np.testing.assert_allclose(dX2, dX, rtol=1e-12, atol=1e-15)
    # rows without stored entries get a zero gradient
    empty = np.setdiff1d(np.arange(20), rows)
    assert np.all(dX[0, empty] == 0.0)


# ------------------------------------------- dense gradient and projection
def test_dense_gradient_is_envelope_derivative_both_sides():
    # at convergence d OT_eps / d x_i = sum_j 2 P_ij (x_i - y_j), and the same for y_j
    X, Y, a, b = _case(23, 9, 11)
    eps, iters = 0.1, 3000

    def ot_value(Xv, Yv):
        f, g = oracle.potentials(Xv, Yv, a, b, eps=[eps], iters=[iters])
        return float(a @ f + b @ g)

    f, g = _converge(X, Y, a, b, eps, iters)
    r, dX, T = oracle.dense_grad(X, Y, a, b, f, g, eps)
    rY, dY, TY = oracle.dense_grad(Y, X, b, a, g, f, eps)
    h = 1e-5
    for side, P0, ref in (("x", X, dX[0]), ("y", Y, dY[0])):
        fd = np.zeros_like(P0)
        for i in range(P0.shape[0]):
            for k in range(3):
                Pp, Pm = P0.copy(), P0.copy()
                Pp[i, k] += h
                Pm[i, k] -= h
                args_p = (Pp, Y) if side == "x" else (X, Pp)
                args_m = (Pm, Y) if side == "x" else (X, Pm)
                fd[i, k] = (ot_value(*args_p) - ot_value(*args_m)) / (2 * h)
        np.testing.assert_allclose(ref, fd, rtol=1e-6, atol=1e-8)
    # at convergence the row masses are the weights on both sides
    np.testing.assert_allclose(r[0], a, rtol=1e-9)
    np.testing.assert_allclose(rY[0], b, rtol=1e-9)


def test_dense_row_mass_is_exact_after_an_f_update():
    # f from one half-update against any g makes every row sum of P equal a_i
    X, Y, a, b = _case(29, 40, 23)
    eps = 0.04
    g = np.random.default_rng(5).normal(scale=0.1, size=23)
    f = oracle.half_update(X, Y, g, b, eps)
    r, _, _ = oracle.dense_grad(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(r[0], a, rtol=1e-13)


def test_barycentric_projection_approaches_assignment_at_small_eps():
    n = 7
    X, Y, a, b = _case(61, n, n, weights="uniform")
    C = _cost_matrix(X, Y)
    rows, sigma = linear_sum_assignment(C)
    eps = 1e-3
    sched = list(np.geomspace(1.0, eps, 12)) + [eps]
    f, g = oracle.potentials(X, Y, a, b, eps=sched, iters=[500] * 12 + [100000])
    r, dX, T = oracle.dense_grad(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(T[0], Y[sigma], atol=1e-4)
    np.testing.assert_allclose(dX[0], 2.0 / n * (X - Y[sigma]), atol=1e-4)


def test_projection_at_large_eps_is_the_weighted_mean():
    # P -> a b^T: T_i -> sum_j b_j y_j and dX_i -> 2 a_i (x_i - ybar), up to O(1/eps)
    X, Y, a, b = _case(67, 30, 40)
    eps = 1e4
    f, g = _converge(X, Y, a, b, eps, 20)
    r, dX, T = oracle.dense_grad(X, Y, a, b, f, g, eps)
    ybar = b @ Y
    np.testing.assert_allclose(T[0], np.broadcast_to(ybar, T[0].shape), atol=1e-3)
    np.testing.assert_allclose(dX[0], 2 * a[:, None] * (X - ybar), atol=1e-3 * np.abs(dX).max())


def test_dense_grad_translation_and_subset():
    X, Y, a, b = _case(71, 25, 31)
    eps = 0.05
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[15])
    r, dX, T = oracle.dense_grad(X, Y, a, b, f, g, eps)
    t = np.array([4.0, -1.0, 2.5])
    r2, dX2, T2 = oracle.dense_grad(X + t, Y + t, a, b, f, g, eps)   # plan unchanged
    np.testing.assert_allclose(r2, r, rtol=1e-12)
    np.testing.assert_allclose(dX2, dX, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(T2, T + t, rtol=1e-12, atol=1e-12)
    sel = [24, 3, 3, 0]
    r3, dX3, T3 = oracle.dense_grad(X, Y, a, b, f, g, eps, sel=sel)
    np.testing.assert_array_equal(r3, r[0, sel])
    np.testing.assert_array_equal(dX3, dX[0, sel])
    np.testing.assert_array_equal(T3, T[0, sel])


def test_dense_grad_matches_full_support_coo_gradient():
    X, Y, a, b = _case(73, 14, 19)
    eps = 0.03
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[9])
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-300)
    assert len(rows) == 14 * 19
    loss, dXc = oracle.loss_grad(X, Y, rows, cols, vals, offs)
    r, dX, T = oracle.dense_grad(X, Y, a, b, f, g, eps)
    np.testing.assert_allclose(dX, dXc, rtol=1e-12, atol=1e-15)


# ------------------------------------------ cosine cost on normalised vectors
def test_normalize_gives_unit_vectors_along_the_input():
    rng = np.random.default_rng(3)
    X = rng.normal(size=(4, 30, 7))
    X[1, 5] = 0.0
    Xh, nr = oracle.normalize(X)
    live = nr > 0
    np.testing.assert_allclose(np.linalg.norm(Xh, axis=-1)[live], 1.0, rtol=1e-15)
    np.testing.assert_array_equal(Xh[1, 5], 0.0)
    np.testing.assert_allclose(Xh * nr[..., None], X, rtol=1e-14, atol=1e-15)
    # scaling a point by a positive factor leaves its direction unchanged
    Xh2, nr2 = oracle.normalize(X * 3.5)
    np.testing.assert_allclose(Xh2, Xh, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(nr2, 3.5 * nr, rtol=1e-14)


def test_cosine_cost_update_matches_scipy_on_the_cosine_matrix():
    # the squared-Euclidean update on normalised points is the update of the
    # cosine cost 2 - 2 xh.yh, computed here directly with numpy and scipy
    rng = np.random.default_rng(8)
    X, Y = rng.normal(size=(40, 16)), rng.normal(size=(33, 16)) * 5.0
    Xh, _ = oracle.normalize(X)
    Yh, _ = oracle.normalize(Y)
    g = rng.normal(scale=0.1, size=33)
    b = rng.dirichlet(np.ones(33))
    eps = 0.05
    f = oracle.half_update(Xh, Yh, g, b, eps)
    C = 2.0 - 2.0 * (X / np.linalg.norm(X, axis=1, keepdims=True)) @ \
        (Y / np.linalg.norm(Y, axis=1, keepdims=True)).T
    ref = -eps * logsumexp((g[None, :] - C) / eps, b=b[None, :], axis=1)
    np.testing.assert_allclose(f, ref, rtol=1e-12, atol=1e-12)


def test_normalize_backward_is_the_derivative_of_the_normalisation():
    rng = np.random.default_rng(9)
    X = rng.normal(size=(6, 5))
    W = rng.normal(size=(6, 5))
    Xh, nr = oracle.normalize(X)
    dX = oracle.normalize_backward(Xh, nr, W)      # d/dX of sum(W * X/||X||)
    h = 1e-6
    fd = np.zeros_like(X)
    for i in range(6):
        for k in range(5):
            Xp, Xm = X.copy(), X.copy()
            Xp[i, k] += h
            Xm[i, k] -= h
            fd[i, k] = ((W * oracle.normalize(Xp)[0]).sum()
                        - (W * oracle.normalize(Xm)[0]).sum()) / (2 * h)
    np.testing.assert_allclose(dX, fd, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose((dX * X).sum(-1), 0.0, atol=1e-12)   # orthogonal to x


def test_y_gradient_from_the_transposed_sparse_plan():
    # the COO of (Y, X, b, a, g, f) is the transpose of that of (X, Y, a, b, f, g); its
    # row-segment gradient is dL/dY = sum_i 2 P_ij (y_j - x_i), checked against finite
    # differences of the converged dual in y
    X, Y, a, b = _case(37, 10, 8)
    eps, iters = 0.1, 3000
    f, g = _converge(X, Y, a, b, eps, iters)
    r1, c1, v1, o1 = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-300)
    r2, c2, v2, o2 = oracle.plan_coo(Y, X, b, a, g, f, eps, rel_thr=1e-300)
    order = np.lexsort((r1, c1))        # CSR entries in column-major order
    np.testing.assert_array_equal(r2, c1[order])
    np.testing.assert_array_equal(c2, r1[order])
    # log P is symmetric in the two sides, roundings included: equal values bit for bit
    np.testing.assert_array_equal(v2, v1[order])
    _, dY = oracle.loss_grad(Y, X, r2, c2, v2, o2)

    def ot_value(Yv):
        fv, gv = oracle.potentials(X, Yv, a, b, eps=[eps], iters=[iters])
        return float(a @ fv + b @ gv)

    h = 1e-5
    fd = np.zeros_like(Y)
    for j in range(Y.shape[0]):
        for k in range(3):
            Yp, Ym = Y.copy(), Y.copy()
            Yp[j, k] += h
            Ym[j, k] -= h
            fd[j, k] = (ot_value(Yp) - ot_value(Ym)) / (2 * h)
    np.testing.assert_allclose(dY[0], fd, rtol=1e-6, atol=1e-8)


# ---------------------------------------- Sinkhorn normalisation in COO form
def test_coo_normalisation_of_the_full_support_reaches_the_dense_solution():
    # scaling the plan of early potentials on its full support converges to the
    # unique plan with marginals a, b of the same Gibbs kernel: converged Sinkhorn
    X, Y, a, b = _case(41, 18, 23)
    eps = 0.1
    f5, g5 = oracle.potentials(X, Y, a, b, eps=[eps], iters=[5])
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f5, g5, eps, rel_thr=1e-300)
    assert len(rows) == 18 * 23
    vn, err = oracle.coo_normalize(rows, cols, vals, offs, a, b, 18, 23, iters=3000)
    assert err[0, 0] < 1e-12 and err[0, 1] < 1e-12
    fc, gc = _converge(X, Y, a, b, eps, 3000)
    _, _, vref, _ = oracle.plan_coo(X, Y, a, b, fc, gc, eps, rel_thr=1e-300)
    np.testing.assert_allclose(vn, vref, rtol=1e-9)


def test_coo_normalisation_ignores_row_and_column_scalings_of_its_input():
    X, Y, a, b = _case(43, 30, 25)
    eps = 0.03
    f, g = oracle.potentials(X, Y, a, b, eps=[eps], iters=[8])
    rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-6)
    rng = np.random.default_rng(1)
    ru, cv = rng.uniform(0.1, 10, 30), rng.uniform(0.1, 10, 25)
    # the fixed point is unique on a support that admits the marginals
    v1, e1 = oracle.coo_normalize(rows, cols, vals, offs, a, b, 30, 25, iters=3000)
    v2, e2 = oracle.coo_normalize(rows, cols, vals * ru[rows] * cv[cols], offs, a, b, 30, 25,
                                  iters=3000)
    assert e1.max() < 1e-10 and e2.max() < 1e-10
    np.testing.assert_allclose(v2, v1, rtol=1e-7)
    # after a finite number of rounds the columns are exact (the last half-step)
    _, e3 = oracle.coo_normalize(rows, cols, vals, offs, a, b, 30, 25, iters=3)
    assert e3[0, 1] < 1e-13 < e3[0, 0]


def test_coo_normalisation_two_by_two_closed_form():
    # the scaled 2x2 matrix keeps the cross-ratio q11 q22 / (q12 q21) and has the
    # marginals: with x = q11, x (1 - a1 - b1 + x) = rho (a1 - x)(b1 - x)
    P = np.array([[0.3, 0.05], [0.2, 0.45]])
    a, b = np.array([0.4, 0.6]), np.array([0.7, 0.3])
    rows, cols = np.array([0, 0, 1, 1]), np.array([0, 1, 0, 1])
    vn, err = oracle.coo_normalize(rows, cols, P.ravel(), [0, 4], a, b, 2, 2, iters=500)
    rho = P[0, 0] * P[1, 1] / (P[0, 1] * P[1, 0])
    A, B1 = a[0], b[0]
    qa, qb, qc = 1 - rho, 1 - A - B1 + rho * (A + B1), -rho * A * B1
    roots = np.roots([qa, qb, qc])
    x = [r.real for r in roots if max(0, A + B1 - 1) < r.real < min(A, B1)][0]
    ref = np.array([x, A - x, B1 - x, 1 - A - B1 + x])
    np.testing.assert_allclose(vn, ref, rtol=1e-12)


# ---------------------------------------------------- Hessian-vector product
def test_hvp_is_the_derivative_of_the_converged_gradient():
    X, Y, a, b = _case(47, 9, 11)
    eps, iters = 0.1, 3000
    V = np.random.default_rng(4).normal(size=X.shape)

    def grad(Xv):
        f, g = oracle.potentials(Xv, Y, a, b, eps=[eps], iters=[iters])
        return oracle.dense_grad(Xv, Y, a, b, f, g, eps)[1][0]

    f, g = _converge(X, Y, a, b, eps, iters)
    HV = oracle.hvp(X, Y, a, b, f, g, eps, V)[0]
    h = 1e-5
    fd = (grad(X + h * V) - grad(X - h * V)) / (2 * h)
    np.testing.assert_allclose(HV, fd, rtol=1e-6, atol=1e-8 * np.abs(fd).max())


def test_hvp_is_symmetric():
    X, Y, a, b = _case(53, 12, 10, d=4)
    eps = 0.05
    f, g = _converge(X, Y, a, b, eps, 4000)
    rng = np.random.default_rng(5)
    U, V = rng.normal(size=X.shape), rng.normal(size=X.shape)
    HU = oracle.hvp(X, Y, a, b, f, g, eps, U)[0]
    HV = oracle.hvp(X, Y, a, b, f, g, eps, V)[0]
    assert abs((U * HV).sum() - (V * HU).sum()) <= 1e-10 * np.abs(U * HV).sum()


def test_hvp_zero_weight_points_are_absent_points():
    # a point of weight 0 carries no plan mass: the HVP of the other rows equals
    # that of the problem without the point, and the row of weight 0 gets 0
    X, Y, a, b = _case(59, 10, 9, d=3)
    a[3], b[[0, 5]] = 0.0, 0.0
    a, b = a / a.sum(), b / b.sum()
    eps = 0.1
    f, g = _converge(X, Y, a, b, eps, 3000)
    V = np.random.default_rng(6).normal(size=X.shape)
    HV = oracle.hvp(X, Y, a, b, f, g, eps, V)[0]
    kx, ky = np.arange(10) != 3, ~np.isin(np.arange(9), [0, 5])
    f, g = np.ravel(f), np.ravel(g)
    HVr = oracle.hvp(X[kx], Y[ky], a[kx], b[ky], f[kx], g[ky], eps, V[kx])[0]
    assert np.all(HV[3] == 0.0)
    np.testing.assert_allclose(HV[kx], HVr, rtol=1e-9, atol=1e-12 * np.abs(HVr).max())
