"""Double-precision CPU oracle for entropic OT between point clouds.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``sinkhorn_point_cloud_amd``) never imports, links or calls it, and the two
share no code.

The arithmetic lives in ``sinkhorn_oracle.c`` (plain C99, fp64, OpenMP over
rows); this module only marshals numpy arrays to it.  What each function
computes, and which page/section it follows, is documented in that file:

  [FS] "FlashSinkhorn: IO-bewuste Entropische Optimale Transport op GPU",
       Methodologie 1 (Propositie 1): the log-domain f-update and its attention
       form; the g-update is its mirror.
  [AP] "From Theory to Throughput: CUDA-Optimized APML for Large-Batch 3D
       Learning", Abstract / Innovation: thresholded sparse (COO) plan, loss
       and gradient on the stored support.

Parity status of each function (what pins it) is listed in ``PINS`` below;
every entry has at least one pin in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sinkhorn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# tests/test_oracle_mutations.py only: load this build (a deliberately broken
# copy of the oracle) instead, to check that the pins catch the mistake
_LIB_OVERRIDE = os.environ.get("SK_ORACLE_LIB")

PINS = {
    "half_update": "scipy logsumexp; brute-force assignment; 2x2 closed form; marginals",
    "potentials(direct)": "marginals at convergence; brute-force OT bound; large-eps limit;"
                          " n=1; 2x2 closed form; translation and swap invariance",
    "potentials(attention)": "agrees with the direct form (two different computations)",
    "plan_stats": "dense numpy enumeration; strong duality at convergence",
    "plan_coo": "dense numpy enumeration on small shapes",
    "loss_grad": "finite differences of the dual (envelope theorem); dense sums",
    "coo_normalize": "full support converges to the dense Sinkhorn plan; marginals at"
                     " convergence; invariance to row and column scalings of the input;"
                     " 2x2 closed form (cross-ratio kept)",
    "hvp": "finite differences of the converged dense gradient; symmetry <U, HV> = <V, HU>",
    "normalize": "unit norms, direction and scale invariance; cosine cost matrix 2 - 2 x.y"
                 " from numpy with scipy logsumexp for one update",
    "normalize_backward": "finite differences of a function of the normalised points;"
                          " orthogonality to the point",
    "dense_grad": "finite differences of the dual (envelope theorem); assignment limit of"
                  " the projection at small eps; product-plan limit at large eps; row mass"
                  " after an f-update; translation",
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_num_threads.restype = i32
        lib.oracle_half_update.argtypes = [P, i32, P, i32, i32, P, P, f64, P, i32, P]
        lib.oracle_half_update.restype = None
        lib.oracle_potentials.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, i32, i32, i32,
                                          P, P]
        lib.oracle_potentials.restype = i32
        lib.oracle_plan_stats.argtypes = [P, P, P, P, P, P, f64, i32, i32, i32, i32, P]
        lib.oracle_plan_stats.restype = None
        lib.oracle_plan_coo.argtypes = [P, P, P, P, P, P, f64, f64, i32, i32, i32, i32, i64,
                                        P, P, P, P]
        lib.oracle_plan_coo.restype = i64
        lib.oracle_loss_grad.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P, P]
        lib.oracle_loss_grad.restype = i32
        lib.oracle_dense_grad.argtypes = [P, P, P, P, P, P, f64, i32, i32, i32, i32, P, i64,
                                          P, P, P]
        lib.oracle_dense_grad.restype = None
        lib.oracle_normalize.argtypes = [P, i64, i32, P, P]
        lib.oracle_normalize.restype = None
        lib.oracle_normalize_backward.argtypes = [P, P, P, i64, i32, P]
        lib.oracle_normalize_backward.restype = None
        lib.oracle_coo_normalize.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P]
        lib.oracle_coo_normalize.restype = i32
        lib.oracle_hvp.argtypes = [P, P, P, P, P, P, f64, i32, i32, i32, i32, P, P]
        lib.oracle_hvp.restype = i32
        _lib = lib
    return _lib


def _d(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return x.ctypes.data_as(ctypes.c_void_p)


def _shapes(X, Y):
    X, Y = _d(X), _d(Y)
    if X.ndim == 2:
        X = X[None]
    if Y.ndim == 2:
        Y = Y[None]
    B, n, d = X.shape
    assert Y.shape[0] == B and Y.shape[2] == d
    return X, Y, B, n, Y.shape[1], d


def _weights(w, B, k):
    if w is None:
        return np.full((B, k), 1.0 / k)
    w = _d(w)
    return np.ascontiguousarray(w.reshape(B, k))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def half_update(P, Q, pot_q, w_q, eps, rows=None):
    """out_r = -eps * LSE_j[(pot_j - ||p_r - q_j||^2)/eps + log w_j] (single pair)."""
    lib = _load()
    P, Q = _d(P), _d(Q)
    pot_q, logw = _d(pot_q), np.log(_d(w_q))
    np_, d = P.shape
    nq = Q.shape[0]
    if rows is None:
        out = np.empty(np_)
        lib.oracle_half_update(_p(P), np_, _p(Q), nq, d, _p(pot_q), _p(logw), float(eps),
                               None, 0, _p(out))
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        out = np.empty(r.size)
        lib.oracle_half_update(_p(P), np_, _p(Q), nq, d, _p(pot_q), _p(logw), float(eps),
                               _p(r), int(r.size), _p(out))
    return out


def potentials(X, Y, a=None, b=None, eps=(0.05,), iters=(100,), form="direct",
               f0=None, g0=None):
    """Run the schedule; returns (f, g) shaped [B,n], [B,m] (or [n], [m] for 2-D input)."""
    lib = _load()
    squeeze = np.asarray(X).ndim == 2
    X, Y, B, n, m, d = _shapes(X, Y)
    a, b = _weights(a, B, n), _weights(b, B, m)
    eps = _d(np.atleast_1d(eps))
    it = np.ascontiguousarray(np.atleast_1d(iters).astype(np.int32))
    assert eps.size == it.size
    warm = g0 is not None
    f = np.zeros((B, n)) if f0 is None else _d(f0).reshape(B, n).copy()
    g = np.zeros((B, m)) if g0 is None else _d(g0).reshape(B, m).copy()
    rc = lib.oracle_potentials(_p(X), _p(Y), _p(a), _p(b), B, n, m, d, _p(eps), _p(it),
                               int(eps.size), 0 if form == "direct" else 1, int(warm),
                               _p(f), _p(g))
    if rc != 0:
        raise ValueError("oracle_potentials: bad arguments")
    return (f[0], g[0]) if squeeze else (f, g)


def plan_stats(X, Y, a, b, f, g, eps):
    """Per pair: dict of arrays cost, dual, row_err, col_err, kl (see the C file)."""
    lib = _load()
    X, Y, B, n, m, d = _shapes(X, Y)
    a, b = _weights(a, B, n), _weights(b, B, m)
    f, g = _d(f).reshape(B, n), _d(g).reshape(B, m)
    out = np.empty((B, 5))
    lib.oracle_plan_stats(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), float(eps), B, n, m, d,
                          _p(out))
    keys = ("cost", "dual", "row_err", "col_err", "kl")
    return {k: out[:, i].copy() for i, k in enumerate(keys)}


def plan_coo(X, Y, a, b, f, g, eps, rel_thr=1e-8):
    """Thresholded plan: (rows int32, cols int32, vals f64, pair_offsets int64[B+1])."""
    lib = _load()
    X, Y, B, n, m, d = _shapes(X, Y)
    a, b = _weights(a, B, n), _weights(b, B, m)
    f, g = _d(f).reshape(B, n), _d(g).reshape(B, m)
    offs = np.zeros(B + 1, dtype=np.int64)
    args = (_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), float(eps), float(rel_thr), B, n, m, d)
    total = lib.oracle_plan_coo(*args, 0, None, None, None, _p(offs))
    if total < 0:
        raise ValueError("oracle_plan_coo: bad arguments")
    rows = np.empty(max(total, 1), dtype=np.int32)
    cols = np.empty(max(total, 1), dtype=np.int32)
    vals = np.empty(max(total, 1), dtype=np.float64)
    total2 = lib.oracle_plan_coo(*args, int(total), _p(rows), _p(cols), _p(vals), _p(offs))
    assert total2 == total
    return rows[:total], cols[:total], vals[:total], offs


def loss_grad(X, Y, rows, cols, vals, pair_offsets):
    """(loss[B], dX[B,n,d]) on the stored support."""
    lib = _load()
    X, Y, B, n, m, d = _shapes(X, Y)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int32))
    vals = _d(vals)
    offs = np.ascontiguousarray(np.asarray(pair_offsets, dtype=np.int64))
    loss = np.empty(B)
    dX = np.empty((B, n, d))
    rc = lib.oracle_loss_grad(_p(X), _p(Y), B, n, m, d, _p(rows), _p(cols), _p(vals), _p(offs),
                              _p(loss), _p(dX))
    if rc != 0:
        raise ValueError("oracle_loss_grad: index out of range")
    return loss, dX


def dense_grad(X, Y, a, b, f, g, eps, sel=None):
    """Dense transport application at eps (X side): (r, dX, T).

    r[k] = sum_j P_ij, dX[k] = sum_j 2 P_ij (x_i - y_j), T[k] = sum_j P_ij y_j / r[k]
    for the rows listed in ``sel`` (flat indices p * n + i; None: all rows, shaped
    [B,n] / [B,n,d]).  For the Y side pass (Y, X, b, a, g, f)."""
    lib = _load()
    X, Y, B, n, m, d = _shapes(X, Y)
    a, b = _weights(a, B, n), _weights(b, B, m)
    f, g = _d(f).reshape(B, n), _d(g).reshape(B, m)
    if sel is None:
        k = B * n
        selp, cnt = None, 0
    else:
        s = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
        assert s.min() >= 0 and s.max() < B * n
        k, selp, cnt = s.size, _p(s), s.size
    r = np.empty(k)
    dX = np.empty((k, d))
    T = np.empty((k, d))
    lib.oracle_dense_grad(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), float(eps), B, n, m, d,
                          selp, cnt, _p(r), _p(dX), _p(T))
    if sel is None:
        return r.reshape(B, n), dX.reshape(B, n, d), T.reshape(B, n, d)
    return r, dX, T


def normalize(X):
    """(Xh, norms): points scaled to unit length (zero vectors stay 0), any leading shape."""
    lib = _load()
    X = _d(X)
    d = X.shape[-1]
    count = X.size // d
    out = np.empty_like(X)
    norms = np.empty(X.shape[:-1])
    lib.oracle_normalize(_p(X), count, d, _p(out), _p(norms))
    return out, norms


def normalize_backward(Xh, norms, G):
    """dX = (G - xh (xh . G)) / ||x||, the gradient through x -> x / ||x||."""
    lib = _load()
    Xh, norms, G = _d(Xh), _d(norms), _d(G)
    d = Xh.shape[-1]
    dX = np.empty_like(Xh)
    lib.oracle_normalize_backward(_p(Xh), _p(norms), _p(G), Xh.size // d, d, _p(dX))
    return dX


def coo_normalize(rows, cols, vals, pair_offsets, a, b, n, m, iters):
    """Sinkhorn normalisation of a COO plan on its support: (vals', err[B,2])."""
    lib = _load()
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int32))
    vals = _d(vals).copy()
    offs = np.ascontiguousarray(np.asarray(pair_offsets, dtype=np.int64))
    B = offs.size - 1
    a, b = _weights(a, B, n), _weights(b, B, m)
    err = np.empty((B, 2))
    rc = lib.oracle_coo_normalize(_p(rows), _p(cols), _p(vals), _p(offs), _p(a), _p(b), B, n, m,
                                  int(iters), _p(err))
    if rc != 0:
        raise ValueError("oracle_coo_normalize: index out of range")
    return vals, err


def hvp(X, Y, a, b, f, g, eps, V):
    """Hessian-vector product of the entropic OT value in X along V [B,n,d] (dense, small)."""
    lib = _load()
    X, Y, B, n, m, d = _shapes(X, Y)
    a, b = _weights(a, B, n), _weights(b, B, m)
    f, g = _d(f).reshape(B, n), _d(g).reshape(B, m)
    V = _d(V).reshape(B, n, d)
    HV = np.empty((B, n, d))
    rc = lib.oracle_hvp(_p(X), _p(Y), _p(a), _p(b), _p(f), _p(g), float(eps), B, n, m, d, _p(V),
                        _p(HV))
    if rc != 0:
        raise ValueError("oracle_hvp: system not positive definite")
    return HV
