"""Seeded synthetic inputs for the five point-cloud workloads and for small tests.

This module only draws numbers: it holds none of the transport arithmetic, and
both sides (the GPU library and the CPU oracle) take their inputs from here.
Every array is produced in float64 with numpy's PCG64 generator and then
rounded once to the dtype handed to the GPU (float32, or bfloat16 with
round-to-nearest-even); the oracle receives exactly those rounded values,
up-cast to float64, so input quantisation never counts as error.

Workloads (sizes and distributions as the pages' point-cloud settings):
  pair-1k    1 pair, n=m=1024, d=3: X, Y i.i.d. uniform in [0,1]^3 (seed 0),
             uniform weights, eps=0.05, 100 full iterations -> potentials + cost.
  sphere-2k  32 pairs, n=m=2048, d=3: X on the unit sphere + N(0, 0.01^2),
             Y = permuted X + N(0, 0.02^2); uniform weights; eps=0.01,
             50 iterations -> COO plan at 1e-8 * max P per pair, loss.
  blobs-1k   256 pairs, n=m=1024, d=3: 4-cluster blobs (centres U[-1,1]^3,
             sigma 0.1), Y independent; eps=0.02, 30 iterations -> COO plan,
             loss, dL/dX.  Stands in for large-batch point-cloud training.
  gmm-64k    1 pair, n=m=65536, d=3: 8-component mixtures (centres U[-2,2]^3,
             sigma 0.15); Dirichlet(1) weights; eps annealed geometrically
             1.0 -> 0.01 over 10 stages of 20 iterations -> potentials + cost.
  feat-50k   1 pair, n=50000, m=60000, d=64: N(0,1)/8 entries stored as bf16;
             uniform weights; eps=0.1, 50 iterations -> potentials + cost.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = ("pair-1k", "sphere-2k", "blobs-1k", "gmm-64k", "feat-50k")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    bits = bits.astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))


def _blobs(rng, n, k, lo, hi, sigma):
    centres = rng.uniform(lo, hi, size=(k, 3))
    labels = rng.integers(0, k, size=n)
    return centres[labels] + sigma * rng.standard_normal((n, 3))


def _sphere_pair(p, n):
    rng = np.random.default_rng([2, p, 0])
    z = rng.standard_normal((n, 3))
    x = z / np.linalg.norm(z, axis=1, keepdims=True) + 0.01 * rng.standard_normal((n, 3))
    perm = rng.permutation(n)
    y = x[perm] + 0.02 * rng.standard_normal((n, 3))
    return x, y


def geometric_schedule(start: float, stop: float, stages: int) -> np.ndarray:
    """Geometric eps schedule with both end points, rounded to float32."""
    k = np.arange(stages, dtype=np.float64)
    eps = start * (stop / start) ** (k / (stages - 1)) if stages > 1 else np.array([stop])
    return eps.astype(np.float32)


def make(name: str, pairs=None) -> dict:
    """Inputs for one workload.  ``pairs`` selects a subset of the batch (the
    per-pair streams are independent, so a subset is bit-identical to the same
    pairs of the full batch).  Returns a dict with X, Y (float32 [B,n,d]; for
    bf16 workloads also X_bits/Y_bits uint16), a, b (float32 [B,n], [B,m]),
    eps (float32 [stages]), iters (int32 [stages]), dtype, threshold, pairs."""
    if name == "pair-1k":
        rng = np.random.default_rng(0)
        X = rng.random((1024, 3))
        Y = rng.random((1024, 3))
        out = dict(X=_f32(X)[None], Y=_f32(Y)[None], eps=np.float32([0.05]), iters=[100],
                   dtype="f32", threshold=None, pair_ids=[0])
        n = m = 1024
        out["a"] = np.full((1, n), 1.0 / n, dtype=np.float32)
        out["b"] = np.full((1, m), 1.0 / m, dtype=np.float32)
    elif name == "sphere-2k":
        ids = list(range(32)) if pairs is None else list(pairs)
        n = 2048
        xs, ys = zip(*[_sphere_pair(p, n) for p in ids])
        out = dict(X=_f32(np.stack(xs)), Y=_f32(np.stack(ys)), eps=np.float32([0.01]),
                   iters=[50], dtype="f32", threshold=1e-8, pair_ids=ids)
        out["a"] = np.full((len(ids), n), 1.0 / n, dtype=np.float32)
        out["b"] = np.full((len(ids), n), 1.0 / n, dtype=np.float32)
    elif name == "blobs-1k":
        ids = list(range(256)) if pairs is None else list(pairs)
        n = 1024
        xs = [_blobs(np.random.default_rng([3, p, 0]), n, 4, -1.0, 1.0, 0.1) for p in ids]
        ys = [_blobs(np.random.default_rng([3, p, 1]), n, 4, -1.0, 1.0, 0.1) for p in ids]
        out = dict(X=_f32(np.stack(xs)), Y=_f32(np.stack(ys)), eps=np.float32([0.02]),
                   iters=[30], dtype="f32", threshold=1e-8, pair_ids=ids)
        out["a"] = np.full((len(ids), n), 1.0 / n, dtype=np.float32)
        out["b"] = np.full((len(ids), n), 1.0 / n, dtype=np.float32)
    elif name == "gmm-64k":
        n = m = 65536
        X = _blobs(np.random.default_rng([4, 0, 0]), n, 8, -2.0, 2.0, 0.15)
        Y = _blobs(np.random.default_rng([4, 0, 1]), m, 8, -2.0, 2.0, 0.15)
        a = np.random.default_rng([4, 0, 2]).dirichlet(np.ones(n))
        b = np.random.default_rng([4, 0, 3]).dirichlet(np.ones(m))
        out = dict(X=_f32(X)[None], Y=_f32(Y)[None], a=_f32(a / a.sum())[None],
                   b=_f32(b / b.sum())[None], eps=geometric_schedule(1.0, 0.01, 10),
                   iters=[20] * 10, dtype="f32", threshold=None, pair_ids=[0])
    elif name == "feat-50k":
        n, m, d = 50000, 60000, 64
        X = np.random.default_rng([5, 0, 0]).standard_normal((n, d)) / 8.0
        Y = np.random.default_rng([5, 0, 1]).standard_normal((m, d)) / 8.0
        xb, yb = bf16_round(X), bf16_round(Y)
        out = dict(X_bits=xb[None], Y_bits=yb[None], X=bf16_to_f32(xb)[None],
                   Y=bf16_to_f32(yb)[None], eps=np.float32([0.1]), iters=[50],
                   dtype="bf16", threshold=None, pair_ids=[0])
        out["a"] = np.full((1, n), 1.0 / n, dtype=np.float32)
        out["b"] = np.full((1, m), 1.0 / m, dtype=np.float32)
    else:
        raise KeyError(f"unknown workload {name!r}; known: {WORKLOADS}")
    out["iters"] = np.asarray(out["iters"], dtype=np.int32)
    out["name"] = name
    return out


def random_case(seed: int, B: int, n: int, m: int, d: int, weights: str = "uniform",
                spread: float = 1.0, dtype: str = "f32", zero_weights: int = 0) -> dict:
    """Small random pair batch for tests: points uniform in [0, spread]^d,
    weights uniform or Dirichlet(1) (normalised in float64, then rounded).
    ``zero_weights`` > 0 sets that many leading entries of a and b to 0
    before normalising."""
    rng = np.random.default_rng([7, seed, B, n, m, d])
    X = spread * rng.random((B, n, d))
    Y = spread * rng.random((B, m, d))
    if weights == "uniform":
        a = np.full((B, n), 1.0 / n)
        b = np.full((B, m), 1.0 / m)
    else:
        a = rng.dirichlet(np.ones(n), size=B)
        b = rng.dirichlet(np.ones(m), size=B)
    if zero_weights:
        a[:, :zero_weights] = 0.0
        b[:, :zero_weights] = 0.0
        a /= a.sum(axis=1, keepdims=True)
        b /= b.sum(axis=1, keepdims=True)
    out = dict(a=_f32(a), b=_f32(b), dtype=dtype)
    if dtype == "bf16":
        xb, yb = bf16_round(X), bf16_round(Y)
        out.update(X_bits=xb, Y_bits=yb, X=bf16_to_f32(xb), Y=bf16_to_f32(yb))
    else:
        out.update(X=_f32(X), Y=_f32(Y))
    return out
