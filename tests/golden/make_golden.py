"""Write the oracle's expected values for the five workloads.

Usage:  python tests/golden/make_golden.py [workload ...]   (default: all)

Every stored number comes from ``oracle/`` (the fp64 CPU oracle) run on the
inputs from ``workloads.make``; nothing here touches the GPU library.  One
compressed ``<workload>.npz`` per workload holds:
  input_sum   float64 checksum of X, Y, a, b (guards against generator drift)
  f, g        potentials [B,n], [B,m] (float64 for pair-1k, float32 otherwise:
              the parity tolerance is 1e-4, far above float32 rounding)
  cost, dual, row_err, col_err   per pair, at the final eps
  coo_nnz, loss    per pair, for the workloads with a sparse plan, from the
              oracle's own COO of its own potentials
  dX_pairs, dX     gradient of a few sampled pairs
  seconds, threads  oracle wall time and OpenMP threads used
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
DX_PAIRS = {"sphere-2k": [0, 31], "blobs-1k": [0, 1, 128, 255]}


def input_sum(w):
    return float(sum(np.asarray(w[k], dtype=np.float64).sum() for k in ("X", "Y", "a", "b")))


def run(name):
    w = workloads.make(name)
    X, Y, a, b = (w[k].astype(np.float64) for k in ("X", "Y", "a", "b"))
    eps = w["eps"].astype(np.float64)
    t0 = time.time()
    f, g = oracle.potentials(X, Y, a, b, eps=eps, iters=w["iters"])
    seconds = time.time() - t0
    out = dict(input_sum=input_sum(w), seconds=seconds, threads=oracle.num_threads())
    st = oracle.plan_stats(X, Y, a, b, f, g, eps[-1])
    out.update({k: st[k] for k in ("cost", "dual", "row_err", "col_err")})
    if w["threshold"] is not None:
        rows, cols, vals, offs = oracle.plan_coo(X, Y, a, b, f, g, eps[-1], w["threshold"])
        loss, dX = oracle.loss_grad(X, Y, rows, cols, vals, offs)
        out["coo_nnz"] = np.diff(offs)
        out["loss"] = loss
        out["dX_pairs"] = np.asarray(DX_PAIRS[name], dtype=np.int64)
        out["dX"] = dX[DX_PAIRS[name]].astype(np.float32)
    store = np.float64 if name == "pair-1k" else np.float32
    out["f"], out["g"] = f.astype(store), g.astype(store)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: oracle {seconds:.1f} s on {out['threads']} threads; "
          f"cost {out['cost'][:3]} -> {path}", flush=True)


if __name__ == "__main__":
    for name in sys.argv[1:] or workloads.WORKLOADS:
        run(name)
