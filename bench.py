"""Benchmark of the streaming Sinkhorn hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gmm-64k] [--no-cpu-baseline]

One step is the whole workload's hot path on inputs already resident in HBM:
pack, every (annealed) Sinkhorn half-iteration, then the transport-cost pass
(gmm-64k: 65536 x 65536 points, d = 3, eps 1.0 -> 0.01 over 10 stages of 20
iterations; pair-1k; feat-50k) or, for the sparse-plan workloads (sphere-2k,
blobs-1k), the thresholded COO plan and the loss and dL/dX computed from it.  Prints ONE JSON line with
  value      B*n*m*iters / step time   (cost-entry updates per second)
  roofline   the dominant kernel: entry evaluations per launch / its average
             launch time (events on the library's stream: a potentials call with
             the workload's schedule minus the same call with every iteration
             count 0, divided by the launches the iterations make -- one per
             half-iteration, or one per stage for the per-pair launch), against
             the chip's exp issue bound (one exponential per entry; the d = 3
             scores run on the matrix cores) or, for bf16 features, the matrix
             cores; beside it the metric's min(FP32, exp) roofline and the
             kernel's own instruction-issue floor
  cpu_baseline  the fp64 oracle timed on two full iterations of the same
             problem on this host's cores, scaled to updates per second, with
             the cached time of the oracle's full run.
  --rates    adds the chip's measured instruction rates and clock (probe kernels).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X (gfx950) unit counts and clock
N_CU = 256
N_SIMD = 4 * N_CU
CLOCK_HZ = 2.4e9
FP32_VECTOR_PEAK = 157.3e12        # flop/s (packed FP32 FMA)
BF16_MFMA_PEAK = 2.5e15            # flop/s, dense
FLOPS_PER_EVAL_D3 = 9              # 3 mul + 3 add (score with bias) + max, subtract, accumulate
# v_exp_f32 issues at a quarter of the FP32 lane rate: 128 FMA lanes per compute unit
# per clock (157.3 TFLOP/s / 256 CUs / 2.4 GHz / 2), 32 exponential lanes (the rate
# probe measures 29.2 and 112; profiles/rates_mi355x.md)
EXP_LANES_PER_CLK_CU = 32

# SIMD cycles per wave and 16-key tile (64 rows x 16 keys = 1024 entries) of each
# streaming kernel's instruction mix, measured by the rate probe on the mix itself
# (profiles/rates_mi355x.md): the d = 3 tile, 4 MFMA + 16 exp + 16 add on their
# outputs, 220; the d = 64 bf16 feature tile, 8 MFMA + 16 fma + 16 exp + 16 add, 314.
# The vector kernels' mixes are priced with the probe's single-instruction costs
# (exp 8.8 cycles, fp32 add or fma 2.3).
TILE_CYCLES = {
    "lse3m_kernel": 220.0,
    "lse3p_kernel": 220.0,
    "lse3s_kernel": 220.0,
    "lseFs_kernel": 314.0,
    "lse3_kernel": 16 * 8.8 + 64 * 2.3,        # 3 fma + 1 add per entry on top of the exp
    "lseF_kernel": 16 * 8.8 + 16 * 66 * 2.3,   # 64-dim dot products on the vector ALUs
}
TILE_PROBE = {"lse3m_kernel": "d3_tile", "lse3p_kernel": "d3_tile", "lse3s_kernel": "d3_tile",
              "lseFs_kernel": "feature_tile"}


def issue_floor_evals_per_s(kernel, cycles=None):
    """Entry evaluations per second if every SIMD issued the kernel's tile mix back
    to back at the nominal clock (the kernel's own instruction-issue bound)."""
    return N_SIMD * CLOCK_HZ * 1024 / (cycles or TILE_CYCLES[kernel])


def roofline_evals_per_s(d, kernel):
    """(peak, bound, basis, algorithmic min(FP32, exp) bound) in evaluations/s.
    Every entry needs one exponential, so the exp issue rate bounds every design:
    256 CUs x 32 lanes x 2.4 GHz.  d = 3 with scores on the matrix cores: the vector
    ALUs keep only the exponential and the accumulation, so the exp bound is the peak
    (the 9 FP32 flops of the algorithmic count run on the matrix cores).  d = 3 with
    vector scores: min(FP32 vector / 9 flops, exp).  bf16 features: min(MFMA dense
    bf16 / 2d flops, exp)."""
    exp = N_CU * CLOCK_HZ * EXP_LANES_PER_CLK_CU
    fp32 = FP32_VECTOR_PEAK / FLOPS_PER_EVAL_D3
    algo = min(fp32, exp)
    if d == 3 and kernel in ("lse3m_kernel", "lse3p_kernel", "lse3s_kernel"):
        return exp, "alu", ("exp issue: 256 CUs x 32 v_exp_f32 lanes/clk x 2.4 GHz, one exp per "
                            "entry (score and bias on the matrix cores)"), algo
    if d == 3:
        return algo, "alu", "min(FP32 157.3 TFLOP/s / 9 flops, exp issue)", algo
    mfma = BF16_MFMA_PEAK / (2 * d)
    peak = min(mfma, exp)
    return peak, "mfma" if peak == mfma else "alu", (
        f"min(bf16 MFMA 2.5 PFLOP/s / {2 * d} flops, exp issue)"), algo


# sources whose change invalidates a kernel's committed traffic counters
KERNEL_SOURCES = {
    "lse3m_kernel": ("sinkhorn_point_cloud_amd/csrc/lse_d3.hip",
                     "sinkhorn_point_cloud_amd/csrc/common.h"),
    "lse3p_kernel": ("sinkhorn_point_cloud_amd/csrc/lse_d3.hip",
                     "sinkhorn_point_cloud_amd/csrc/common.h"),
    "lse3s_kernel": ("sinkhorn_point_cloud_amd/csrc/lse_d3.hip",
                     "sinkhorn_point_cloud_amd/csrc/common.h"),
    "lseFs_kernel": ("sinkhorn_point_cloud_amd/csrc/lse_feat.hip",
                     "sinkhorn_point_cloud_amd/csrc/common.h"),
}


def source_hash(sources):
    """First 16 hex digits of the sha256 of the kernel's source files, in order."""
    import hashlib

    h = hashlib.sha256()
    for src in sources:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel's sources have changed since it was taken."""
    import glob

    sha = source_hash(sources)
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md")):
        for line in open(path):
            parts = line.split()
            if (len(parts) == 6 and parts[0] == "traffic_bytes_per_launch"
                    and parts[1] == kernel and parts[2] == workload):
                return float(parts[3]) if parts[5] == sha else None
    return None


PROBE_KINDS = (  # kind: (name, per wave per iteration: {instruction: count})
    (0, "exp", {"v_exp_f32": 16}),
    (1, "fma", {"v_fma_f32": 16}),
    (2, "exp_add", {"v_exp_f32": 16, "v_add_f32": 16}),
    (3, "mfma", {"v_mfma_f32_16x16x32_bf16": 4}),
    (4, "d3_tile", {"v_mfma_f32_16x16x32_bf16": 4, "v_exp_f32": 16, "v_add_f32": 16}),
    (5, "fma_f64", {"v_fma_f64": 16}),
    (6, "feature_tile", {"v_mfma_f32_16x16x32_bf16": 8, "v_fma_f32": 16, "v_exp_f32": 16,
                         "v_add_f32": 16}),
    (7, "mfma32", {"v_mfma_f32_32x32x16_bf16": 2}),
    (8, "feature_tile_32x32", {"v_mfma_f32_32x32x16_bf16": 4, "v_fma_f32": 16, "v_exp_f32": 16,
                               "v_add_f32": 16}),
)


def measure_rates(dev, blocks_per_cu=8, target_s=0.02):
    """Instruction rates of the chip from the library's probe kernels: per mix, the
    shader clock under load (core-clock counter over the constant-rate wall clock)
    and the rate per compute unit per clock of each instruction it issues."""
    import ctypes

    import torch

    import sinkhorn_point_cloud_amd as sk

    lib = sk.load_library()
    lib.sinkhorn_probe_rates.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.sinkhorn_probe_rates.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * blocks_per_cu
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.empty(blocks * 4, dtype=torch.int64, device=dev)
    hz = ctypes.c_double(0.0)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {"compute_units": cus, "work_groups": blocks, "waves_per_simd": blocks_per_cu}

    def run(kind, iters):
        rc = lib.sinkhorn_probe_rates(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.c_void_p(clocks.data_ptr()), ctypes.byref(hz),
                                      stream)
        assert rc == 0, f"rate probe {kind}: status {rc}"
        torch.cuda.synchronize()
        c = clocks.view(blocks, 4).cpu().numpy().astype("float64")
        wall = (c[:, 3].max() - c[:, 2].min()) / hz.value     # first start to last end
        sclk = (c[:, 1] - c[:, 0]).sum() / (c[:, 3] - c[:, 2]).sum() * hz.value
        return wall, sclk

    for kind, name, mix in PROBE_KINDS:
        iters = 256
        run(kind, iters)
        wall, _ = run(kind, iters)
        iters = max(256, int(iters * target_s / max(wall, 1e-6)))
        wall, sclk = run(kind, iters)
        waves = blocks * 4
        rec = {"iters": iters, "seconds": wall, "sclk_ghz": sclk / 1e9}
        for ins, cnt in mix.items():
            per_cu_clk = waves * iters * cnt * 64 / (wall * sclk * cus)   # lanes
            rec[ins + "_lanes_per_clk_cu"] = per_cu_clk
        cycles = wall * sclk * cus * 4 / (waves * iters)   # SIMD cycles per wave-iteration
        rec["simd_cycles_per_wave_iteration"] = cycles
        out[name] = rec
    return out


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="gmm-64k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--valu-scores", action="store_true",
                   help="d = 3: form scores on the vector ALUs (comparison)")
    p.add_argument("--graph", action="store_true",
                   help="capture one step in a HIP graph and time its replays (the remedy for "
                        "launch-bound shapes; the potentials after the timed replays are "
                        "checked against an eager step)")
    p.add_argument("--rates", action="store_true",
                   help="also measure the chip's instruction rates with the library's probe "
                        "kernels (exp, FMA, MFMA, the d = 3 tile mix, fp64 FMA) and the clock")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy, so that HBM byte counters of "
                        "a profiler run can be scaled by a kernel of known traffic")
    return p.parse_args()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, iters=2):
    """Oracle (as it stands) on `iters` full iterations of the workload at its final eps,
    beside the cached time of the oracle's full run of the same workload (written by
    tests/golden/make_golden.py, on the host and thread count stored with it)."""
    import numpy as np
    import oracle

    X, Y, a, b = (w[k].astype(np.float64) for k in ("X", "Y", "a", "b"))
    B, n, m = X.shape[0], X.shape[1], Y.shape[1]
    t0 = time.perf_counter()
    oracle.potentials(X, Y, a, b, eps=[float(w["eps"][-1])], iters=[iters])
    dt = time.perf_counter() - t0
    out = {"value": B * n * m * iters / dt, "unit": "updates/s", "cores": oracle.num_threads(),
           "kind": "oracle", "cpu_model": cpu_model(),
           "logical_cpus_visible": len(os.sched_getaffinity(0)),
           "sample": f"{iters} full iterations (f- and g-updates, {2 * iters * B * n * m:.3g} "
                     f"entry evaluations) of {w['name']} at eps={float(w['eps'][-1]):g}, fp64, "
                     f"{dt:.2f} s (extrapolated rate)"}
    gold = os.path.join(ROOT, "tests", "golden", f"{w['name']}.npz")
    if os.path.exists(gold):
        z = np.load(gold)
        total = B * n * m * int(np.sum(w["iters"]))
        out["cached_full_run"] = {"seconds": float(z["seconds"]), "threads": int(z["threads"]),
                                  "value": total / float(z["seconds"]), "unit": "updates/s",
                                  "note": "the oracle's full schedule, timed once when the "
                                          "expected values were written (build container)"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); splitting the path "
              "across GPUs is designed, not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sinkhorn_point_cloud_amd as sk
    import workloads

    w = workloads.make(args.workload)
    dev = torch.device("cuda:0")
    if w["dtype"] == "bf16":
        X = torch.from_numpy(w["X_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        Y = torch.from_numpy(w["Y_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        X, Y = torch.from_numpy(w["X"]).to(dev), torch.from_numpy(w["Y"]).to(dev)
    a, b = torch.from_numpy(w["a"]).to(dev), torch.from_numpy(w["b"]).to(dev)
    B, n, d = X.shape
    m = Y.shape[1]
    eps = [float(e) for e in w["eps"]]
    iters = [int(i) for i in w["iters"]]
    total_iters = sum(iters)
    f = torch.empty(B, n, device=dev)
    g = torch.empty(B, m, device=dev)
    cost = torch.empty(B, device=dev)
    dt = sk.SK_F32 if w["dtype"] == "f32" else sk.SK_BF16
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_POTENTIALS, B, n, m, d, dt), dtype=torch.uint8,
                     device=dev)

    sparse = w["threshold"] is not None
    with_cost_default = not sparse
    coo = loss_out = nnz_dev = None
    if sparse:
        # size the plan once (untimed); the timed steps reuse the buffers
        sk.potentials(X, Y, a, b, eps=eps, iters=iters, out=(f, g, None), cost=False,
                      workspace=ws)
        r0, _, _, _ = sk.plan_coo(X, Y, a, b, f, g, eps[-1], w["threshold"])
        cap = int(r0.numel() * 1.05) + 1024
        coo = (torch.empty(cap, dtype=torch.int32, device=dev),
               torch.empty(cap, dtype=torch.int32, device=dev),
               torch.empty(cap, dtype=torch.float32, device=dev),
               torch.empty(B + 1, dtype=torch.int64, device=dev))
        coo_ws = torch.empty(sk.workspace_bytes(sk.SK_OP_PLAN_COO, B, n, m, d, dt),
                             dtype=torch.uint8, device=dev)
        loss_out = (torch.empty(B, device=dev), torch.empty(B, n, d, device=dev))
        nnz_dev = torch.empty(1, dtype=torch.int64, device=dev)

    def step(it=iters, with_cost=with_cost_default):
        sk.potentials(X, Y, a, b, eps=eps, iters=it, out=(f, g, cost if with_cost else None),
                      cost=with_cost, workspace=ws, valu_scores=args.valu_scores)
        if sparse:
            # the loss and dL/dX are accumulated while the plan is emitted; no host
            # wait inside the step (the count is checked against the capacity after)
            sk.plan_coo_async(X, Y, a, b, f, g, eps[-1], w["threshold"], coo, loss_out=loss_out,
                              workspace=coo_ws, nnz=nnz_dev)

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    def warm(fn, calls, seconds):
        # untimed calls until both counts are reached: the GPU's clocks ramp up over
        # the first tens of milliseconds of sustained work (a kernel runs 10-15%
        # slower right after an idle gap), and the timed region should see them settled
        torch.cuda.synchronize()
        t0, k = time.perf_counter(), 0
        while k < calls or time.perf_counter() - t0 < seconds:
            fn()
            k += 1
            torch.cuda.synchronize()

    run_step = step
    if args.graph:
        # one eager step for reference, then the same step captured once and replayed
        warm(step, 1, 0.0)
        ref = [t.clone() for t in (f, g)]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step()
        torch.cuda.synchronize()
        run_step = graph.replay
    warm(run_step, args.warmup, 0.25)
    t0 = time.perf_counter()
    t_step = timed(run_step, args.steps)
    wall = time.perf_counter() - t0
    if args.graph:
        for t, r in zip((f, g), ref):
            assert torch.equal(t, r), "graph replay differs from the eager step"
    assert torch.isfinite(f).all() and torch.isfinite(g).all()
    assert sparse or torch.isfinite(cost).all()
    assert not sparse or int(nnz_dev) <= coo[0].numel(), "plan outgrew its buffers"

    if d == 3:
        # how the library runs the iterations for these sizes on this device: one
        # launch per half-iteration, or one per eps stage (a work-group per pair for
        # large batches, each pair over 16-row work-groups for small ones)
        import ctypes

        lib = sk.load_library()
        lib.sinkhorn_probe_potentials_path.argtypes = [ctypes.c_int] * 5 + [ctypes.c_uint]
        lib.sinkhorn_probe_potentials_path.restype = ctypes.c_int
        shape = lib.sinkhorn_probe_potentials_path(
            B, n, m, d, dt, sk.SK_VALU_SCORES if args.valu_scores else 0)
        assert 0 <= shape <= 3, f"launch shape query: {shape}"
        kernel = ("lse3m_kernel", "lse3p_kernel", "lse3s_kernel", "lse3_kernel")[shape]
        pairwise = shape in (1, 2)   # one launch per stage
    else:
        pairwise = False
        kernel = "lseFs_kernel" if dt == sk.SK_BF16 and d % 32 == 0 else "lseF_kernel"

    # the dominant kernel's average launch: one potentials call (no cost pass, no
    # plan) less the same call with every iteration count 0 (centering and packing
    # only), over the launches its iterations make: one per half-iteration, or one
    # per stage for the per-pair launch.  The difference also holds the query
    # records built once per stage (two small launches).
    def potentials_only(it):
        sk.potentials(X, Y, a, b, eps=eps, iters=it, out=(f, g, None), cost=False,
                      workspace=ws, valu_scores=args.valu_scores)

    reps = max(3, args.steps)
    warm(lambda: potentials_only(iters), 1, 0.1)
    t_iterations = (timed(lambda: potentials_only(iters), reps)
                    - timed(lambda: potentials_only([0] * len(iters)), reps))
    potentials_only(iters)   # the converged potentials again, for the phases below
    launches = sum(1 for i in iters if i) if pairwise else 2 * total_iters
    t_launch = t_iterations / launches
    evals_per_launch = 2 * B * n * m * total_iters / launches
    achieved = evals_per_launch / t_launch
    peak, bound, basis, algo = roofline_evals_per_s(d, kernel)
    floor = issue_floor_evals_per_s(kernel)

    updates = B * n * m * total_iters
    line = {
        "metric": "Sinkhorn cost-entry updates/s (B*n*m*iters/s); % of exp/FP32 roofline",
        "value": updates / t_step,
        "unit": "updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "n": n, "m": m, "d": d,
                   "eps": f"{eps[0]:g}->{eps[-1]:g} over {len(eps)} stage(s)",
                   "iters": total_iters,
                   "launch": "hip graph replay of the step" if args.graph else "eager",
                   # the d = 3 score does not run on the vector ALUs as the pages expected:
                   # it runs on bf16 matrix cores from an exact three-piece split of the
                   # fp32 operands (--valu-scores times the vector-score kernel instead)
                   "scores": ("vector ALUs (fp32 FMAs)" if args.valu_scores or kernel.startswith(
                       ("lse3_kernel", "lseF_kernel")) else
                              "bf16 matrix cores, exact 3-piece split of the fp32 operands"
                              if d == 3 else "bf16 matrix cores (bf16 inputs)"),
                   "outputs": ("potentials, COO plan at %g x max P per pair, loss and dL/dX"
                               % w["threshold"]) if sparse
                   else "potentials f, g and transport cost",
                   **({"plan_entries": int(coo[3][-1].item())} if sparse else {})},
        "roofline": {"bound": bound, "achieved": achieved / 1e12, "peak": peak / 1e12,
                     "unit": "Teval/s", "frac": achieved / peak,
                     "traffic": measured_traffic(kernel, w["name"], KERNEL_SOURCES[kernel])
                     if kernel in KERNEL_SOURCES else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "scaled by a 256 MiB copy)",
                     "kernel": kernel + (" (one launch: a stage of %d iterations for every pair%s)"
                                         % (total_iters // launches,
                                            ", each pair over work-groups of 16 rows"
                                            if kernel == "lse3s_kernel" else "")
                                         if pairwise else " (one launch: a half-iteration)"),
                     "launch_ms": t_launch * 1e3, "evals_per_launch": evals_per_launch,
                     "peak_basis": basis,
                     # the metric's exp/FP32 roofline: min(FP32 vector / 9 flops, exp issue)
                     "exp_fp32_roofline": algo / 1e12, "frac_of_exp_fp32_roofline": achieved / algo,
                     # the kernel's own instruction-issue bound: its per-tile mix of MFMAs,
                     # exponentials and other vector instructions issued back to back
                     "issue_floor": floor / 1e12, "frac_of_issue_floor": achieved / floor,
                     "tile_cycles": TILE_CYCLES[kernel]},
        "phases_ms": {"step": t_step * 1e3, "iterations": t_iterations * 1e3,
                      ("pack_plan_and_loss" if sparse else "pack_and_cost_pass"):
                      (t_step - t_iterations) * 1e3},
        "wall_s_timed": wall,
    }
    if sparse:
        # Sinkhorn normalisation of the sparse plan on its support (10 rounds),
        # with the transposed plan it needs; reported beside the step
        t_rows = torch.empty(cap, dtype=torch.int32, device=dev)
        t_cols = torch.empty(cap, dtype=torch.int32, device=dev)
        t_vals = torch.empty(cap, dtype=torch.float32, device=dev)
        t_offs = torch.empty(B + 1, dtype=torch.int64, device=dev)
        rows, cols, vals, offs = sk.plan_coo(X, Y, a, b, f, g, eps[-1], w["threshold"],
                                             workspace=coo_ws, out=coo)
        tr = sk.plan_coo(Y, X, b, a, g, f, eps[-1], w["threshold"], workspace=coo_ws,
                         out=(t_rows, t_cols, t_vals, t_offs))
        cn_ws = torch.empty(sk.load_library().sinkhorn_coo_workspace_bytes(B, n, m, rows.numel()),
                            dtype=torch.uint8, device=dev)
        base, t_base = vals.clone(), tr[2].clone()

        def normalise():
            vals.copy_(base)
            tr[2].copy_(t_base)
            sk.coo_normalize((rows, cols, vals, offs), tr, a, b, n, m, 10, workspace=cn_ws)

        normalise()
        t_tr = timed(lambda: sk.plan_coo(Y, X, b, a, g, f, eps[-1], w["threshold"],
                                         workspace=coo_ws, out=(t_rows, t_cols, t_vals, t_offs)), 2)
        t_cn = timed(normalise, 2)
        line["phases_ms"]["transposed_plan"] = t_tr * 1e3
        line["phases_ms"]["coo_sinkhorn_normalisation_10_rounds"] = t_cn * 1e3
        # the cosine cost's own kernels: both clouds to unit length, dL/dY from the
        # transposed plan, and dL/dX, dL/dY back through the normalisation (the
        # potentials and plans of the normalised clouds are the kernels above)
        lg_ws = torch.empty(sk.workspace_bytes(sk.SK_OP_LOSS_GRAD, B, m, n, d, dt),
                            dtype=torch.uint8, device=dev)
        ly, dY = torch.empty(B, device=dev), torch.empty(B, m, d, device=dev)
        gX = torch.ones(B, n, d, device=dev)

        def cosine_kernels():
            Xh, nx = sk.normalize(X)
            Yh, ny = sk.normalize(Y)
            sk.loss_grad(Y, X, *tr, workspace=lg_ws, out=(ly, dY))
            return sk.normalize_backward(Xh, nx, gX), sk.normalize_backward(Yh, ny, dY)

        cosine_kernels()
        t_cos = timed(cosine_kernels, 2)
        line["phases_ms"]["cosine_normalise_dY_and_backward"] = t_cos * 1e3
    if not sparse:
        # dense gradient and barycentric projection of both clouds at the final eps
        # (one streamed pass per side); reported beside the step, not inside it
        dg_ws = torch.empty(sk.workspace_bytes(sk.SK_OP_DENSE_GRAD, B, n, m, d, dt),
                            dtype=torch.uint8, device=dev)
        dg_out = (torch.empty(B, n, d, device=dev), torch.empty(B, n, d, device=dev),
                  torch.empty(B, m, d, device=dev), torch.empty(B, m, d, device=dev))

        def dense_grad():
            sk.dense_grad(X, Y, a, b, f, g, eps[-1], workspace=dg_ws, out=dg_out)

        dense_grad()
        t_dg = timed(dense_grad, 2)
        assert all(bool(torch.isfinite(t).all()) for t in dg_out)
        line["phases_ms"]["dense_grad_and_projection_both_sides"] = t_dg * 1e3
        hv_bytes = sk.workspace_bytes(sk.SK_OP_HVP, B, n, m, d, dt)
        if hv_bytes > 0:
            # Hessian-vector product in X along the gradient direction, 20 CG steps
            # (fp64 plan passes for d <= 16, matrix-core passes for bf16 d = 32 / 64)
            hv_ws = torch.empty(hv_bytes, dtype=torch.uint8, device=dev)
            V, HV = dg_out[0].clone(), torch.empty_like(dg_out[0])

            def hvp():
                sk.hvp(X, Y, a, b, f, g, eps[-1], V, cg_iters=20, workspace=hv_ws, out=HV)

            hvp()
            t_hv = timed(hvp, 1)
            assert bool(torch.isfinite(HV).all())
            line["phases_ms"]["hvp_20_cg_steps"] = t_hv * 1e3
    if args.rates:
        rates = measure_rates(dev)
        line["measured_rates"] = rates
        if kernel in TILE_PROBE:
            cyc = rates[TILE_PROBE[kernel]]["simd_cycles_per_wave_iteration"]
            live = issue_floor_evals_per_s(kernel, cyc)
            line["roofline"]["issue_floor_live_probe"] = live / 1e12
            line["roofline"]["frac_of_issue_floor_live_probe"] = achieved / live
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
