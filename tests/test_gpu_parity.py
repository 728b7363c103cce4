"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Tolerances (the stated targets):
  potentials   ||f - f_ref||_inf / max(||f_ref||_inf, eps) <= 1e-4   (1e-2 bf16 MFMA config)
  scalars      |c - c_ref| / |c_ref| <= 1e-4 (cost, each loss)
  gradient     ||dX - dX_ref||_inf / ||dX_ref||_inf <= 1e-4
  sparse plan  identical support except entries whose value is within 1e-3
               (relative) of the threshold; values on the common support
               agree to 1e-4 relative.
Both sides always receive the same fp32 (or bf16) inputs; where one stage's
output is the next one's input (potentials -> plan -> loss), the oracle's own
values, rounded to fp32, are handed to the GPU, never the other way round.
"""
import os

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
sk = pytest.importorskip("sinkhorn_point_cloud_amd")

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.detach().cpu().double().numpy()


def rel_inf(got, ref, floor=0.0):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return np.abs(got - ref).max() / max(np.abs(ref).max(), floor)


def points(c):
    if c.get("dtype") == "bf16":
        return (dev(c["X_bits"].view(np.int16)).view(torch.bfloat16),
                dev(c["Y_bits"].view(np.int16)).view(torch.bfloat16))
    return dev(c["X"]), dev(c["Y"])


def run_gpu(c, eps, iters, **kw):
    X, Y = points(c)
    f, g, cost = sk.potentials(X, Y, dev(c["a"]), dev(c["b"]), eps=eps, iters=iters, **kw)
    torch.cuda.synchronize()
    return f, g, cost


def check_potentials(c, eps, iters, tol=1e-4, cost_tol=1e-4, **kw):
    eps32 = np.float32(eps)
    f, g, cost = run_gpu(c, eps, iters, **kw)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=eps32, iters=iters)
    e_last = float(eps32[-1])
    for p in range(c["X"].shape[0]):
        assert rel_inf(host(f)[p], fo[p], e_last) <= tol, f"f pair {p}"
        assert rel_inf(host(g)[p], go[p], e_last) <= tol, f"g pair {p}"
    st = oracle.plan_stats(c["X"], c["Y"], c["a"], c["b"], fo, go, e_last)
    np.testing.assert_allclose(host(cost), st["cost"], rtol=cost_tol, atol=0)
    return f, g, fo, go


# ------------------------------------------------------------ small, d = 3
SMALL = [  # (B, n, m, weights, zero weights, eps, iters)
    (1, 1, 1, "uniform", 0, [0.1], [3]),
    (1, 7, 5, "dirichlet", 0, [0.05], [20]),
    (1, 64, 64, "uniform", 0, [0.05], [10]),
    (2, 100, 37, "dirichlet", 0, [0.03], [25]),
    (3, 257, 300, "dirichlet", 2, [0.05], [15]),
    (1, 1000, 1, "uniform", 0, [0.2], [4]),
    (1, 1, 999, "dirichlet", 0, [0.2], [4]),
    (2, 129, 1030, "dirichlet", 0, [1.0, 0.3, 0.1, 0.03], [3, 3, 3, 10]),
    (1, 2000, 1500, "dirichlet", 0, [0.01], [30]),
    # few rows against long key ranges: the key range is split across work-groups
    (1, 100, 12000, "dirichlet", 0, [0.05, 0.02], [4, 6]),
    (2, 9000, 70, "uniform", 3, [0.03], [8]),
    # the first 3000 points of each cloud weigh nothing: whole key splits of the
    # f-update hold only masked keys
    (1, 3200, 12000, "dirichlet", 3000, [0.05], [5]),
]


@pytest.mark.parametrize("scores", ["mfma", "valu"])
@pytest.mark.parametrize("B,n,m,w,zw,eps,iters", SMALL)
def test_potentials_d3_match_oracle(B, n, m, w, zw, eps, iters, scores):
    c = workloads.random_case(100 + n + m, B, n, m, 3, weights=w, zero_weights=zw)
    check_potentials(c, eps, iters, valu_scores=scores == "valu")


@pytest.mark.parametrize("scores", ["mfma", "valu"])
@pytest.mark.parametrize("B,n,m,eps,iters", [(2, 300, 257, [0.05], [15]),
                                             (1, 100, 12000, [0.05, 0.02], [4, 6]),
                                             (256, 200, 150, [0.2, 0.03], [3, 8])])
def test_bf16_point_clouds_match_oracle(scores, B, n, m, eps, iters):
    # bf16 coordinates on the 3-D path: one launch per half-iteration, split key
    # ranges, and per-pair stage launches (the oracle takes the same bf16 values)
    c = workloads.random_case(600 + n, B, n, m, 3, weights="dirichlet", dtype="bf16")
    check_potentials(c, eps, iters, valu_scores=scores == "valu")


@pytest.mark.parametrize("scores", ["mfma", "valu"])
def test_far_from_origin_and_huge_score_range(scores):
    # clouds far from the origin at small eps: scores span thousands of log2
    # units, so the first pass's shifts are far off and every block takes the
    # exact-shift pass (the vector path raises its running maximum many times,
    # and the first keys it sees are far below the row maximum)
    c = workloads.random_case(77, 2, 300, 333, 3, weights="dirichlet", spread=4.0)
    c = dict(c, X=c["X"] + np.float32(10.0), Y=c["Y"] + np.float32(10.0))
    check_potentials(c, [0.003], [5], valu_scores=scores == "valu")


@pytest.mark.parametrize("B,n,m,eps,iters", [
    # a short side against a long key range split across work-groups: on the
    # first pass every merged row of the f-update is out of range, and the
    # repair launch recomputes its blocks with exact shifts
    (1, 300, 20000, [0.003], [5]),
    # a mid-size pair, both updates split, under a schedule whose eps jumps
    # leave the shifts of some blocks stale
    (1, 12000, 11000, [1.0, 0.1, 0.01, 0.003], [2, 2, 2, 3]),
])
def test_split_key_ranges_with_stale_shifts(B, n, m, eps, iters):
    c = workloads.random_case(91 + n, B, n, m, 3, weights="dirichlet", spread=4.0)
    c = dict(c, X=c["X"] + np.float32(10.0), Y=c["Y"] + np.float32(10.0))
    check_potentials(c, eps, iters)


def test_split_keys_with_xcd_placement_and_repair():
    # 4 pairs of 128 rows against 20000 keys: 2 row blocks x 78 key splits x 4 pairs =
    # 624 work-groups (a multiple of 8, so batches are placed XCD by XCD), far from
    # the origin at a small eps, so merged rows go stale and the repair launch
    # (8 work-groups, also placed by XCD) recomputes them; twice, bit for bit
    c = workloads.random_case(83, 4, 128, 20000, 3, weights="dirichlet", spread=4.0)
    c = dict(c, X=c["X"] + np.float32(10.0), Y=c["Y"] + np.float32(10.0))
    f1, g1, _, _ = check_potentials(c, [0.003], [3])
    f2, g2, _ = run_gpu(c, [0.003], [3])
    assert torch.equal(f1, f2) and torch.equal(g1, g2)


@pytest.mark.parametrize("n,m", [(1 << 24, 64), (64, 1 << 24)])
def test_largest_cloud_per_pair(n, m):
    # 2^24 points on one side (the largest the boundary accepts) against 64 on the
    # other: the long side's half-update splits its key range across work-groups
    c = workloads.random_case(501, 1, n, m, 3, weights="dirichlet")
    check_potentials(c, [0.1], [1])


def test_feature_matrix_cores_at_a_million_points():
    # 2^20 bf16 points of d = 64 against 300: the row pass's d-vector partials
    # hold 2^26 floats, the Y side's keys are split 64 ways; the dense gradient
    # on sampled rows of both sides against the oracle, and the HVP's symmetry
    n, m, d, eps = 1 << 20, 300, 64, 0.5
    c = workloads.random_case(503, 1, n, m, d, weights="uniform", dtype="bf16")
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    f, g, _ = sk.potentials(X, Y, a, b, eps=[eps], iters=[20])
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    sel_x = np.sort(rng.choice(n, 64, replace=False))
    sel_y = np.sort(rng.choice(m, 16, replace=False))
    check_dense_grad(c, eps, host(f), host(g), sel_x, sel_y, tol=1e-4)
    U = dev((rng.normal(size=(1, n, d)) / 8).astype(np.float32))
    V = dev((rng.normal(size=(1, n, d)) / 8).astype(np.float32))
    HU, ru = sk.hvp(X, Y, a, b, f, g, eps, U, cg_iters=60)
    HV, rv = sk.hvp(X, Y, a, b, f, g, eps, V, cg_iters=60)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(HU).all()) and bool(torch.isfinite(HV).all())
    assert float(ru[0]) < 1e-4 and float(rv[0]) < 1e-4
    uhv = float((U.double() * HV.double()).sum())
    vhu = float((V.double() * HU.double()).sum())
    assert abs(uhv - vhu) <= 1e-4 * float((U.double() * HV.double()).abs().sum())


def test_most_pairs_per_call():
    # 65535 pairs (the largest batch the boundary accepts) of small clouds: every
    # per-pair grid dimension at its limit, potentials, plan and fused loss
    B, n, m = 65535, 5, 3
    c = workloads.random_case(502, B, n, m, 3, weights="dirichlet")
    eps = 0.05
    _, _, fo, go = check_potentials(c, [eps], [3])
    # plan and loss on both sides from the oracle's potentials rounded to fp32
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    X, Y = points(c)
    loss = torch.empty(B, device=X.device)
    dX = torch.empty(B, n, 3, device=X.device)
    rows, cols, vals, offs = sk.plan_coo(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32), eps,
                                         1e-8, loss_out=(loss, dX))
    ro, co, vo, oo = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], f32, g32,
                                     float(np.float32(eps)), 1e-8)
    lo, dXo = oracle.loss_grad(c["X"], c["Y"], ro, co, vo.astype(np.float32), oo)
    # the support of every pair, not only the total count
    got = tuple(t.cpu().numpy() for t in (rows, cols, vals, offs))
    compare_coo_all_pairs(got, (ro, co, vo, oo), n, m)
    np.testing.assert_allclose(host(loss), lo, rtol=1e-4)
    assert rel_inf(host(dX), dXo) <= 1e-4


def test_coincident_clouds_closed_form():
    # every x_i = p and every y_j = q: C_ij = |p - q|^2 = c for all (i, j), so from
    # g = 0 the first f-update gives f = c, the g-update gives g = 0, and the plan
    # is a (x) b: cost c, every entry kept, loss c, dX_i = 2 a_i (p - q)
    n, m = 300, 200
    p = np.float32([0.3, -0.2, 0.5])
    q = np.float32([-0.1, 0.4, 0.2])
    X = np.broadcast_to(p, (1, n, 3)).copy()
    Y = np.broadcast_to(q, (1, m, 3)).copy()
    c = float(((p.astype(np.float64) - q.astype(np.float64)) ** 2).sum())
    a = np.full((1, n), 1.0 / n, dtype=np.float32)
    b = np.full((1, m), 1.0 / m, dtype=np.float32)
    eps = 0.05
    for valu in (False, True):
        f, g, cost = sk.potentials(dev(X), dev(Y), dev(a), dev(b), eps=[eps], iters=[5],
                                   valu_scores=valu)
        assert np.abs(host(f) - c).max() <= 1e-4 * max(c, eps)
        assert np.abs(host(g)).max() <= 1e-4 * max(c, eps)
        assert abs(host(cost)[0] - c) <= 1e-4 * c
    loss = torch.empty(1, device=f.device)
    dX = torch.empty(1, n, 3, device=f.device)
    rows, cols, vals, offs = sk.plan_coo(dev(X), dev(Y), dev(a), dev(b), f, g, eps, 1e-8,
                                         loss_out=(loss, dX))
    assert int(offs[-1]) == n * m
    np.testing.assert_allclose(host(vals), 1.0 / (n * m), rtol=1e-4)
    assert abs(host(loss)[0] - c) <= 1e-4 * c
    ref = 2.0 * (p.astype(np.float64) - q.astype(np.float64)) / n
    np.testing.assert_allclose(host(dX)[0], np.broadcast_to(ref, (n, 3)), rtol=1e-4)


@pytest.mark.parametrize("scores", ["mfma", "valu"])
@pytest.mark.parametrize("B,n,m", [(260, 300, 200), (256, 1100, 70)])
def test_batch_of_many_pairs(scores, B, n, m):
    # at least as many pairs as compute units: the matrix-core path runs each
    # stage per pair in one launch (several 64-row blocks per side, more blocks
    # than waves on one side, ragged sizes, zero weights, two stages); the
    # vector path is the usual one
    c = workloads.random_case(503 + n, B, n, m, 3, weights="dirichlet", zero_weights=2)
    check_potentials(c, [0.2, 0.03], [4, 12], valu_scores=scores == "valu")


def test_batch_of_many_pairs_from_a_stale_start():
    # warm start from potentials far from the solution: every row block of the
    # per-pair launch finds its shifts stale on the first pass and makes them
    # exact (a warm start never skips the first shifted pass)
    c = workloads.random_case(504, 256, 130, 140, 3, weights="uniform")
    X, Y = points(c)
    eps = 0.02
    f0 = np.full((256, 130), 40.0, dtype=np.float32)
    g0 = np.full((256, 140), -35.0, dtype=np.float32)
    f, g, _ = sk.potentials(X, Y, dev(c["a"]), dev(c["b"]), eps=[eps], iters=[6],
                            f0=dev(f0), g0=dev(g0))
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([eps]), iters=[6],
                               f0=f0.astype(np.float64), g0=g0.astype(np.float64))
    for p in (0, 77, 255):
        assert rel_inf(host(f)[p], fo[p], eps) <= 1e-4
        assert rel_inf(host(g)[p], go[p], eps) <= 1e-4


# A small batch of clouds of at most 1024 points (padded) whose work-groups fit
# on half of the compute units runs each stage in one launch: work-group (pair,
# part) owns 16 rows of each side and the work-groups hand their new biases to
# one another between half-iterations through bounded waits.
SPLIT = [  # (B, n, m, weights, zero weights, eps, iters)
    # one pair of 1024 points (64 work-groups), eps falling between stages
    (1, 1024, 1024, "uniform", 0, [0.5, 0.05, 0.01], [3, 5, 8]),
    # a stage of one iteration (its first f-update is the cold start's exact
    # pass and its g-update the stage's last), ragged sides, zero weights
    (2, 1000, 700, "dirichlet", 3, [0.1, 0.02], [1, 6]),
    # most work-groups own no row of the short side
    (2, 17, 650, "dirichlet", 0, [0.2, 0.03], [4, 6]),
    (1, 1024, 16, "dirichlet", 0, [0.05], [7]),
    # 32 small pairs of 4 work-groups each (the batch at the half-chip limit)
    (32, 50, 60, "dirichlet", 0, [0.2, 0.05], [3, 5]),
    # one point on one side: 60 of the 64 work-groups own no row of it
    (2, 1, 1000, "uniform", 0, [0.1], [6]),
]


@pytest.mark.parametrize("B,n,m,w,zw,eps,iters", SPLIT)
def test_split_stage_launch_matches_oracle(B, n, m, w, zw, eps, iters):
    c = workloads.random_case(700 + n + m, B, n, m, 3, weights=w, zero_weights=zw)
    check_potentials(c, eps, iters)


def test_split_stage_launch_from_a_stale_start_and_far_from_the_origin():
    # warm start from potentials far off, clouds far from the origin at small
    # eps: every work-group finds its shifts stale on the first pass
    c = workloads.random_case(708, 1, 900, 1000, 3, weights="dirichlet", spread=4.0)
    c = dict(c, X=c["X"] + np.float32(10.0), Y=c["Y"] + np.float32(10.0))
    f0 = np.full((1, 900), 30.0, dtype=np.float32)
    g0 = np.full((1, 1000), -25.0, dtype=np.float32)
    eps = [0.01, 0.003]
    f, g, _ = run_gpu(c, eps, [2, 3], f0=dev(f0), g0=dev(g0))
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32(eps), iters=[2, 3],
                               f0=f0.astype(np.float64), g0=g0.astype(np.float64))
    assert rel_inf(host(f), fo, eps[-1]) <= 1e-4
    assert rel_inf(host(g), go, eps[-1]) <= 1e-4


def test_split_stage_launch_is_deterministic():
    c = workloads.random_case(709, 2, 1000, 1024, 3, weights="dirichlet")
    r1 = run_gpu(c, [0.3, 0.02], [3, 8])
    r2 = run_gpu(c, [0.3, 0.02], [3, 8])
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


def test_launch_shape_query_names_the_launch_each_workload_takes():
    # the probe that bench.py asks which kernel it times: on this device the
    # five workloads' d = 3 shapes and the vector-score flag
    import ctypes
    lib = sk.load_library()
    f = lib.sinkhorn_probe_potentials_path
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_uint]
    f.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert f(1, 1024, 1024, 3, sk.SK_F32, 0) == (2 if 2 * 64 <= cus else 0)       # pair-1k
    assert f(32, 2048, 2048, 3, sk.SK_F32, 0) == 0                                # sphere-2k
    assert f(256, 1024, 1024, 3, sk.SK_F32, 0) == (1 if 256 >= cus else 0)        # blobs-1k
    assert f(1, 65536, 65536, 3, sk.SK_F32, 0) == 0                               # gmm-64k
    assert f(1, 50000, 60000, 64, sk.SK_BF16, 0) == 4                             # feat-50k
    assert f(1, 1024, 1024, 3, sk.SK_F32, sk.SK_VALU_SCORES) == 3


def test_split_stage_launches_on_two_streams_at_once():
    # two small batches on two streams at the same time: each split stage
    # launch takes at most half of the compute units (64 and 120 work-groups
    # here), so both fit on the chip together and neither's waits run out; each
    # result equals its run alone bit for bit
    sched = dict(eps=[0.1, 0.02], iters=[5, 20])
    cases = [workloads.random_case(730, 1, 1024, 1000, 3, weights="dirichlet"),
             workloads.random_case(731, 2, 700, 900, 3, weights="dirichlet")]
    args = []
    for c in cases:
        X, Y = points(c)
        args.append((X, Y, dev(c["a"]), dev(c["b"])))
    refs = [sk.potentials(*a, **sched) for a in args]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for a, st in zip(args, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(sk.potentials(*a, **sched))
    torch.cuda.synchronize()
    for out, ref in zip(outs, refs):
        for u, v in zip(out, ref):
            assert torch.isfinite(u).all()
            assert torch.equal(u, v)


def test_split_stage_launch_wait_that_runs_out_gives_nan():
    # the hand-over waits are bounded: with the limit set so that every wait
    # fails at once (the host-side test hook), the launch still ends and the
    # potentials come back NaN; with the default limit the same call is exact
    import ctypes
    lib = sk.load_library()
    lib.sinkhorn_probe_wait_limit.argtypes = [ctypes.c_longlong]
    lib.sinkhorn_probe_wait_limit.restype = ctypes.c_longlong
    c = workloads.random_case(710, 1, 1024, 1000, 3, weights="dirichlet")
    prev = lib.sinkhorn_probe_wait_limit(-1)
    try:
        f, g, _ = run_gpu(c, [0.05], [4])
    finally:
        assert lib.sinkhorn_probe_wait_limit(prev) == -1
    assert torch.isnan(f).all() and torch.isnan(g).all()
    check_potentials(c, [0.05], [4])


def test_schedule_with_empty_stages_and_zero_iterations():
    c = workloads.random_case(5, 1, 90, 70, 3, weights="dirichlet")
    check_potentials(c, [0.5, 0.2, 0.05], [0, 6, 8])
    f, g, cost = run_gpu(c, [0.05], [0])
    assert torch.all(f == 0) and torch.all(g == 0)


@pytest.mark.parametrize("B,n,m", [(256, 130, 140), (1, 300, 20000), (1, 800, 1000)])
def test_empty_stages_on_per_pair_and_split_launches(B, n, m):
    # empty stages before, between and after others: the cold start's exact
    # shifts belong to the first stage that runs, and each stage hands the next
    # running stage's eps to its last g-update (per-pair stage launches; split
    # key ranges with merge marks and repair; split stage launches)
    c = workloads.random_case(506 + B, B, n, m, 3, weights="dirichlet", spread=2.0)
    check_potentials(c, [1.0, 0.1, 0.05, 0.03, 0.02], [0, 3, 0, 4, 0])


def test_translated_clouds_give_the_same_potentials():
    # the cost is translation invariant; the GPU's attention form must stay accurate
    c = workloads.random_case(8, 1, 300, 200, 3, weights="dirichlet")
    check_potentials(c, [0.05], [20])
    shifted = dict(c, X=(c["X"] + np.float32(3.0)), Y=(c["Y"] + np.float32(3.0)))
    check_potentials(shifted, [0.05], [20])


# ---------------------------------------------------------- feature path
@pytest.mark.parametrize("dtype,d,n,m", [("f32", 8, 130, 77), ("f32", 64, 300, 257),
                                          ("bf16", 64, 200, 333), ("bf16", 3, 65, 64),
                                          ("f32", 128, 64, 100), ("bf16", 32, 1, 500)])
def test_feature_potentials_match_oracle(dtype, d, n, m):
    c = workloads.random_case(9 + d, 2, n, m, d, weights="dirichlet", dtype=dtype,
                              spread=0.25)
    check_potentials(c, [0.5, 0.1], [5, 10])


@pytest.mark.parametrize("d,n,m", [(64, 8192, 1000), (32, 4100, 3000), (128, 8200, 700)])
def test_feature_matrix_core_path_matches_oracle(d, n, m):
    # bf16 with whole 32-dim blocks and >= 128 row blocks: the MFMA kernel
    c = workloads.random_case(30 + d, 2, n, m, d, weights="dirichlet", dtype="bf16",
                              spread=0.25)
    check_potentials(c, [0.5, 0.05], [3, 4])


def test_feature_matrix_core_fallback_on_stale_shift():
    # warm start from potentials far off: every row block must take the fallback
    c = workloads.random_case(35, 1, 8192, 900, 64, weights="uniform", dtype="bf16",
                              spread=0.25)
    f0 = np.full((1, 8192), 500.0, dtype=np.float32)
    g0 = np.full((1, 900), -500.0, dtype=np.float32)
    f, g, _ = run_gpu(c, [0.05], [2], f0=f0, g0=g0)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([0.05]),
                               iters=[2], f0=f0.astype(np.float64), g0=g0.astype(np.float64))
    assert rel_inf(host(f), fo, 0.05) <= 1e-4
    assert rel_inf(host(g), go, 0.05) <= 1e-4


# ---------------------------------------------------- warm start, determinism
def test_warm_start_split_matches_single_run():
    c = workloads.random_case(12, 2, 500, 400, 3, weights="dirichlet")
    f1, g1, _ = run_gpu(c, [0.1, 0.03], [10, 10])
    fa, ga, _ = run_gpu(c, [0.1], [10])
    f2, g2, _ = run_gpu(c, [0.03], [10], f0=fa, g0=ga)
    assert rel_inf(host(f2), host(f1), 0.03) < 1e-5
    assert rel_inf(host(g2), host(g1), 0.03) < 1e-5


def test_per_pair_launch_is_deterministic():
    c = workloads.random_case(66, 256, 200, 150, 3, weights="dirichlet")
    r1 = run_gpu(c, [0.3, 0.02], [3, 8])
    r2 = run_gpu(c, [0.3, 0.02], [3, 8])
    for u, v in zip(r1, r2):
        assert torch.equal(u, v)


@pytest.mark.parametrize("scores", ["mfma", "valu"])
def test_potentials_are_deterministic(scores):
    c = workloads.random_case(13, 3, 700, 650, 3, weights="dirichlet")
    r1 = run_gpu(c, [0.02], [10], valu_scores=scores == "valu")
    r2 = run_gpu(c, [0.02], [10], valu_scores=scores == "valu")
    for a_, b_ in zip(r1, r2):
        assert torch.equal(a_, b_)


def test_matrix_and_vector_score_paths_agree():
    c = workloads.random_case(14, 2, 1000, 900, 3, weights="dirichlet")
    f1, g1, c1 = run_gpu(c, [0.1, 0.02], [10, 10])
    f2, g2, c2 = run_gpu(c, [0.1, 0.02], [10, 10], valu_scores=True)
    assert rel_inf(host(f1), host(f2), 0.02) < 2e-5
    assert rel_inf(host(g1), host(g2), 0.02) < 2e-5


# ------------------------------------------------------------ sparse plan
def compare_coo(got, ref, m, thr_val, band=1e-3, val_tol=1e-4):
    """got/ref: (rows, cols, vals) of one pair.  Support equal except entries
    within `band` (relative) of the threshold value; values agree on the rest."""
    gk = got[0].astype(np.int64) * m + got[1]
    rk = ref[0].astype(np.int64) * m + ref[1]
    only_g = ~np.isin(gk, rk)
    only_r = ~np.isin(rk, gk)
    for v in np.concatenate([got[2][only_g], ref[2][only_r]]):
        assert abs(v / thr_val - 1.0) <= band, f"value {v} vs threshold {thr_val}"
    common, ig, ir = np.intersect1d(gk, rk, assume_unique=True, return_indices=True)
    gv, rv = got[2][ig].astype(np.float64), ref[2][ir]
    assert np.all(np.abs(gv - rv) <= val_tol * rv)
    return len(common)


def compare_coo_all_pairs(got, ref, n, m, thr=1e-8, band=1e-3, val_tol=1e-4):
    """got/ref: (rows, cols, vals, pair_offsets) of a whole batch.  Per pair, the
    supports are equal except entries within `band` (relative) of that pair's
    threshold value, and every pair's entries are in strictly increasing
    (row, column) order; values agree on the common support."""
    def keys(rows, cols, offs):
        pair = np.repeat(np.arange(len(offs) - 1, dtype=np.int64), np.diff(offs))
        return pair, (pair * n + rows.astype(np.int64)) * m + cols
    gp, gk = keys(*got[:2], got[3])
    rp, rk = keys(*ref[:2], ref[3])
    assert np.all(np.diff(gk) > 0), "entries out of (pair, row, column) order"
    B = len(ref[3]) - 1
    vmax = np.zeros(B)
    nonempty = np.diff(ref[3]) > 0
    vmax[nonempty] = np.maximum.reduceat(ref[2], ref[3][:-1][nonempty])
    thr_val = thr * vmax
    only_g = ~np.isin(gk, rk)
    only_r = ~np.isin(rk, gk)
    for v, pp in ((got[2][only_g], gp[only_g]), (ref[2][only_r], rp[only_r])):
        assert np.all(np.abs(v / thr_val[pp] - 1.0) <= band), "support differs off the threshold"
    common, ig, ir = np.intersect1d(gk, rk, assume_unique=True, return_indices=True)
    gv, rv = got[2][ig].astype(np.float64), ref[2][ir].astype(np.float64)
    assert np.all(np.abs(gv - rv) <= val_tol * rv)
    return len(common), int(only_g.sum()), int(only_r.sum())


def check_coo_given_potentials(c, eps, fo, go, pairs=None, thr=1e-8):
    """Both sides get the oracle's potentials rounded to fp32."""
    B = c["X"].shape[0]
    pairs = range(B) if pairs is None else pairs
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    X, Y = points(c)
    rows, cols, vals, offs = sk.plan_coo(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32),
                                         eps, thr)
    rows, cols, vals, offs = (t.cpu().numpy() for t in (rows, cols, vals, offs))
    assert offs[0] == 0 and np.all(np.diff(offs) >= 0) and offs[-1] == len(rows)
    for p in pairs:
        s = slice(offs[p], offs[p + 1])
        # row-major order, no duplicates
        key = rows[s].astype(np.int64) * c["Y"].shape[1] + cols[s]
        assert np.all(np.diff(key) > 0)
        ro, co, vo, oo = oracle.plan_coo(c["X"][p], c["Y"][p], c["a"][p], c["b"][p], f32[p],
                                         g32[p], float(np.float32(eps)), thr)
        thr_val = thr * np.max(vo)
        compare_coo((rows[s], cols[s], vals[s]), (ro, co, vo), c["Y"].shape[1], thr_val)
    return rows, cols, vals, offs


@pytest.mark.parametrize("B,n,m,eps,thr", [(1, 33, 47, 0.02, 1e-8), (2, 300, 257, 0.01, 1e-8),
                                           (3, 129, 64, 0.05, 1e-3), (1, 500, 700, 0.02, 1.0)])
def test_coo_matches_oracle(B, n, m, eps, thr):
    c = workloads.random_case(21 + n, B, n, m, 3, weights="dirichlet")
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([eps]),
                               iters=[15])
    check_coo_given_potentials(c, eps, fo, go, thr=thr)


def test_coo_capacity_protocol():
    c = workloads.random_case(31, 2, 200, 150, 3, weights="dirichlet")
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([0.05]),
                               iters=[10])
    X, Y = points(c)
    args = (X, Y, dev(c["a"]), dev(c["b"]), dev(fo.astype(np.float32)),
            dev(go.astype(np.float32)), 0.05, 1e-8)
    with pytest.raises(sk.SinkhornError) as ei:
        sk.plan_coo(*args, capacity=3)
    assert ei.value.status == sk.SK_ERR_CAPACITY
    rows, cols, vals, offs = sk.plan_coo(*args)
    rows2, cols2, vals2, offs2 = sk.plan_coo(*args, capacity=rows.numel() + 5)
    assert torch.equal(rows, rows2) and torch.equal(cols, cols2) and torch.equal(vals, vals2)
    assert torch.equal(offs, offs2)


# ------------------------------------------------------------ loss / grad
def check_loss_grad_given_coo(c, rows, cols, vals, offs, tol=1e-5, pairs=None):
    X, Y = points(c)
    loss, dX = sk.loss_grad(X, Y, dev(rows.astype(np.int32)), dev(cols.astype(np.int32)),
                            dev(vals.astype(np.float32)), dev(offs.astype(np.int64)))
    lo, dXo = oracle.loss_grad(c["X"], c["Y"], rows, cols, vals.astype(np.float32), offs)
    pairs = range(c["X"].shape[0]) if pairs is None else pairs
    for p in pairs:
        assert abs(host(loss)[p] - lo[p]) <= tol * abs(lo[p]) + 1e-30
        assert rel_inf(host(dX)[p], dXo[p], 1e-30) <= tol
    return loss, dX


@pytest.mark.parametrize("B,n,m,d,dtype", [(2, 100, 80, 3, "f32"), (1, 257, 300, 3, "f32"),
                                           (2, 70, 90, 64, "bf16"), (1, 40, 50, 8, "f32")])
def test_loss_grad_matches_oracle(B, n, m, d, dtype):
    c = workloads.random_case(41 + n, B, n, m, d, weights="dirichlet", dtype=dtype,
                              spread=1.0 if d <= 8 else 0.25)
    eps = 0.05
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([eps]),
                               iters=[10])
    rows, cols, vals, offs = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], fo, go,
                                             float(np.float32(eps)), 1e-6)
    check_loss_grad_given_coo(c, rows, cols, vals, offs)


def test_loss_grad_rows_without_entries_and_empty_pairs():
    c = workloads.random_case(43, 3, 50, 40, 3, weights="dirichlet")
    rows = np.array([0, 0, 7, 49, 3, 3, 3], dtype=np.int32)
    cols = np.array([1, 39, 0, 5, 2, 8, 9], dtype=np.int32)
    vals = np.array([0.1, 0.2, 0.3, 0.05, 0.5, 0.25, 0.125], dtype=np.float32)
    offs = np.array([0, 4, 4, 7], dtype=np.int64)     # pair 1 has no entries
    loss, dX = check_loss_grad_given_coo(c, rows, cols, vals, offs)
    assert host(loss)[1] == 0.0 and np.all(host(dX)[1] == 0.0)
    assert np.all(host(dX)[0, 1:7] == 0.0)


def fused_plan_loss(X, Y, a, b, f, g, eps, thr):
    """plan_coo with the loss and dL/dX accumulated during the emission, checked
    against loss_grad on the emitted plan (same per-entry arithmetic, another
    summation order: agreement to a few fp32 roundings)."""
    B, n, d = X.shape
    loss = torch.full((B,), 7.0, device=X.device)
    dX = torch.full((B, n, d), 7.0, device=X.device)
    plan = sk.plan_coo(X, Y, a, b, f, g, eps, thr, loss_out=(loss, dX))
    l2, dX2 = sk.loss_grad(X, Y, *plan)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(loss), host(l2), rtol=1e-5, atol=1e-30)
    for p in range(B):
        assert rel_inf(host(dX)[p], host(dX2)[p], 1e-30) <= 1e-5
    return plan, loss, dX


def test_plan_chain_on_gpu_potentials():
    # GPU potentials -> GPU plan -> GPU loss against the oracle's own chain
    c = workloads.random_case(44, 2, 400, 350, 3, weights="dirichlet")
    eps = [0.02]
    f, g, _ = run_gpu(c, eps, [20])
    X, Y = points(c)
    rows, cols, vals, offs = sk.plan_coo(X, Y, dev(c["a"]), dev(c["b"]), f, g, eps[0], 1e-8)
    loss, dX = sk.loss_grad(X, Y, rows, cols, vals, offs)
    _, loss_f, dX_f = fused_plan_loss(X, Y, dev(c["a"]), dev(c["b"]), f, g, eps[0], 1e-8)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32(eps), iters=[20])
    ro, co, vo, oo = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], fo, go,
                                     float(np.float32(eps[0])), 1e-8)
    lo, dXo = oracle.loss_grad(c["X"], c["Y"], ro, co, vo, oo)
    for l_gpu, dX_gpu in ((loss, dX), (loss_f, dX_f)):
        np.testing.assert_allclose(host(l_gpu), lo, rtol=1e-4)
        for p in range(2):
            assert rel_inf(host(dX_gpu)[p], dXo[p]) <= 1e-4


@pytest.mark.parametrize("B,n,m,d,dtype,thr", [(2, 150, 1300, 3, "f32", 1e-8),
                                               (1, 97, 80, 4, "bf16", 1e-3),
                                               (2, 70, 90, 8, "f32", 1e-6),
                                               (1, 60, 75, 64, "bf16", 1e-4),
                                               (2, 50, 40, 3, "f32", 1.0)])
def test_fused_loss_matches_oracle(B, n, m, d, dtype, thr):
    # m = 1300 spans two LDS chunks of the staged emission; d = 8 and 64 take the
    # unstaged one; thr = 1 keeps only each pair's largest entry, so nearly every
    # row has no entry and must get a zero gradient
    c = workloads.random_case(47 + d, B, n, m, d, weights="dirichlet", dtype=dtype,
                              spread=1.0 if d <= 8 else 0.25)
    eps = 0.05
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([eps]),
                               iters=[10])
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    X, Y = points(c)
    (rows, cols, vals, offs), loss, dX = fused_plan_loss(X, Y, dev(c["a"]), dev(c["b"]),
                                                         dev(f32), dev(g32), eps, thr)
    # the oracle's chain from the same fp32 potentials (entries within the
    # threshold band that one side keeps and the other drops weigh ~1e-8 of the max)
    ro, co, vo, oo = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], f32, g32,
                                     float(np.float32(eps)), thr)
    lo, dXo = oracle.loss_grad(c["X"], c["Y"], ro, co, vo.astype(np.float32), oo)
    np.testing.assert_allclose(host(loss), lo, rtol=1e-4)
    for p in range(B):
        assert rel_inf(host(dX)[p], dXo[p], 1e-30) <= 1e-4
    if thr == 1.0:
        for p in range(B):
            empty = np.setdiff1d(np.arange(n), ro[oo[p]:oo[p + 1]])
            assert len(empty) >= n - 2 and np.all(host(dX)[p][empty] == 0.0)


def test_fused_loss_untouched_when_the_plan_does_not_fit():
    c = workloads.random_case(48, 1, 64, 60, 3)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=np.float32([0.05]),
                               iters=[5])
    X, Y = points(c)
    loss = torch.full((1,), 7.0, device=X.device)
    dX = torch.full((1, 64, 3), 7.0, device=X.device)
    with pytest.raises(sk.SinkhornError) as ei:
        sk.plan_coo(X, Y, None, None, dev(fo.astype(np.float32)), dev(go.astype(np.float32)),
                    0.05, 1e-8, capacity=3, loss_out=(loss, dX))
    assert ei.value.status == sk.SK_ERR_CAPACITY
    assert bool((loss == 7.0).all()) and bool((dX == 7.0).all())


# ------------------------------------------------------------ workloads
def golden(name):
    path = os.path.join(GOLDEN, f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"no stored oracle values for {name}")
    z = np.load(path)
    return {k: z[k] for k in z.files}


def load_workload(name):
    w = workloads.make(name)
    gold = golden(name)
    s = sum(np.asarray(w[k], dtype=np.float64).sum() for k in ("X", "Y", "a", "b"))
    assert s == gold["input_sum"], "input generator drifted from the stored oracle run"
    return w, gold


def check_workload_potentials(name, tol):
    w, gold = load_workload(name)
    f, g, cost = run_gpu(w, list(w["eps"]), list(w["iters"]))
    e_last = float(w["eps"][-1])
    for p in range(w["X"].shape[0]):
        assert rel_inf(host(f)[p], gold["f"][p], e_last) <= tol, f"f pair {p}"
        assert rel_inf(host(g)[p], gold["g"][p], e_last) <= tol, f"g pair {p}"
    np.testing.assert_allclose(host(cost), gold["cost"], rtol=tol)
    return w, gold, f, g


def test_workload_pair_1k():
    check_workload_potentials("pair-1k", 1e-4)


@pytest.mark.parametrize("name,pairs", [("sphere-2k", list(range(32))),
                                        ("blobs-1k", list(range(256)))])
def test_workload_sparse_plan_and_loss(name, pairs):
    w, gold, f, g = check_workload_potentials(name, 1e-4)
    eps = float(w["eps"][-1])
    # plan: both sides from the oracle's potentials (rounded to fp32): support,
    # order and values on every pair
    f32, g32 = gold["f"].astype(np.float32), gold["g"].astype(np.float32)
    rows, cols, vals, offs = check_coo_given_potentials(
        w, eps, f32.astype(np.float64), g32.astype(np.float64), pairs=pairs)
    # loss and dL/dX of the same pairs: the GPU on its plan, the oracle on its own
    X, Y = points(w)
    loss, dX = sk.loss_grad(X, Y, dev(rows), dev(cols), dev(vals), dev(offs))
    loss, dX = host(loss), host(dX)
    for p in pairs:
        ro, co, vo, oo = oracle.plan_coo(w["X"][p], w["Y"][p], w["a"][p], w["b"][p], f32[p],
                                         g32[p], float(np.float32(eps)), w["threshold"])
        lo, dXo = oracle.loss_grad(w["X"][p], w["Y"][p], ro, co, vo.astype(np.float32), oo)
        assert abs(loss[p] - lo[0]) <= 1e-4 * abs(lo[0]), f"loss pair {p}"
        assert rel_inf(dX[p], dXo[0]) <= 1e-4, f"dX pair {p}"
    # full GPU chain against the oracle's chain, every pair
    X, Y = points(w)
    rows, cols, vals, offs = sk.plan_coo(X, Y, dev(w["a"]), dev(w["b"]), f, g, eps,
                                         w["threshold"])
    loss, dX = sk.loss_grad(X, Y, rows, cols, vals, offs)
    _, loss_f, dX_f = fused_plan_loss(X, Y, dev(w["a"]), dev(w["b"]), f, g, eps, w["threshold"])
    for l_gpu, dX_gpu in ((loss, dX), (loss_f, dX_f)):
        np.testing.assert_allclose(host(l_gpu), gold["loss"], rtol=1e-4)
        for k, p in enumerate(gold["dX_pairs"]):
            assert rel_inf(host(dX_gpu)[p], gold["dX"][k]) <= 1e-4


def test_workload_gmm_64k():
    check_workload_potentials("gmm-64k", 1e-4)


def test_workload_feat_50k():
    check_workload_potentials("feat-50k", 1e-2)


# ------------------------------------------------ dense gradient and projection
def check_dense_grad(c, eps, fo, go, sel_x=None, sel_y=None, tol=1e-4):
    """GPU dense_grad against the oracle, both from the same fp32 potentials."""
    f32 = np.asarray(fo, dtype=np.float32)
    g32 = np.asarray(go, dtype=np.float32)
    X, Y = points(c)
    dX, TX, dY, TY = sk.dense_grad(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32), eps)
    torch.cuda.synchronize()
    B, n, d = c["X"].shape
    m = c["Y"].shape[1]
    for side, P, Q, wp, wq, fp, gq, k, sel, dG, T in (
            ("x", c["X"], c["Y"], c["a"], c["b"], f32, g32, n, sel_x, dX, TX),
            ("y", c["Y"], c["X"], c["b"], c["a"], g32, f32, m, sel_y, dY, TY)):
        r_o, dG_o, T_o = oracle.dense_grad(P, Q, wp, wq, fp.astype(np.float64),
                                           gq.astype(np.float64), eps, sel=sel)
        got_dG = host(dG).reshape(B * k, d)
        got_T = host(T).reshape(B * k, d)
        if sel is None:
            dG_o, T_o = dG_o.reshape(B * k, d), T_o.reshape(B * k, d)
        else:
            got_dG, got_T = got_dG[sel], got_T[sel]
        assert rel_inf(got_dG, dG_o) <= tol, f"gradient, {side} side"
        # the projection is a point: compare against the cloud's extent
        ext = max(np.abs(P).max(), np.abs(Q).max())
        assert np.abs(got_T - T_o).max() / ext <= tol, f"projection, {side} side"
    return dX, TX, dY, TY


# The bf16 matrix-core kernel forms the exponent as 2c x.y + alpha + beta in
# fp32, so P carries a relative error of about ln2 * 2c * max|x.y| * 2^-24
# (2e-4 for d = 64 points in [0,1] at eps = 0.02, where max|x.y| ~ 16); the
# case with that bound above 1e-4 gets 1e-3.  The contract for bf16 input is 1e-2.
@pytest.mark.parametrize("B,n,m,d,dtype,w,eps,tol", [
    (1, 33, 47, 3, "f32", "uniform", 0.05, 1e-4),
    (2, 300, 257, 3, "f32", "dirichlet", 0.01, 1e-4),
    (1, 150, 140, 3, "bf16", "dirichlet", 0.05, 1e-4),
    (1, 130, 77, 8, "f32", "dirichlet", 0.1, 1e-4),
    (1, 200, 190, 64, "bf16", "uniform", 0.2, 1e-4),
    (2, 1100, 900, 64, "bf16", "dirichlet", 0.1, 1e-4),
    (2, 300, 170, 32, "bf16", "dirichlet", 0.05, 1e-4),
    (1, 129, 1000, 64, "bf16", "dirichlet", 0.02, 1e-3),
    (1, 90, 100, 100, "f32", "uniform", 0.5, 1e-4),
    (1, 70, 60, 96, "bf16", "uniform", 0.3, 1e-4),
])
def test_dense_grad_matches_oracle(B, n, m, d, dtype, w, eps, tol):
    c = workloads.random_case(11, B, n, m, d, weights=w, dtype=dtype)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[20])
    check_dense_grad(c, np.float32(eps), fo, go, tol=tol)


def test_dense_grad_zero_mass_rows_and_single_side():
    c = workloads.random_case(12, 1, 70, 50, 3, weights="dirichlet", zero_weights=4)
    eps = np.float32(0.03)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[10])
    dX, TX, dY, TY = check_dense_grad(c, eps, fo, go)
    assert np.all(host(dX)[0, :4] == 0) and np.all(host(TX)[0, :4] == 0)
    assert np.all(host(dY)[0, :4] == 0) and np.all(host(TY)[0, :4] == 0)
    # one output or one side at a time gives the same values
    X, Y = points(c)
    f32, g32 = dev(fo.astype(np.float32)), dev(go.astype(np.float32))
    a, b = dev(c["a"]), dev(c["b"])
    only_dX = sk.dense_grad(X, Y, a, b, f32, g32, float(eps),
                            out=(torch.empty_like(dX), None, None, None))
    only_y = sk.dense_grad(X, Y, a, b, f32, g32, float(eps), sides="y")
    torch.cuda.synchronize()
    assert torch.equal(only_dX[0], dX) and only_dX[1] is None
    assert only_y[0] is None and only_y[1] is None
    assert torch.equal(only_y[2], dY) and torch.equal(only_y[3], TY)


def test_dense_grad_agrees_with_full_support_coo_gradient():
    c = workloads.random_case(13, 2, 120, 110, 3, weights="dirichlet")
    eps = 0.05
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[15])
    X, Y = points(c)
    f32, g32 = dev(fo.astype(np.float32)), dev(go.astype(np.float32))
    a, b = dev(c["a"]), dev(c["b"])
    rows, cols, vals, offs = sk.plan_coo(X, Y, a, b, f32, g32, eps, 1e-30)
    _, dXc = sk.loss_grad(X, Y, rows, cols, vals, offs)
    dX, _, _, _ = sk.dense_grad(X, Y, a, b, f32, g32, eps, sides="x")
    for p in range(2):
        assert rel_inf(host(dX)[p], host(dXc)[p]) <= 1e-5


def test_workload_pair_1k_dense_grad():
    w, gold = load_workload("pair-1k")
    check_dense_grad(w, float(w["eps"][-1]), gold["f"], gold["g"])


def test_workload_gmm_64k_dense_grad_sampled_rows():
    w, gold = load_workload("gmm-64k")
    rng = np.random.default_rng(1)
    sel_x = np.sort(rng.choice(65536, 256, replace=False))
    sel_y = np.sort(rng.choice(65536, 256, replace=False))
    check_dense_grad(w, float(w["eps"][-1]), gold["f"], gold["g"], sel_x, sel_y)


def test_workload_feat_50k_dense_grad_sampled_rows():
    w, gold = load_workload("feat-50k")
    rng = np.random.default_rng(2)
    sel_x = np.sort(rng.choice(50000, 64, replace=False))
    sel_y = np.sort(rng.choice(60000, 64, replace=False))
    check_dense_grad(w, float(w["eps"][-1]), gold["f"], gold["g"], sel_x, sel_y, tol=1e-2)


def test_dense_grad_matrix_core_fallback_block():
    # rows 64..127 get f raised by 110 eps ln2: their plan mass is 2^110 times the
    # weight, outside the matrix-core kernel's range check, so that block goes to
    # the fp64 pass; the other blocks stay on the matrix cores
    c = workloads.random_case(14, 1, 200, 150, 64, weights="dirichlet", dtype="bf16")
    eps = 0.05
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[30])
    f32 = fo.astype(np.float32)
    f32[0, 64:128] += np.float32(110 * eps * np.log(2.0))
    X, Y = points(c)
    dX, TX, _, _ = sk.dense_grad(X, Y, dev(c["a"]), dev(c["b"]), dev(f32),
                                 dev(go.astype(np.float32)), eps, sides="x")
    torch.cuda.synchronize()
    r_o, dX_o, T_o = oracle.dense_grad(c["X"], c["Y"], c["a"], c["b"], f32.astype(np.float64),
                                       go.astype(np.float32).astype(np.float64), eps)
    # matrix-core blocks to the fp32 exponent bound (see above), the redone block
    # to the fp64 pass's accuracy
    for rows, tol in ((slice(0, 64), 1e-3), (slice(64, 128), 1e-5), (slice(128, 200), 1e-3)):
        assert rel_inf(host(dX)[0, rows], dX_o[0, rows]) <= tol
        assert np.abs(host(TX)[0, rows] - T_o[0, rows]).max() <= tol


# ------------------------------------------- cosine cost and the Y-side gradient
@pytest.mark.parametrize("dtype,d", [("f32", 3), ("bf16", 64), ("f32", 300)])
def test_normalize_and_backward_match_oracle(dtype, d):
    c = workloads.random_case(15, 2, 70, 5, d, dtype=dtype, spread=4.0)
    X = c["X"].copy()
    X[0, 3] = 0.0                                   # a zero vector stays zero
    Xd = dev(X) if dtype == "f32" else \
        dev(workloads.bf16_round(X).view(np.int16)).view(torch.bfloat16)
    Xh, nr = sk.normalize(Xd)
    G = np.random.default_rng(2).normal(size=X.shape).astype(np.float32)
    dX = sk.normalize_backward(Xh, nr, dev(G))
    torch.cuda.synchronize()
    Xh_o, nr_o = oracle.normalize(X)
    np.testing.assert_allclose(host(Xh), Xh_o, rtol=0, atol=1e-7)
    np.testing.assert_allclose(host(nr), nr_o, rtol=1e-7)
    dX_o = oracle.normalize_backward(Xh_o, nr_o, G)
    assert rel_inf(host(dX), dX_o) <= 1e-6
    assert np.all(host(Xh)[0, 3] == 0) and np.all(host(dX)[0, 3] == 0)


@pytest.mark.parametrize("d,eps", [(3, 0.02), (16, 0.05)])
def test_cosine_cost_chain_matches_oracle(d, eps):
    # raw clouds -> normalised -> potentials -> sparse plan -> loss and dL/dX with
    # respect to the raw points, on both sides
    c = workloads.random_case(16, 2, 150, 130, d, weights="dirichlet", spread=3.0)
    X, Y, a, b = dev(c["X"]), dev(c["Y"]), dev(c["a"]), dev(c["b"])
    Xh, nx = sk.normalize(X)
    Yh, ny = sk.normalize(Y)
    f, g, cost = sk.potentials(Xh, Yh, a, b, eps=[eps], iters=[25])
    Xh_o, nx_o = oracle.normalize(c["X"])
    Yh_o, ny_o = oracle.normalize(c["Y"])
    fo, go = oracle.potentials(Xh_o, Yh_o, c["a"], c["b"], eps=[np.float32(eps)], iters=[25])
    torch.cuda.synchronize()
    for p in range(2):
        assert rel_inf(host(f)[p], fo[p], eps) <= 1e-4
        assert rel_inf(host(g)[p], go[p], eps) <= 1e-4
    st = oracle.plan_stats(Xh_o, Yh_o, c["a"], c["b"], fo, go, float(np.float32(eps)))
    np.testing.assert_allclose(host(cost), st["cost"], rtol=1e-4)
    # sparse plan and gradients from the oracle's potentials, on both sides
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    rows, cols, vals, offs = sk.plan_coo(Xh, Yh, a, b, dev(f32), dev(g32), eps, 1e-8)
    loss, dXh = sk.loss_grad(Xh, Yh, rows, cols, vals, offs)
    dX = sk.normalize_backward(Xh, nx, dXh)
    torch.cuda.synchronize()
    ro, co, vo, oo = oracle.plan_coo(Xh_o, Yh_o, c["a"], c["b"], f32.astype(np.float64),
                                     g32.astype(np.float64), float(np.float32(eps)), 1e-8)
    lo, dXh_o = oracle.loss_grad(Xh_o, Yh_o, ro, co, vo, oo)
    dX_o = oracle.normalize_backward(Xh_o, nx_o, dXh_o)
    np.testing.assert_allclose(host(loss), lo, rtol=1e-4)
    for p in range(2):
        assert rel_inf(host(dX)[p], dX_o[p]) <= 1e-4


def test_transposed_sparse_plan_and_y_gradient():
    c = workloads.random_case(17, 2, 260, 300, 3, weights="dirichlet")
    eps = 0.02
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[15])
    X, Y, a, b = dev(c["X"]), dev(c["Y"]), dev(c["a"]), dev(c["b"])
    f32, g32 = dev(fo.astype(np.float32)), dev(go.astype(np.float32))
    r1, c1, v1, o1 = sk.plan_coo(X, Y, a, b, f32, g32, eps, 1e-8)
    r2, c2, v2, o2 = sk.plan_coo(Y, X, b, a, g32, f32, eps, 1e-8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    R1, C1, V1, O1 = (t.cpu().numpy() for t in (r1, c1, v1, o1))
    R2, C2, V2 = (t.cpu().numpy() for t in (r2, c2, v2))
    for p in range(2):
        s1, s2 = slice(O1[p], O1[p + 1]), slice(O1[p], O1[p + 1])
        order = np.lexsort((R1[s1], C1[s1]))
        # exactly the transpose: same entries, bit-identical values
        np.testing.assert_array_equal(R2[s2], C1[s1][order])
        np.testing.assert_array_equal(C2[s2], R1[s1][order])
        np.testing.assert_array_equal(V2[s2], V1[s1][order])
    _, dY = sk.loss_grad(Y, X, r2, c2, v2, o2)
    torch.cuda.synchronize()
    ro, co, vo, oo = oracle.plan_coo(c["Y"], c["X"], c["b"], c["a"],
                                     go.astype(np.float32).astype(np.float64),
                                     fo.astype(np.float32).astype(np.float64), eps, 1e-8)
    _, dY_o = oracle.loss_grad(c["Y"], c["X"], ro, co, vo, oo)
    for p in range(2):
        assert rel_inf(host(dY)[p], dY_o[p]) <= 1e-4


# --------------------------------------------- Sinkhorn normalisation in COO form
def _coo_dev(coo):
    rows, cols, vals, offs = coo
    return (dev(rows.astype(np.int32)), dev(cols.astype(np.int32)),
            dev(vals.astype(np.float32)), dev(offs.astype(np.int64)))


@pytest.mark.parametrize("B,n,m,eps,thr,iters", [(1, 33, 47, 0.05, 1e-8, 1),
                                                  (2, 300, 257, 0.01, 1e-8, 20),
                                                  (3, 128, 200, 0.02, 1e-4, 200)])
def test_coo_normalize_matches_oracle(B, n, m, eps, thr, iters):
    # both sides normalise the oracle's plan (fp32 values), so the supports agree
    c = workloads.random_case(18, B, n, m, 3, weights="dirichlet")
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[10])
    plan = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], fo, go, eps, rel_thr=thr)
    tr = oracle.plan_coo(c["Y"], c["X"], c["b"], c["a"], go, fo, eps, rel_thr=thr)
    vals32 = plan[2].astype(np.float32)
    v_o, err_o = oracle.coo_normalize(plan[0], plan[1], vals32.astype(np.float64), plan[3],
                                      c["a"], c["b"], n, m, iters)
    P = _coo_dev((plan[0], plan[1], vals32, plan[3]))
    T = _coo_dev(tr)
    err = sk.coo_normalize(P, T, dev(c["a"]), dev(c["b"]), n, m, iters)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(P[2]), v_o, rtol=1e-4, atol=0)
    np.testing.assert_allclose(host(err), err_o, rtol=1e-3, atol=1e-6)
    _assert_transposes(P, T, B)


def test_coo_normalize_unaligned_values():
    # value arrays that start 4 bytes past a 16-byte boundary take the log pass's
    # one-entry-at-a-time form; the result is the aligned call's, bit for bit
    c = workloads.random_case(19, 2, 150, 170, 3, weights="dirichlet")
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[0.03], iters=[10])
    plan = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], fo, go, 0.03, rel_thr=1e-8)
    tr = oracle.plan_coo(c["Y"], c["X"], c["b"], c["a"], go, fo, 0.03, rel_thr=1e-8)
    runs = []
    for shift in (0, 1):
        P = list(_coo_dev((plan[0], plan[1], plan[2].astype(np.float32), plan[3])))
        T = list(_coo_dev(tr))
        for Z in (P, T):
            buf = torch.zeros(Z[2].numel() + 4, dtype=torch.float32, device=Z[2].device)
            view = buf[shift:shift + Z[2].numel()]
            view.copy_(Z[2])
            Z[2] = view
        assert (P[2].data_ptr() % 16 == 0) == (shift == 0)
        err = sk.coo_normalize(tuple(P), tuple(T), dev(c["a"]), dev(c["b"]), 150, 170, 20)
        torch.cuda.synchronize()
        runs.append((host(P[2]), host(T[2]), host(err)))
    for u, v in zip(runs[0], runs[1]):
        np.testing.assert_array_equal(u, v)


def _assert_transposes(P, T, B):
    """T holds P's entries and values, bit for bit, in column-major order."""
    r1, c1, v1, o1 = (host(t) for t in P)
    r2, c2, v2, o2 = (host(t) for t in T)
    for p in range(B):
        s1 = slice(int(o1[p]), int(o1[p + 1]))
        s2 = slice(int(o2[p]), int(o2[p + 1]))
        order = np.lexsort((r1[s1], c1[s1]))
        np.testing.assert_array_equal(r2[s2], c1[s1][order])
        np.testing.assert_array_equal(c2[s2], r1[s1][order])
        np.testing.assert_array_equal(v2[s2], v1[s1][order])


def test_coo_normalize_degenerate_support():
    # a row with no entry, a stored zero, a zero row weight and a column reached
    # only through that row: scalings of empty rows and columns stay 0, a zero
    # weight empties its row, and both sides agree with the oracle
    B, n, m = 2, 6, 5
    rng = np.random.default_rng(65)
    rows, cols, vals, offs = [], [], [], [0]
    for p in range(B):
        for i in range(n):
            if i == 2:
                continue                                  # row 2: no entry
            for j in sorted(rng.choice(m, size=rng.integers(1, m + 1), replace=False)):
                if p == 1 and j == 4 and i != 0:
                    continue                              # column 4 of pair 1 only via row 0
                rows.append(i)
                cols.append(j)
                vals.append(0.0 if (i, j) == (3, 1) else rng.random() + 0.05)
        offs.append(len(rows))
    rows, cols = np.array(rows, dtype=np.int32), np.array(cols, dtype=np.int32)
    vals, offs = np.array(vals, dtype=np.float32), np.array(offs, dtype=np.int64)
    a = rng.dirichlet(np.ones(n), size=B).astype(np.float32)
    a[1, 0] = 0.0                                         # zero weight on row 0 of pair 1
    b = rng.dirichlet(np.ones(m), size=B).astype(np.float32)
    # the transpose: the same entries in column-major order
    t_rows, t_cols, t_vals = [], [], []
    for p in range(B):
        s_ = slice(offs[p], offs[p + 1])
        order = np.lexsort((rows[s_], cols[s_]))
        t_rows.append(cols[s_][order])
        t_cols.append(rows[s_][order])
        t_vals.append(vals[s_][order])
    T = _coo_dev((np.concatenate(t_rows), np.concatenate(t_cols), np.concatenate(t_vals), offs))
    P = _coo_dev((rows, cols, vals, offs))
    v_o, err_o = oracle.coo_normalize(rows, cols, vals.astype(np.float64), offs, a, b, n, m, 25)
    err = sk.coo_normalize(P, T, dev(a), dev(b), n, m, 25)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(P[2]), v_o, rtol=1e-4, atol=1e-30)
    np.testing.assert_allclose(host(err), err_o, rtol=1e-3, atol=1e-6)
    assert host(P[2])[(rows == 3) & (cols == 1)].max() == 0.0
    _assert_transposes(P, T, B)


def test_coo_normalize_gpu_chain_reaches_the_marginals():
    c = workloads.random_case(19, 2, 400, 350, 3, weights="dirichlet")
    eps = 0.02
    X, Y, a, b = dev(c["X"]), dev(c["Y"]), dev(c["a"]), dev(c["b"])
    f, g, _ = sk.potentials(X, Y, a, b, eps=[eps], iters=[10])
    P = sk.plan_coo(X, Y, a, b, f, g, eps, 1e-8)
    T = sk.plan_coo(Y, X, b, a, g, f, eps, 1e-8)
    _assert_transposes(P, T, 2)   # the two extractions agree before normalisation
    before = P[2].clone()
    err = sk.coo_normalize(P, T, a, b, 400, 350, 300)
    torch.cuda.synchronize()
    e = host(err)
    assert np.all(e[:, 1] < 1e-5) and np.all(e[:, 0] < 1e-4), e
    # the column sums after the last half-step are b; the support is unchanged
    assert P[2].shape == before.shape and bool((P[2] >= 0).all())
    _assert_transposes(P, T, 2)   # and after it


def test_coo_normalize_rejects_a_mismatched_transpose():
    c = workloads.random_case(20, 1, 64, 70, 3)
    eps = 0.05
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[5])
    plan = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], fo, go, eps, rel_thr=1e-3)
    tr = list(oracle.plan_coo(c["Y"], c["X"], c["b"], c["a"], go, fo, eps, rel_thr=1e-3))
    bad_col = [tr[0], tr[1].copy(), tr[2], tr[3]]
    bad_col[1][0] = (bad_col[1][0] + 1) % 64        # one transposed entry points elsewhere
    bad_val = [tr[0], tr[1], tr[2].astype(np.float32), tr[3]]
    bad_val[2][len(bad_val[2]) // 2] *= 1.5         # one transposed value differs
    for t in (bad_col, bad_val):
        P, T = _coo_dev(plan), _coo_dev(t)
        before, t_before = P[2].clone(), T[2].clone()
        with pytest.raises(sk.SinkhornError) as ex:
            sk.coo_normalize(P, T, None, None, 64, 70, 5)
        assert ex.value.status == sk.SK_ERR_INVALID_ARG
        assert torch.equal(P[2], before) and torch.equal(T[2], t_before)


@pytest.mark.parametrize("name,pairs", [("sphere-2k", [0, 31]), ("blobs-1k", [0, 255])])
def test_workload_coo_normalize_sampled_pairs(name, pairs):
    w = workloads.make(name, pairs=pairs)
    gold = golden(name)
    eps = float(w["eps"][-1])
    n, m = w["X"].shape[1], w["Y"].shape[1]
    fo = gold["f"][pairs].astype(np.float32).astype(np.float64)
    go = gold["g"][pairs].astype(np.float32).astype(np.float64)
    plan = oracle.plan_coo(w["X"], w["Y"], w["a"], w["b"], fo, go, eps, rel_thr=w["threshold"])
    tr = oracle.plan_coo(w["Y"], w["X"], w["b"], w["a"], go, fo, eps, rel_thr=w["threshold"])
    vals32 = plan[2].astype(np.float32)
    v_o, err_o = oracle.coo_normalize(plan[0], plan[1], vals32.astype(np.float64), plan[3],
                                      w["a"], w["b"], n, m, 10)
    P = _coo_dev((plan[0], plan[1], vals32, plan[3]))
    T = _coo_dev(tr)
    err = sk.coo_normalize(P, T, dev(w["a"]), dev(w["b"]), n, m, 10)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(P[2]), v_o, rtol=1e-4, atol=0)
    np.testing.assert_allclose(host(err), err_o, rtol=1e-3, atol=1e-6)
    _assert_transposes(P, T, len(pairs))


# ------------------------------------------------------- Hessian-vector product
# bf16 with d = 32 / 64 runs on the matrix cores: fp32 plan entries (exponent
# bound ln2 * 2c * max|x.y| * 2^-24, under 1e-5 here), the direction in two bf16
# pieces (2^-17) and fp32 sums, all below the 1e-4 held for the fp64 path.
@pytest.mark.parametrize("B,n,m,d,dtype,eps,zw", [(1, 40, 50, 3, "f32", 0.1, 0),
                                                  (2, 120, 90, 3, "f32", 0.05, 0),
                                                  (1, 60, 70, 3, "bf16", 0.1, 0),
                                                  (1, 80, 90, 3, "f32", 0.1, 5),
                                                  (1, 64, 70, 8, "f32", 0.2, 0),
                                                  (1, 50, 45, 16, "bf16", 0.5, 0),
                                                  (1, 50, 45, 64, "bf16", 0.5, 0),
                                                  (2, 70, 90, 32, "bf16", 1.0, 0),
                                                  (1, 150, 170, 64, "bf16", 0.5, 0),
                                                  (2, 20, 600, 64, "bf16", 1.0, 0),
                                                  (1, 97, 81, 64, "bf16", 0.5, 3)])
def test_hvp_matches_oracle(B, n, m, d, dtype, eps, zw):
    c = workloads.random_case(21, B, n, m, d, weights="dirichlet", dtype=dtype, zero_weights=zw)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[2000])
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    V = np.random.default_rng(3).normal(size=(B, n, d)).astype(np.float32)
    X, Y = points(c)
    HV, res = sk.hvp(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32), eps, dev(V),
                     cg_iters=300)
    torch.cuda.synchronize()
    HVo = oracle.hvp(c["X"], c["Y"], c["a"], c["b"], f32.astype(np.float64),
                     g32.astype(np.float64), np.float32(eps), V)
    assert np.all(host(res) < 1e-4), host(res)
    for p in range(B):
        assert rel_inf(host(HV)[p], HVo[p]) <= 1e-4


@pytest.mark.parametrize("B,n,m,d,dtype,eps,iters", [(1, 1000, 1100, 3, "f32", 0.1, 2000),
                                                    (1, 1000, 900, 64, "bf16", 0.5, 200),
                                                    (2, 700, 650, 64, "bf16", 1.0, 200)])
def test_hvp_matches_oracle_at_a_thousand_points(B, n, m, d, dtype, eps, iters):
    # the product against the oracle's dense one at sizes that span many row
    # blocks and key splits of either path (fp64 passes for d = 3, matrix cores
    # for bf16 features), with ragged sides
    c = workloads.random_case(22, B, n, m, d, weights="dirichlet", dtype=dtype)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[iters])
    f32, g32 = fo.astype(np.float32), go.astype(np.float32)
    V = np.random.default_rng(3).normal(size=(B, n, d)).astype(np.float32)
    X, Y = points(c)
    HV, res = sk.hvp(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32), eps, dev(V),
                     cg_iters=300)
    torch.cuda.synchronize()
    HVo = oracle.hvp(c["X"], c["Y"], c["a"], c["b"], f32.astype(np.float64),
                     g32.astype(np.float64), np.float32(eps), V)
    assert np.all(host(res) < 1e-4), host(res)
    for p in range(B):
        assert rel_inf(host(HV)[p], HVo[p]) <= 1e-4


def hvp_case(seed, B, n, m, d, eps, iters=2000, dtype="bf16"):
    c = workloads.random_case(seed, B, n, m, d, weights="dirichlet", dtype=dtype)
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[iters])
    X, Y = points(c)
    return c, X, Y, dev(c["a"]), dev(c["b"]), dev(fo.astype(np.float32)), dev(go.astype(np.float32))


def test_hvp_matrix_cores_symmetric_linear_and_deterministic():
    c, X, Y, a, b, f, g = hvp_case(23, 2, 300, 260, 64, 0.5)
    rng = np.random.default_rng(8)
    U = dev(rng.normal(size=(2, 300, 64)).astype(np.float32))
    V = dev(rng.normal(size=(2, 300, 64)).astype(np.float32))
    HU, ru = sk.hvp(X, Y, a, b, f, g, 0.5, U, cg_iters=200)
    HV, rv = sk.hvp(X, Y, a, b, f, g, 0.5, V, cg_iters=200)
    HW, _ = sk.hvp(X, Y, a, b, f, g, 0.5, 2.0 * U - V, cg_iters=200)
    HV2, rv2 = sk.hvp(X, Y, a, b, f, g, 0.5, V, cg_iters=200)
    torch.cuda.synchronize()
    assert torch.equal(HV, HV2) and torch.equal(rv, rv2)
    assert np.all(host(ru) < 1e-4) and np.all(host(rv) < 1e-4)
    for p in range(2):
        hu, hv, hw, u, v = (host(t)[p] for t in (HU, HV, HW, U, V))
        assert rel_inf(hw, 2.0 * hu - hv) <= 1e-4
        assert abs((u * hv).sum() - (v * hu).sum()) <= 1e-4 * np.abs(u * hv).sum()


def test_hvp_matrix_cores_far_potentials_give_nan():
    # zero potentials at a small eps put every row's plan mass far below 2^-64 of
    # its weight: the matrix-core path marks the pair and returns NaN
    c = workloads.random_case(24, 2, 60, 70, 64, weights="uniform", dtype="bf16")
    X, Y = points(c)
    eps = 0.01
    f = torch.zeros(2, 60, device="cuda")
    g = torch.zeros(2, 70, device="cuda")
    V = torch.ones(2, 60, 64, device="cuda")
    HV, res = sk.hvp(X, Y, dev(c["a"]), dev(c["b"]), f, g, eps, V, cg_iters=3)
    torch.cuda.synchronize()
    assert torch.isnan(HV).all() and torch.isnan(res).all()


def test_workload_feat_50k_hvp_properties():
    # full size: the plan is n x m = 3e9 entries, beyond the oracle's dense HVP;
    # properties that hold at any size stand in (symmetry of u.Hv, linearity,
    # CG convergence, finiteness), on the stored potentials
    w, gold = load_workload("feat-50k")
    X, Y = points(w)
    a, b = dev(w["a"]), dev(w["b"])
    f, g = dev(gold["f"].astype(np.float32)), dev(gold["g"].astype(np.float32))
    eps = float(w["eps"][-1])
    rng = np.random.default_rng(9)
    U = dev((rng.normal(size=(1, 50000, 64)) / 8).astype(np.float32))
    V = dev((rng.normal(size=(1, 50000, 64)) / 8).astype(np.float32))
    HU, ru = sk.hvp(X, Y, a, b, f, g, eps, U, cg_iters=60)
    HV, rv = sk.hvp(X, Y, a, b, f, g, eps, V, cg_iters=60)
    HW, rw = sk.hvp(X, Y, a, b, f, g, eps, U + V, cg_iters=60)
    torch.cuda.synchronize()
    print("feat-50k hvp residuals", host(ru), host(rv), host(rw), flush=True)
    for t in (HU, HV, HW):
        assert bool(torch.isfinite(t).all())
    assert np.all(host(ru) < 1e-3) and np.all(host(rv) < 1e-3)
    hu, hv, hw, u, v = (host(t)[0].astype(np.float64) for t in (HU, HV, HW, U, V))
    assert rel_inf(hw, hu + hv) <= 1e-3
    assert abs((u * hv).sum() - (v * hu).sum()) <= 1e-3 * np.abs(u * hv).sum()


def test_hvp_is_linear_and_symmetric_on_gpu():
    c = workloads.random_case(22, 1, 80, 60, 3, weights="dirichlet")
    eps = 0.1
    fo, go = oracle.potentials(c["X"], c["Y"], c["a"], c["b"], eps=[eps], iters=[2000])
    X, Y, a, b = dev(c["X"]), dev(c["Y"]), dev(c["a"]), dev(c["b"])
    f32, g32 = dev(fo.astype(np.float32)), dev(go.astype(np.float32))
    rng = np.random.default_rng(6)
    U = dev(rng.normal(size=(1, 80, 3)).astype(np.float32))
    V = dev(rng.normal(size=(1, 80, 3)).astype(np.float32))
    HU, _ = sk.hvp(X, Y, a, b, f32, g32, eps, U, cg_iters=200)
    HV, _ = sk.hvp(X, Y, a, b, f32, g32, eps, V, cg_iters=200)
    HW, _ = sk.hvp(X, Y, a, b, f32, g32, eps, 2.0 * U - V, cg_iters=200)
    torch.cuda.synchronize()
    hu, hv, hw, u, v = (host(t)[0] for t in (HU, HV, HW, U, V))
    assert rel_inf(hw, 2.0 * hu - hv) <= 1e-5
    assert abs((u * hv).sum() - (v * hu).sum()) <= 1e-5 * np.abs(u * hv).sum()


# ------------------------------------------------- property-based random shapes
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(B=st.integers(1, 4), n=st.integers(1, 300), m=st.integers(1, 300),
       kind=st.sampled_from([(3, "f32"), (3, "bf16"), (64, "f32"), (64, "bf16")]),
       weights=st.sampled_from(["uniform", "dirichlet"]),
       eps=st.sampled_from([0.02, 0.05, 0.2]), iters=st.integers(1, 12),
       seed=st.integers(0, 1 << 16))
def test_random_shapes_match_oracle(B, n, m, kind, weights, eps, iters, seed):
    d, dtype = kind
    print(f"case B={B} n={n} m={m} d={d} {dtype} {weights} eps={eps} iters={iters} "
          f"seed={seed}", flush=True)
    c = workloads.random_case(1000 + seed, B, n, m, d, weights=weights, dtype=dtype,
                              spread=1.0 if d == 3 else 0.25)
    _, _, fo, go = check_potentials(c, [eps], [iters])
    if d == 3:
        # sparse plan and fused loss from the oracle's potentials (rounded to fp32)
        check_coo_given_potentials(c, eps, fo, go)
        f32, g32 = fo.astype(np.float32), go.astype(np.float32)
        X, Y = points(c)
        _, loss, dX = fused_plan_loss(X, Y, dev(c["a"]), dev(c["b"]), dev(f32), dev(g32), eps,
                                      1e-8)
        ro, co, vo, oo = oracle.plan_coo(c["X"], c["Y"], c["a"], c["b"], f32, g32,
                                         float(np.float32(eps)), 1e-8)
        lo, dXo = oracle.loss_grad(c["X"], c["Y"], ro, co, vo.astype(np.float32), oo)
        np.testing.assert_allclose(host(loss), lo, rtol=1e-4)
        for p in range(B):
            assert rel_inf(host(dX)[p], dXo[p], 1e-30) <= 1e-4


# ------------------------------------------------------- streams and graph capture
def test_work_follows_the_callers_stream():
    # inputs produced on a side stream and every call issued there: the results
    # equal those of the default stream (nothing runs on another stream)
    c = workloads.random_case(61, 3, 500, 400, 3, weights="dirichlet")
    eps = 0.03
    X0, Y0 = points(c)
    a0, b0 = dev(c["a"]), dev(c["b"])
    f0, g0, cost0 = sk.potentials(X0, Y0, a0, b0, eps=[eps], iters=[20])
    loss0 = torch.empty(3, device=X0.device)
    dX0 = torch.empty(3, 500, 3, device=X0.device)
    plan0 = sk.plan_coo(X0, Y0, a0, b0, f0, g0, eps, 1e-8, loss_out=(loss0, dX0))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        X, Y = X0 * 1.0, Y0 * 1.0          # produced on s
        a, b = a0 * 1.0, b0 * 1.0
        f, g, cost = sk.potentials(X, Y, a, b, eps=[eps], iters=[20])
        loss = torch.empty(3, device=X.device)
        dX = torch.empty(3, 500, 3, device=X.device)
        plan = sk.plan_coo(X, Y, a, b, f, g, eps, 1e-8, loss_out=(loss, dX))
    s.synchronize()
    for u, v in ((f, f0), (g, g0), (cost, cost0), (loss, loss0), (dX, dX0)):
        assert torch.equal(u, v)
    for u, v in zip(plan, plan0):
        assert torch.equal(u, v)


@pytest.mark.parametrize("shape", ["batch", "split_keys_stale", "per_pair_stages",
                                   "split_stages"])
def test_potentials_replay_from_a_captured_graph(shape):
    # the potentials entry point launches kernels only (no allocation, copy or
    # wait), so a caller can capture it; every replay equals the eager result.
    # Shapes: one launch per half-iteration; split key ranges whose merged rows
    # go stale (merge marks and repair launch inside the graph); whole stages
    # per pair (cold start with exact shifts); whole stages of one pair split
    # over work-groups (the hand-over words zeroed by a kernel in each stage)
    if shape == "batch":
        B, n, m, seed, sched = 2, 700, 600, 62, dict(eps=[0.3, 0.05, 0.02], iters=[3, 5, 10])
        c = workloads.random_case(seed, B, n, m, 3, weights="dirichlet")
    elif shape == "split_keys_stale":
        B, n, m, seed, sched = 1, 300, 20000, 64, dict(eps=[0.05, 0.003], iters=[2, 3])
        c = workloads.random_case(seed, B, n, m, 3, weights="dirichlet", spread=4.0)
        c = dict(c, X=c["X"] + np.float32(10.0), Y=c["Y"] + np.float32(10.0))
    elif shape == "per_pair_stages":
        B, n, m, seed, sched = 256, 130, 140, 65, dict(eps=[0.1, 0.02], iters=[2, 4])
        c = workloads.random_case(seed, B, n, m, 3, weights="dirichlet")
    else:
        B, n, m, seed, sched = 1, 1000, 900, 66, dict(eps=[0.1, 0.1, 0.02], iters=[1, 3, 4])
        c = workloads.random_case(seed, B, n, m, 3, weights="dirichlet")
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_POTENTIALS, B, n, m, 3, sk.SK_F32),
                     dtype=torch.uint8, device=X.device)
    out = (torch.empty(B, n, device=X.device), torch.empty(B, m, device=X.device),
           torch.empty(B, device=X.device))
    sk.potentials(X, Y, a, b, out=out, workspace=ws, **sched)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            sk.potentials(X, Y, a, b, out=out, workspace=ws, **sched)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))          # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(out, ref):
            assert torch.equal(t, r), f"replay {rep}"


def _plan_buffers(cap, B, n, dev_):
    return ((torch.full((cap,), -5, dtype=torch.int32, device=dev_),
             torch.full((cap,), -5, dtype=torch.int32, device=dev_),
             torch.full((cap,), -5.0, dtype=torch.float32, device=dev_),
             torch.full((B + 1,), -5, dtype=torch.int64, device=dev_)),
            (torch.full((B,), -5.0, device=dev_), torch.full((B, n, 3), -5.0, device=dev_)))


def test_plan_without_waiting_equals_the_waiting_plan():
    c = workloads.random_case(63, 3, 400, 350, 3, weights="dirichlet")
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    eps = 0.02
    f, g, _ = sk.potentials(X, Y, a, b, eps=[eps], iters=[15])
    loss = torch.empty(3, device=X.device)
    dX = torch.empty(3, 400, 3, device=X.device)
    ref = sk.plan_coo(X, Y, a, b, f, g, eps, 1e-8, loss_out=(loss, dX))
    total = int(ref[3][-1])
    # room to spare: the same plan, loss and gradient, bit for bit
    out, lo = _plan_buffers(total + 100, 3, 400, X.device)
    nnz = sk.plan_coo_async(X, Y, a, b, f, g, eps, 1e-8, out, loss_out=lo)
    torch.cuda.synchronize()
    assert int(nnz) == total
    for u, v in zip(out[:3], ref[:3]):
        assert torch.equal(u[:total], v)
    assert torch.equal(out[3], ref[3]) and torch.equal(lo[0], loss) and torch.equal(lo[1], dX)
    # one entry short: the count and the offsets are written, nothing else
    out, lo = _plan_buffers(total - 1, 3, 400, X.device)
    nnz = sk.plan_coo_async(X, Y, a, b, f, g, eps, 1e-8, out, loss_out=lo)
    torch.cuda.synchronize()
    assert int(nnz) == total and torch.equal(out[3], ref[3])
    for t in list(out[:3]) + list(lo):
        assert bool((t == -5).all())


def test_forward_and_gradient_replay_from_a_captured_graph():
    # potentials, the sparse plan and its loss and gradient with no host wait:
    # the whole step is captured once and replayed
    c = workloads.random_case(64, 4, 300, 280, 3, weights="dirichlet")
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    B, n, m = 4, 300, 280
    eps = 0.03
    ws = torch.empty(sk.workspace_bytes(sk.SK_OP_POTENTIALS, B, n, m, 3, sk.SK_F32),
                     dtype=torch.uint8, device=X.device)
    cws = torch.empty(sk.workspace_bytes(sk.SK_OP_PLAN_COO, B, n, m, 3, sk.SK_F32),
                      dtype=torch.uint8, device=X.device)
    pot = (torch.empty(B, n, device=X.device), torch.empty(B, m, device=X.device), None)
    out, lo = _plan_buffers(B * n * m, B, n, X.device)
    nnz = torch.empty(1, dtype=torch.int64, device=X.device)

    def step():
        sk.potentials(X, Y, a, b, eps=[eps], iters=[12], cost=False, out=pot, workspace=ws)
        sk.plan_coo_async(X, Y, a, b, pot[0], pot[1], eps, 1e-8, out, loss_out=lo,
                          workspace=cws, nnz=nnz)

    step()
    torch.cuda.synchronize()
    total = int(nnz)
    assert total <= B * n * m

    def results():   # the written part of every output
        return list(pot[:2]) + [t[:total] for t in out[:3]] + [out[3]] + list(lo) + [nnz]

    ref = [t.clone() for t in results()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in list(pot[:2]) + list(lo):
            t.fill_(float("nan"))
        out[2].fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(results(), ref):
            assert torch.equal(t, r), f"replay {rep}"


@pytest.mark.parametrize("d,dtype", [(3, "f32"), (64, "bf16")])
def test_hvp_and_dense_grad_replay_from_a_captured_graph(d, dtype):
    # the Hessian-vector product (fp64 passes for d = 3, matrix cores for bf16
    # d = 64, with its CG stop decided on the device) and the dense gradient
    # launch kernels only: captured once, every replay equals the eager run
    B, n, m = 2, 150, 170
    eps = 0.5 if d == 64 else 0.1
    c = workloads.random_case(66, B, n, m, d, weights="dirichlet", dtype=dtype)
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    f, g, _ = sk.potentials(X, Y, a, b, eps=[eps], iters=[300])
    V = dev(np.random.default_rng(12).normal(size=(B, n, d)).astype(np.float32))
    dt = sk.SK_BF16 if dtype == "bf16" else sk.SK_F32
    hws = torch.empty(sk.workspace_bytes(sk.SK_OP_HVP, B, n, m, d, dt), dtype=torch.uint8,
                      device=X.device)
    gws = torch.empty(sk.workspace_bytes(sk.SK_OP_DENSE_GRAD, B, n, m, d, dt),
                      dtype=torch.uint8, device=X.device)
    HV = torch.empty(B, n, d, device=X.device)
    dg = (torch.empty(B, n, d, device=X.device), torch.empty(B, n, d, device=X.device),
          torch.empty(B, m, d, device=X.device), torch.empty(B, m, d, device=X.device))

    def step():
        _, res = sk.hvp(X, Y, a, b, f, g, eps, V, cg_iters=40, workspace=hws, out=HV)
        sk.dense_grad(X, Y, a, b, f, g, eps, workspace=gws, out=dg)
        return res

    res = step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (HV, *dg, res)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            res_g = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (HV, *dg, res_g):
            t.fill_(float("nan"))          # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip((HV, *dg, res_g), ref):
            assert torch.equal(t, r), f"replay {rep}"


def test_binding_refuses_bad_output_buffers_before_the_call():
    # each public function checks caller-provided outputs (dtype, exact shape,
    # contiguous layout, device) before a pointer reaches the C ABI; the
    # refused call leaves the buffers untouched
    c = workloads.random_case(90, 2, 40, 30, 3)
    X, Y = points(c)
    a, b = dev(c["a"]), dev(c["b"])
    d0 = X.device
    f, g, _ = sk.potentials(X, Y, a, b, eps=[0.1], iters=[2])
    torch.cuda.synchronize()
    sentinel = torch.full((2, 40), 5.0, device=d0)
    with pytest.raises(ValueError):   # f of the wrong shape
        sk.potentials(X, Y, a, b, eps=[0.1], iters=[2],
                      out=(torch.empty(2, 41, device=d0), torch.empty(2, 30, device=d0), None))
    with pytest.raises(ValueError):   # strided g
        sk.potentials(X, Y, a, b, eps=[0.1], iters=[2],
                      out=(sentinel, torch.empty(30, 2, device=d0).t(), None))
    assert bool((sentinel == 5.0).all())
    cap = 100
    with pytest.raises(ValueError):   # cols shorter than rows
        sk.plan_coo(X, Y, a, b, f, g, 0.1, 1e-8,
                    out=(torch.empty(cap, dtype=torch.int32, device=d0),
                         torch.empty(cap - 1, dtype=torch.int32, device=d0),
                         torch.empty(cap, device=d0), torch.empty(3, dtype=torch.int64, device=d0)))
    with pytest.raises(ValueError):   # nnz of the wrong dtype
        sk.plan_coo_async(X, Y, a, b, f, g, 0.1, 1e-8,
                          out=(torch.empty(cap, dtype=torch.int32, device=d0),
                               torch.empty(cap, dtype=torch.int32, device=d0),
                               torch.empty(cap, device=d0),
                               torch.empty(3, dtype=torch.int64, device=d0)),
                          nnz=torch.empty(1, dtype=torch.int32, device=d0))
    with pytest.raises(ValueError):   # loss_out dX of the wrong shape
        sk.plan_coo(X, Y, a, b, f, g, 0.1, 1e-8,
                    loss_out=(None, torch.empty(2, 40, 4, device=d0)))
    rows, cols, vals, offs = sk.plan_coo(X, Y, a, b, f, g, 0.1, 1e-8)
    with pytest.raises(ValueError):   # float64 loss
        sk.loss_grad(X, Y, rows, cols, vals, offs,
                     out=(torch.empty(2, dtype=torch.float64, device=d0), None))
    with pytest.raises(ValueError):   # vals shorter than rows
        sk.loss_grad(X, Y, rows, cols, vals[:-1], offs)
    with pytest.raises(ValueError):   # strided dY
        sk.dense_grad(X, Y, a, b, f, g, 0.1,
                      out=(None, None, torch.empty(2, 3, 30, device=d0).transpose(1, 2), None))
    with pytest.raises(ValueError):   # HV of the wrong shape
        sk.hvp(X, Y, a, b, f, g, 0.1, torch.zeros(2, 40, 3, device=d0), cg_iters=2,
               out=torch.empty(2, 40, 2, device=d0))
    with pytest.raises(ValueError):   # offsets that run past the plan's entries
        bad_offs = offs.clone()
        bad_offs[-1] = rows.numel() + 5
        sk.coo_normalize((rows, cols, vals.clone(), bad_offs), (rows, cols, vals.clone(), offs),
                         a, b, 40, 30, 2)
