"""sinkhorn_potentials_noalloc (static scratch, no workspace, no allocation)
against sinkhorn_potentials (caller workspace) on the same inputs.

Both entry points run the same kernels in the same order, so their potentials
and costs must agree bit for bit; the calls come in a row, each on a smaller
input than the one before, so that the shared scratch holds the previous
call's contents when the next one starts.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
sk = pytest.importorskip("sinkhorn_point_cloud_amd")

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _inputs(c):
    if c.get("dtype") == "bf16":
        X = dev(c["X_bits"].view(np.int16)).view(torch.bfloat16)
        Y = dev(c["Y_bits"].view(np.int16)).view(torch.bfloat16)
    else:
        X, Y = dev(c["X"]), dev(c["Y"])
    return X, Y, dev(c["a"]), dev(c["b"])


def _outputs(B, n, m, with_cost=True):
    d0 = torch.device("cuda:0")
    return (torch.full((B, n), float("nan"), device=d0),
            torch.full((B, m), float("nan"), device=d0),
            torch.full((B,), float("nan"), device=d0) if with_cost else None)


def _compare(c, eps, iters, warm=None):
    X, Y, a, b = _inputs(c)
    B, n, m = X.shape[0], X.shape[1], Y.shape[1]
    ref = sk.potentials(X, Y, a, b, eps=eps, iters=iters,
                        f0=None if warm is None else dev(warm[0]),
                        g0=None if warm is None else dev(warm[1]))
    out = _outputs(B, n, m)
    if warm is not None:
        out[0].copy_(dev(warm[0]))
        out[1].copy_(dev(warm[1]))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    sk.potentials_noalloc(X, Y, a, b, eps, iters, out, warm_start=warm is not None)
    after = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    assert after == before, "the no-allocation call allocated device memory"
    for name, got, want in zip(("f", "g", "cost"), out, ref):
        assert torch.isfinite(got).all(), name
        assert torch.equal(got, want), f"{name}: max diff {(got - want).abs().max().item()}"
    return out


def test_noalloc_matches_workspace_entry_point_on_successive_calls():
    # 1) two pairs with split-free launches, annealed schedule
    c1 = workloads.random_case(71, 2, 3000, 2500, 3, weights="dirichlet")
    _compare(c1, [0.3, 0.05], [3, 6])
    # 2) one pair whose key range is split across work-groups and whose merged
    #    rows go stale (far from the origin, small eps): merge marks and repair
    c2 = workloads.random_case(72, 1, 300, 20000, 3, weights="dirichlet", spread=4.0)
    c2 = dict(c2, X=c2["X"] + np.float32(10.0), Y=c2["Y"] + np.float32(10.0))
    _compare(c2, [0.05, 0.003], [2, 3])
    # 3) a smaller input after the larger ones (the scratch holds their data)
    c3 = workloads.random_case(73, 1, 300, 257, 3)
    f3, g3, _ = _compare(c3, [0.05], [10])
    # 4) warm start from the previous result, same shape
    _compare(c3, [0.05], [5], warm=(f3.cpu().numpy(), g3.cpu().numpy()))


def test_noalloc_feature_and_per_pair_paths():
    # bf16 features on the matrix cores, then a batch with whole stages per pair
    c = workloads.random_case(74, 1, 8192, 1000, 64, dtype="bf16", spread=0.25)
    _compare(c, [0.5, 0.05], [3, 4])
    # whole stages split over 16-row work-groups, at the largest batch of
    # 1024-point clouds that launch takes (two pairs on half of 256 compute units)
    c = workloads.random_case(77, 2, 1000, 1024, 3, weights="dirichlet")
    _compare(c, [0.1, 0.02], [3, 5])
    c = workloads.random_case(75, 256, 130, 140, 3, weights="dirichlet")
    _compare(c, [0.1, 0.02], [2, 4])
    c = workloads.random_case(76, 1, 64, 70, 3)
    _compare(c, [0.05], [3])


def test_noalloc_rejects_sizes_beyond_the_scratch():
    # 256 pairs of 2048 x 2048 points need more than the static scratch holds
    B, n, m = 256, 2048, 2048
    need = sk.workspace_bytes(sk.SK_OP_POTENTIALS, B, n, m, 3, sk.SK_F32)
    assert need > sk.SK_NOALLOC_SCRATCH_BYTES
    d0 = torch.device("cuda:0")
    X = torch.zeros(B, n, 3, device=d0)
    Y = torch.zeros(B, m, 3, device=d0)
    out = (torch.full((B, n), 7.0, device=d0), torch.full((B, m), 7.0, device=d0), None)
    with pytest.raises(sk.SinkhornError) as e:
        sk.potentials_noalloc(X, Y, None, None, [0.1], [1], out)
    assert e.value.status == sk.SK_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out[0] == 7.0).all()) and bool((out[1] == 7.0).all())
