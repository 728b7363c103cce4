"""Host-side checks of the C ABI that need no GPU.

Argument validation runs before any HIP call, so every call here returns an
error code without touching a device; output buffers are host sentinels that
must come back unchanged.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import sinkhorn_point_cloud_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkhorn.h")
PROBE_HEADER = os.path.join(ROOT, "include", "sinkhorn_probe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sk.library_path()):
        pytest.fail("libsinkhorn_amd.so not built: run __graft_entry__.build()")
    return sk.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sinkhorn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("sinkhorn_potentials", "sinkhorn_plan_coo", "sinkhorn_loss_grad"):
        assert required in names
    assert set(names) == set(sk.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {sk.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings(lib):
    for code in range(6):
        assert lib.sinkhorn_status_string(code)
    assert lib.sinkhorn_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    ws = lib.sinkhorn_workspace_bytes
    for op in (0, 1, 2, 3, 4):
        assert ws(op, 1, 1024, 1024, 3, 0) > 0
        assert ws(op, 2, 1024, 1024, 3, 0) > ws(op, 1, 1024, 1024, 3, 0)
        assert ws(op, 1, 4096, 1024, 3, 0) > ws(op, 1, 1024, 1024, 3, 0)
    assert ws(0, 1, 65536, 65536, 3, 0) < 64 << 20     # O((n + m)), nothing n x m
    assert ws(0, 1, 50000, 60000, 64, 1) > 0
    assert ws(0, 1, 10, 10, 3, 1) > 0                  # bf16 d=3: feature kernel
    assert ws(0, 1, 10, 10, 200, 0) == 0               # d > 128: no kernel
    assert ws(0, 0, 10, 10, 3, 0) == 0
    assert ws(5, 1, 10, 10, 3, 0) == 0
    assert ws(3, 1, 65536, 65536, 3, 0) < 6 << 20      # fp64 log weights and keys, O(n + m)
    assert ws(0, 1, 1 << 25, 10, 3, 0) == 0
    assert ws(0, 65535, 4, 4, 3, 0) > 0 and ws(0, 65536, 4, 4, 3, 0) == 0


DUMMY = ctypes.c_void_p(16)   # never dereferenced: validation fails first


def _host(arr):
    return arr.ctypes.data_as(ctypes.c_void_p)


def _pot(lib, X=DUMMY, Y=DUMMY, dtype=0, B=1, n=8, m=9, d=3, eps=(0.1,), iters=(3,),
         flags=0, cost=None, ws=DUMMY, ws_bytes=1 << 40, f=None, g=None):
    e = (ctypes.c_float * max(1, len(eps)))(*eps)
    it = (ctypes.c_int * max(1, len(iters)))(*iters)
    return lib.sinkhorn_potentials(X, Y, dtype, None, None, B, n, m, d, e, it, len(eps), flags,
                                   f if f is not None else DUMMY, g if g is not None else DUMMY,
                                   cost, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), sk.SK_ERR_INVALID_ARG),
    (dict(B=0), sk.SK_ERR_INVALID_ARG),
    (dict(B=65536, n=4, m=4), sk.SK_ERR_INVALID_ARG),   # pairs index a grid dimension
    (dict(n=0), sk.SK_ERR_INVALID_ARG),
    (dict(m=-1), sk.SK_ERR_INVALID_ARG),
    (dict(dtype=7), sk.SK_ERR_INVALID_ARG),
    (dict(eps=(0.0,)), sk.SK_ERR_INVALID_ARG),
    (dict(eps=(float("nan"),)), sk.SK_ERR_INVALID_ARG),
    (dict(eps=(0.1, float("inf")), iters=(1, 1)), sk.SK_ERR_INVALID_ARG),
    (dict(iters=(-1,)), sk.SK_ERR_INVALID_ARG),
    (dict(flags=4), sk.SK_ERR_INVALID_ARG),
    (dict(eps=(), iters=(), cost=DUMMY), sk.SK_ERR_INVALID_ARG),
    (dict(dtype=1, d=200), sk.SK_ERR_UNSUPPORTED),
    (dict(d=129), sk.SK_ERR_UNSUPPORTED),
    (dict(ws=None), sk.SK_ERR_WORKSPACE),
    (dict(ws_bytes=100), sk.SK_ERR_WORKSPACE),
])
def test_potentials_rejects_bad_arguments_without_writing(lib, kw, code):
    f = np.full(8, 123.0, dtype=np.float32)
    g = np.full(9, 456.0, dtype=np.float32)
    rc = _pot(lib, f=_host(f), g=_host(g), **kw)
    assert rc == code, lib.sinkhorn_last_error()
    assert lib.sinkhorn_last_error()
    assert np.all(f == 123.0) and np.all(g == 456.0)


def _coo(lib, eps=0.1, thr=1e-8, capacity=10, rows=DUMMY, offs=DUMMY, nnz=True, ws_bytes=1 << 40):
    n_out = ctypes.c_int64(-7)
    rc = lib.sinkhorn_plan_coo(DUMMY, DUMMY, 0, None, None, 1, 8, 9, 3, eps, DUMMY, DUMMY, thr,
                               capacity, rows, DUMMY, DUMMY, offs, None, None,
                               ctypes.byref(n_out) if nnz else None, DUMMY, ws_bytes, None)
    return rc, n_out.value


def _coo_async(lib, eps=0.1, thr=1e-8, capacity=10, rows=DUMMY, nnz=DUMMY):
    return lib.sinkhorn_plan_coo_async(DUMMY, DUMMY, 0, None, None, 1, 8, 9, 3, eps, DUMMY, DUMMY,
                                       thr, capacity, rows, DUMMY, DUMMY, DUMMY, None, None, nnz,
                                       DUMMY, 1 << 40, None)


@pytest.mark.parametrize("kw", [dict(eps=0.0), dict(thr=2.0), dict(capacity=0),
                                dict(capacity=-3), dict(rows=None), dict(nnz=None)])
def test_plan_coo_async_rejects_bad_arguments(lib, kw):
    assert _coo_async(lib, **kw) == sk.SK_ERR_INVALID_ARG, lib.sinkhorn_last_error()


@pytest.mark.parametrize("kw", [dict(eps=0.0), dict(eps=-1.0), dict(thr=0.0), dict(thr=1.5),
                                dict(capacity=-1), dict(rows=None), dict(offs=None),
                                dict(nnz=False)])
def test_plan_coo_rejects_bad_arguments(lib, kw):
    rc, n_out = _coo(lib, **kw)
    assert rc == sk.SK_ERR_INVALID_ARG
    assert n_out == -7


def test_plan_coo_workspace_check(lib):
    rc, _ = _coo(lib, ws_bytes=10)
    assert rc == sk.SK_ERR_WORKSPACE


def test_loss_grad_rejects_bad_arguments(lib):
    loss = np.full(1, 5.0, dtype=np.float32)
    rc = lib.sinkhorn_loss_grad(DUMMY, DUMMY, 0, 1, 8, 9, 3, None, DUMMY, DUMMY, DUMMY,
                                _host(loss), None, DUMMY, 1 << 40, None)
    assert rc == sk.SK_ERR_INVALID_ARG
    rc = lib.sinkhorn_loss_grad(DUMMY, DUMMY, 0, 1, 8, 9, 3, DUMMY, DUMMY, DUMMY, DUMMY,
                                _host(loss), None, DUMMY, 8, None)
    assert rc == sk.SK_ERR_WORKSPACE
    assert loss[0] == 5.0


def _dgrad(lib, eps=0.1, f=DUMMY, g=DUMMY, d=3, ws=DUMMY, ws_bytes=1 << 40, out=DUMMY):
    return lib.sinkhorn_dense_grad(DUMMY, DUMMY, 0, None, None, 1, 8, 9, d, eps, f, g, out,
                                   None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(eps=0.0), sk.SK_ERR_INVALID_ARG),
    (dict(eps=float("inf")), sk.SK_ERR_INVALID_ARG),
    (dict(f=None), sk.SK_ERR_INVALID_ARG),
    (dict(g=None), sk.SK_ERR_INVALID_ARG),
    (dict(d=129), sk.SK_ERR_UNSUPPORTED),
    (dict(ws=None), sk.SK_ERR_WORKSPACE),
    (dict(ws_bytes=64), sk.SK_ERR_WORKSPACE),
])
def test_dense_grad_rejects_bad_arguments_without_writing(lib, kw, code):
    dX = np.full(8 * 3, 7.0, dtype=np.float32)
    rc = _dgrad(lib, out=_host(dX), **kw)
    assert rc == code, lib.sinkhorn_last_error()
    assert np.all(dX == 7.0)


@pytest.mark.parametrize("kw", [dict(X=None), dict(dtype=3), dict(B=0), dict(d=0), dict(d=5000),
                                dict(out=None)])
def test_normalize_rejects_bad_arguments_without_writing(lib, kw):
    args = dict(X=DUMMY, dtype=0, B=1, n=4, d=3, out=True)
    args.update(kw)
    xh = np.full(12, 3.0, dtype=np.float32)
    nr = np.full(4, 3.0, dtype=np.float32)
    rc = lib.sinkhorn_normalize(args["X"], args["dtype"], args["B"], args["n"], args["d"],
                                _host(xh) if args["out"] else None, _host(nr), None)
    assert rc == sk.SK_ERR_INVALID_ARG, lib.sinkhorn_last_error()
    assert np.all(xh == 3.0) and np.all(nr == 3.0)
    rc = lib.sinkhorn_normalize_backward(DUMMY, DUMMY, None, 1, 4, 3, _host(xh), None)
    assert rc == sk.SK_ERR_INVALID_ARG and np.all(xh == 3.0)


def test_hvp_rejects_bad_arguments_without_writing(lib):
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 3, 0) > 0
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 17, 0) == 0     # d > 16
    hv = np.full(8 * 3, 2.0, dtype=np.float32)
    for kw, code in ((dict(d=17), sk.SK_ERR_UNSUPPORTED), (dict(eps=0.0), sk.SK_ERR_INVALID_ARG),
                     (dict(it=-1), sk.SK_ERR_INVALID_ARG), (dict(V=None), sk.SK_ERR_INVALID_ARG),
                     (dict(ws=None), sk.SK_ERR_WORKSPACE)):
        a = dict(d=3, eps=0.1, it=10, V=DUMMY, ws=DUMMY)
        a.update(kw)
        rc = lib.sinkhorn_hvp(DUMMY, DUMMY, 0, None, None, 1, 8, 9, a["d"], a["eps"], DUMMY, DUMMY,
                              a["V"], a["it"], _host(hv), None, a["ws"], 1 << 40, None)
        assert rc == code, (kw, lib.sinkhorn_last_error())
    assert np.all(hv == 2.0)


def test_hvp_matrix_core_shapes_and_alignment(lib):
    # bf16 with d = 32 or 64 runs on the matrix cores; other d > 16 stay unsupported
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 64, 1) > 0
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 32, 1) > 0
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 64, 0) == 0
    assert lib.sinkhorn_workspace_bytes(4, 1, 100, 90, 48, 1) == 0
    hv = np.full(8 * 64, 2.0, dtype=np.float32)
    odd = ctypes.c_void_p(24)   # 8 mod 16
    for X, Y, d, code in ((odd, DUMMY, 64, sk.SK_ERR_INVALID_ARG),
                          (DUMMY, odd, 32, sk.SK_ERR_INVALID_ARG),
                          (DUMMY, DUMMY, 48, sk.SK_ERR_UNSUPPORTED)):
        rc = lib.sinkhorn_hvp(X, Y, 1, None, None, 1, 8, 9, d, 0.1, DUMMY, DUMMY, DUMMY, 10,
                              _host(hv), None, DUMMY, 1 << 40, None)
        assert rc == code, (d, lib.sinkhorn_last_error())
    assert np.all(hv == 2.0)


def test_coo_normalize_rejects_bad_arguments(lib):
    assert lib.sinkhorn_coo_workspace_bytes(2, 100, 90, 5000) > 5000 * 8   # two logs per entry
    assert lib.sinkhorn_coo_workspace_bytes(0, 100, 90, 5000) == 0
    assert lib.sinkhorn_coo_workspace_bytes(1, 100, 90, -1) == 0
    for B, n, m, it, null in ((0, 4, 4, 1, False), (1, 0, 4, 1, False), (1, 4, 4, -1, False),
                              (1, 4, 4, 1, True)):
        rc = lib.sinkhorn_coo_normalize(B, n, m, DUMMY, DUMMY, None if null else DUMMY, DUMMY,
                                        DUMMY, DUMMY, DUMMY, DUMMY, None, None, it, None, DUMMY,
                                        1 << 40, None)
        assert rc == sk.SK_ERR_INVALID_ARG, lib.sinkhorn_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    X = torch.zeros(1, 4, 3)
    with pytest.raises(ValueError):
        sk.potentials(X, X)


def test_product_package_does_not_reach_the_oracle():
    pkg = os.path.dirname(sk.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"\b(import|from)\s+oracle|liboracle|sinkhorn_oracle",
                                     text), fn
    out = os.popen(f"ldd {sk.library_path()}").read()
    assert "oracle" not in out


def test_noalloc_potentials_rejects_before_any_device_call(lib):
    # argument checks and the scratch limit come before the first HIP call
    f = np.full(8, 123.0, dtype=np.float32)
    g = np.full(9, 456.0, dtype=np.float32)
    e = (ctypes.c_float * 1)(0.1)
    it = (ctypes.c_int * 1)(3)

    def call(B=1, n=8, m=9, d=3, dtype=0, X=DUMMY, flags=0):
        return lib.sinkhorn_potentials_noalloc(X, DUMMY, dtype, None, None, B, n, m, d, e, it,
                                               1, flags, _host(f), _host(g), None, None)

    assert call(X=None) == sk.SK_ERR_INVALID_ARG
    assert call(flags=8) == sk.SK_ERR_INVALID_ARG
    assert call(d=129) == sk.SK_ERR_UNSUPPORTED
    # 256 pairs of 2048 x 2048: more workspace than the static scratch holds
    assert lib.sinkhorn_workspace_bytes(0, 256, 2048, 2048, 3, 0) > sk.SK_NOALLOC_SCRATCH_BYTES
    assert call(B=256, n=2048, m=2048) == sk.SK_ERR_WORKSPACE
    assert b"static scratch" in lib.sinkhorn_last_error()
    # one pair of 65536 x 65536 fits
    assert lib.sinkhorn_workspace_bytes(0, 1, 65536, 65536, 3, 0) <= sk.SK_NOALLOC_SCRATCH_BYTES
    assert np.all(f == 123.0) and np.all(g == 456.0)


def test_header_states_the_noalloc_scratch_size():
    text = open(HEADER).read()
    assert "#define SK_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)" in text
    assert sk.SK_NOALLOC_SCRATCH_BYTES == 96 << 20


def test_out_buffer_checks_refuse_what_the_abi_would_misuse():
    # the binding checks every caller-provided output before its pointer reaches
    # the C ABI: dtype, exact shape, contiguous layout, device
    import torch
    cpu = torch.device("cpu")
    good = torch.zeros(2, 5, dtype=torch.float32)
    sk._check_out(((good, (2, 5)), (None, (3,))), torch.float32, cpu, "out")
    bad = [torch.zeros(2, 5, dtype=torch.float64),             # dtype
           torch.zeros(2, 6, dtype=torch.float32),             # shape
           torch.zeros(10, dtype=torch.float32),               # same size, wrong shape
           torch.zeros(5, 2, dtype=torch.float32).t(),         # strided
           ]
    for t in bad:
        with pytest.raises(ValueError):
            sk._check_out(((t, (2, 5)),), torch.float32, cpu, "out")
    with pytest.raises(TypeError):
        sk._check_out(((np.zeros((2, 5), np.float32), (2, 5)),), torch.float32, cpu, "out")
    with pytest.raises(ValueError):   # wrong device
        sk._check_out(((good, (2, 5)),), torch.float32, torch.device("meta"), "out")


def test_plan_buffer_checks():
    import torch
    cpu = torch.device("cpu")
    i32 = lambda k: torch.zeros(k, dtype=torch.int32)
    f32 = lambda k: torch.zeros(k, dtype=torch.float32)
    i64 = lambda k: torch.zeros(k, dtype=torch.int64)
    sk._check_plan_out(i32(10), i32(10), f32(10), i64(3), 2, cpu)
    for args in ((i32(10), i32(9), f32(10), i64(3)),        # cols shorter than rows
                 (i32(10), i32(10), f32(8), i64(3)),        # vals shorter
                 (i32(10), i32(10), f32(10), i64(2)),       # offsets not B + 1
                 (i32(10), i64(10), f32(10), i64(3)),       # cols int64
                 (i32(10), i32(10), i32(10), i64(3)),       # vals int32
                 (i32(10), i32(10), f32(20)[::2], i64(3))):  # strided vals
        with pytest.raises(ValueError):
            sk._check_plan_out(*args, 2, cpu)


def test_rate_probe_is_declared_exported_and_checks_arguments(lib):
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = re.findall(r"\b(sinkhorn_\w+)\s*\(", text)
    assert names == ["sinkhorn_probe_rates", "sinkhorn_probe_wait_limit",
                     "sinkhorn_probe_potentials_path"]
    out = os.popen(f"nm -D --defined-only {sk.library_path()}").read()
    for name in names:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name
    f = lib.sinkhorn_probe_rates
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    hz = ctypes.c_double(0.0)
    # argument checks come before any device call
    assert f(9, 8, 10, DUMMY, DUMMY, ctypes.byref(hz), None) == 1
    assert f(-1, 8, 10, DUMMY, DUMMY, ctypes.byref(hz), None) == 1
    assert f(0, 0, 10, DUMMY, DUMMY, ctypes.byref(hz), None) == 1
    assert f(0, 8, 0, DUMMY, DUMMY, ctypes.byref(hz), None) == 1
    assert f(0, 8, 10, None, DUMMY, ctypes.byref(hz), None) == 1
    assert f(0, 8, 10, DUMMY, DUMMY, None, None) == 1


def test_launch_shape_query_refuses_what_potentials_refuses(lib):
    # sizes, dtypes and dimensions that sinkhorn_potentials refuses give -1; the
    # feature path needs no device to be named (4); the d = 3 shapes depend on
    # the device's compute units, and without a device the query says so (-2)
    f = lib.sinkhorn_probe_potentials_path
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_uint]
    f.restype = ctypes.c_int
    assert f(0, 10, 10, 3, sk.SK_F32, 0) == -1
    assert f(1, 0, 10, 3, sk.SK_F32, 0) == -1
    assert f(1, 10, 10, 3, 7, 0) == -1
    assert f(1, 10, 10, 200, sk.SK_F32, 0) == -1
    assert f(65536, 10, 10, 3, sk.SK_F32, 0) == -1
    assert f(2, 300, 257, 64, sk.SK_BF16, 0) == 4
    assert f(1, 1024, 1024, 3, sk.SK_F32, 0) == -2
