"""Streaming log-domain Sinkhorn for point clouds on MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libsinkhorn_amd.so`` (declared in
``include/sinkhorn.h``).  Every step of the computation runs in the library's
HIP kernels; this module only checks tensors, allocates outputs and workspace
with torch (device memory and the current stream are all torch provides) and
marshals pointers.  If the library has not been built, every call raises.

Entry points (same names as the C ABI):
  potentials(X, Y, a, b, eps, iters, ...)   -> f, g, cost
  plan_coo(X, Y, a, b, f, g, eps, ...)      -> rows, cols, vals, pair_offsets
  loss_grad(X, Y, rows, cols, vals, pair_offsets, ...) -> loss, dX
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["SinkhornError", "potentials", "potentials_noalloc", "plan_coo", "loss_grad",
           "workspace_bytes",
           "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsinkhorn_amd.so")

SK_OK, SK_ERR_INVALID_ARG, SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE, SK_ERR_CAPACITY, SK_ERR_HIP = \
    range(6)
SK_F32, SK_BF16 = 0, 1
SK_OP_POTENTIALS, SK_OP_PLAN_COO, SK_OP_LOSS_GRAD, SK_OP_DENSE_GRAD, SK_OP_HVP = range(5)
SK_WARM_START = 1
SK_VALU_SCORES = 2
SK_NOALLOC_SCRATCH_BYTES = 96 << 20   # the static scratch of sinkhorn_potentials_noalloc

EXPORTS = ("sinkhorn_workspace_bytes", "sinkhorn_potentials", "sinkhorn_potentials_noalloc",
           "sinkhorn_plan_coo",
           "sinkhorn_loss_grad", "sinkhorn_dense_grad", "sinkhorn_hvp",
           "sinkhorn_coo_workspace_bytes",
           "sinkhorn_coo_normalize", "sinkhorn_normalize", "sinkhorn_plan_coo_async",
           "sinkhorn_normalize_backward", "sinkhorn_status_string", "sinkhorn_last_error")


class SinkhornError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load (once) and return the ctypes handle; raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m sinkhorn_point_cloud_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, U, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    F, L = ctypes.c_float, ctypes.c_int64
    lib.sinkhorn_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.sinkhorn_workspace_bytes.restype = Z
    lib.sinkhorn_potentials.argtypes = [P, P, I, P, P, I, I, I, I, P, P, I, U, P, P, P, P, Z, P]
    lib.sinkhorn_potentials.restype = I
    lib.sinkhorn_potentials_noalloc.argtypes = [P, P, I, P, P, I, I, I, I, P, P, I, U, P, P, P, P]
    lib.sinkhorn_potentials_noalloc.restype = I
    lib.sinkhorn_plan_coo.argtypes = [P, P, I, P, P, I, I, I, I, F, P, P, F, L, P, P, P, P, P,
                                      P, P, P, Z, P]
    lib.sinkhorn_plan_coo.restype = I
    lib.sinkhorn_plan_coo_async.argtypes = [P, P, I, P, P, I, I, I, I, F, P, P, F, L, P, P, P, P,
                                            P, P, P, P, Z, P]
    lib.sinkhorn_plan_coo_async.restype = I
    lib.sinkhorn_loss_grad.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P, P, Z, P]
    lib.sinkhorn_loss_grad.restype = I
    lib.sinkhorn_dense_grad.argtypes = [P, P, I, P, P, I, I, I, I, F, P, P, P, P, P, P, P, Z, P]
    lib.sinkhorn_dense_grad.restype = I
    lib.sinkhorn_hvp.argtypes = [P, P, I, P, P, I, I, I, I, F, P, P, P, I, P, P, P, Z, P]
    lib.sinkhorn_hvp.restype = I
    lib.sinkhorn_coo_workspace_bytes.argtypes = [I, I, I, L]
    lib.sinkhorn_coo_workspace_bytes.restype = Z
    lib.sinkhorn_coo_normalize.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, P, I, P, P, Z, P]
    lib.sinkhorn_coo_normalize.restype = I
    lib.sinkhorn_normalize.argtypes = [P, I, I, I, I, P, P, P]
    lib.sinkhorn_normalize.restype = I
    lib.sinkhorn_normalize_backward.argtypes = [P, P, P, I, I, I, P, P]
    lib.sinkhorn_normalize_backward.restype = I
    lib.sinkhorn_status_string.argtypes = [I]
    lib.sinkhorn_status_string.restype = ctypes.c_char_p
    lib.sinkhorn_last_error.argtypes = []
    lib.sinkhorn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SK_OK:
        lib = load_library()
        msg = lib.sinkhorn_last_error().decode() or lib.sinkhorn_status_string(rc).decode()
        raise SinkhornError(rc, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _points(X, Y):
    if X.dim() == 2:
        X = X.unsqueeze(0)
    if Y.dim() == 2:
        Y = Y.unsqueeze(0)
    if X.dim() != 3 or Y.dim() != 3 or X.shape[0] != Y.shape[0] or X.shape[2] != Y.shape[2]:
        raise ValueError(f"X {tuple(X.shape)} and Y {tuple(Y.shape)} must be [B,n,d], [B,m,d]")
    if X.dtype != Y.dtype or X.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("X and Y must both be float32 or both bfloat16")
    if not (X.is_cuda and Y.is_cuda):
        raise ValueError("X and Y must be GPU tensors")
    dt = SK_F32 if X.dtype == torch.float32 else SK_BF16
    return X.contiguous(), Y.contiguous(), dt


def _weights(w, B, k, device):
    if w is None:
        return None
    w = torch.as_tensor(w, dtype=torch.float32, device=device)
    if w.numel() != B * k:
        raise ValueError(f"weights need {B * k} entries, got {w.numel()}")
    return w.reshape(B, k).contiguous()


def _check_out(items, dtype, device, what):
    """Refuses caller-provided output tensors that the C ABI would write out of
    bounds or with the wrong layout: each (tensor or None, shape) must have that
    exact shape, the dtype, C-contiguous layout and the device."""
    for t, shape in items:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}: expected a tensor, got {type(t).__name__}")
        if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
                or t.device != device:
            raise ValueError(f"{what}: need a contiguous {dtype} tensor of shape {tuple(shape)} "
                             f"on {device}, got {t.dtype} {tuple(t.shape)} "
                             f"{'contiguous' if t.is_contiguous() else 'strided'} on {t.device}")


def _check_plan_out(rows, cols, vals, offs, B, device):
    """A sparse plan's buffers: rows, cols int32 and vals float32 of one common
    length (the capacity), offs int64 of B + 1 entries, all contiguous on device."""
    for t in (rows, cols, vals, offs):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"plan buffers must be tensors, got {type(t).__name__}")
    cap = rows.numel()
    _check_out(((rows, (cap,)), (cols, (cap,))), torch.int32, device, "plan rows/cols")
    _check_out(((vals, (cap,)),), torch.float32, device, "plan vals")
    _check_out(((offs, (B + 1,)),), torch.int64, device, "plan pair_offsets")


def workspace_bytes(op: int, B: int, n: int, m: int, d: int, dtype: int) -> int:
    return int(load_library().sinkhorn_workspace_bytes(op, B, n, m, d, dtype))


def _workspace(op, B, n, m, d, dt, device, workspace=None):
    need = workspace_bytes(op, B, n, m, d, dt)
    if need == 0:
        raise SinkhornError(SK_ERR_UNSUPPORTED, f"unsupported shape/dtype B={B} n={n} m={m} d={d}")
    if workspace is not None and workspace.numel() >= need:
        return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


def potentials(X, Y, a=None, b=None, eps=(0.05,), iters=(100,), f0=None, g0=None,
               cost: bool = True, out=None, workspace=None, valu_scores: bool = False):
    """Sinkhorn potentials over an eps schedule (one stage per entry of eps/iters).

    X [B,n,d], Y [B,m,d] (float32, or bfloat16), a [B,n], b [B,m] or None
    (uniform).  f0/g0 warm-start the run.  Returns (f [B,n], g [B,m], cost [B] or
    None), all float32 on the device.  ``out`` = (f, g, cost) reuses buffers.
    ``valu_scores`` forms the d = 3 scores on the vector ALUs instead of the
    matrix cores."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    eps_l = [float(e) for e in (eps if hasattr(eps, "__len__") else [eps])]
    it_l = [int(i) for i in (iters if hasattr(iters, "__len__") else [iters])]
    if len(eps_l) != len(it_l):
        raise ValueError("eps and iters need one entry per stage")
    if out is not None:
        f, g, c = out
        if f is None or g is None:
            raise ValueError("out needs f and g tensors")
        _check_out(((f, (B, n)), (g, (B, m)), (c, (B,))), torch.float32, dev, "out")
    else:
        f = torch.empty(B, n, dtype=torch.float32, device=dev)
        g = torch.empty(B, m, dtype=torch.float32, device=dev)
        c = torch.empty(B, dtype=torch.float32, device=dev) if cost else None
    flags = SK_VALU_SCORES if valu_scores else 0
    if (f0 is None) != (g0 is None):
        raise ValueError("warm start needs both f0 and g0")
    if f0 is not None:
        f.copy_(torch.as_tensor(f0, device=dev).reshape(B, n))
        g.copy_(torch.as_tensor(g0, device=dev).reshape(B, m))
        flags |= SK_WARM_START
    ws = _workspace(SK_OP_POTENTIALS, B, n, m, d, dt, dev, workspace)
    eps_a = (ctypes.c_float * max(1, len(eps_l)))(*eps_l)
    it_a = (ctypes.c_int * max(1, len(it_l)))(*it_l)
    rc = lib.sinkhorn_potentials(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d, eps_a, it_a,
                                 len(eps_l), flags, _ptr(f), _ptr(g), _ptr(c), _ptr(ws),
                                 ws.numel(), _stream())
    _check(rc)
    return f, g, c


def potentials_noalloc(X, Y, a, b, eps, iters, out, warm_start: bool = False,
                       valu_scores: bool = False):
    """Sinkhorn potentials through sinkhorn_potentials_noalloc: no workspace, nothing
    allocated.  ``out`` = (f [B,n], g [B,m], cost [B] or None), float32 contiguous
    tensors on X's device; with ``warm_start`` f and g hold the starting potentials.
    X, Y, a and b must already be contiguous (float32 weights of [B,n], [B,m] or
    None), so that no copy is made.  Returns ``out``."""
    lib = load_library()
    if X.dim() != 3 or Y.dim() != 3 or not (X.is_contiguous() and Y.is_contiguous()):
        raise ValueError("X and Y must be contiguous [B,n,d] and [B,m,d] tensors")
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    for w, k, name in ((a, n, "a"), (b, m, "b")):
        if w is not None and (w.dtype != torch.float32 or w.numel() != B * k
                              or not w.is_contiguous() or w.device != dev):
            raise ValueError(f"{name} must be a contiguous float32 tensor of {B * k} entries "
                             f"on {dev}")
    f, g, c = out
    _check_out(((f, (B, n)), (g, (B, m)), (c, (B,))), torch.float32, dev, "out")
    if f is None or g is None:
        raise ValueError("out needs f and g")
    eps_l = [float(e) for e in (eps if hasattr(eps, "__len__") else [eps])]
    it_l = [int(i) for i in (iters if hasattr(iters, "__len__") else [iters])]
    if len(eps_l) != len(it_l):
        raise ValueError("eps and iters need one entry per stage")
    flags = (SK_WARM_START if warm_start else 0) | (SK_VALU_SCORES if valu_scores else 0)
    eps_a = (ctypes.c_float * max(1, len(eps_l)))(*eps_l)
    it_a = (ctypes.c_int * max(1, len(it_l)))(*it_l)
    _check(lib.sinkhorn_potentials_noalloc(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d,
                                           eps_a, it_a, len(eps_l), flags, _ptr(f), _ptr(g),
                                           _ptr(c), _stream()))
    return out


def plan_coo(X, Y, a, b, f, g, eps: float, rel_threshold: float = 1e-8, capacity=None,
             workspace=None, out=None, loss_out=None):
    """Thresholded sparse plan: (rows int32, cols int32, vals float32, pair_offsets int64[B+1]).

    With capacity=None the plan is counted first, then emitted into buffers of
    exactly the right size (two calls of the C entry point).  ``out`` = (rows,
    cols, vals, pair_offsets) reuses buffers; its length is the capacity, and
    a plan that does not fit raises SinkhornError(SK_ERR_CAPACITY).
    ``loss_out`` = (loss [B], dX [B,n,d]) float32 tensors (either may be None)
    receive the loss on the emitted support and its gradient in X, computed
    during the emission."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    f = f.reshape(B, n).contiguous().float()
    g = g.reshape(B, m).contiguous().float()
    ws = _workspace(SK_OP_PLAN_COO, B, n, m, d, dt, dev, workspace)
    loss, dX = loss_out if loss_out is not None else (None, None)
    _check_out(((loss, (B,)), (dX, (B, n, d))), torch.float32, dev, "loss_out")
    nnz = ctypes.c_int64(0)
    if out is not None:
        rows, cols, vals, offs = out
        _check_plan_out(rows, cols, vals, offs, B, dev)
        cap = rows.numel()
    else:
        offs = torch.empty(B + 1, dtype=torch.int64, device=dev)
        cap = 0 if capacity is None else int(capacity)
        rows = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        cols = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        vals = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)

    def call(cap, rows, cols, vals):
        return lib.sinkhorn_plan_coo(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d,
                                     float(eps), _ptr(f), _ptr(g), float(rel_threshold), cap,
                                     _ptr(rows), _ptr(cols), _ptr(vals), _ptr(offs), _ptr(loss),
                                     _ptr(dX), ctypes.byref(nnz), _ptr(ws), ws.numel(), _stream())

    rc = call(cap, rows, cols, vals)
    if rc == SK_ERR_CAPACITY and capacity is None and out is None:
        cap = int(nnz.value)
        rows = torch.empty(cap, dtype=torch.int32, device=dev)
        cols = torch.empty(cap, dtype=torch.int32, device=dev)
        vals = torch.empty(cap, dtype=torch.float32, device=dev)
        rc = call(cap, rows, cols, vals)
    _check(rc)
    k = int(nnz.value)
    return rows[:k], cols[:k], vals[:k], offs


def plan_coo_async(X, Y, a, b, f, g, eps: float, rel_threshold: float, out, loss_out=None,
                   workspace=None, nnz=None):
    """The thresholded plan into ``out`` = (rows, cols, vals, pair_offsets) without
    waiting on the stream (capturable).  Returns ``nnz`` (int64 [1] on the device): the
    number of kept entries.  If it exceeds len(rows), only pair_offsets and nnz are
    written, so check nnz <= len(rows) before using rows/cols/vals or ``loss_out``."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    f = f.reshape(B, n).contiguous().float()
    g = g.reshape(B, m).contiguous().float()
    ws = _workspace(SK_OP_PLAN_COO, B, n, m, d, dt, dev, workspace)
    loss, dX = loss_out if loss_out is not None else (None, None)
    _check_out(((loss, (B,)), (dX, (B, n, d))), torch.float32, dev, "loss_out")
    rows, cols, vals, offs = out
    _check_plan_out(rows, cols, vals, offs, B, dev)
    if rows.numel() < 1:
        raise ValueError("out needs a capacity of at least one entry")
    if nnz is None:
        nnz = torch.empty(1, dtype=torch.int64, device=dev)
    _check_out(((nnz, (1,)),), torch.int64, dev, "nnz")
    rc = lib.sinkhorn_plan_coo_async(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d,
                                     float(eps), _ptr(f), _ptr(g), float(rel_threshold),
                                     rows.numel(), _ptr(rows), _ptr(cols), _ptr(vals), _ptr(offs),
                                     _ptr(loss), _ptr(dX), _ptr(nnz), _ptr(ws), ws.numel(),
                                     _stream())
    _check(rc)
    return nnz


def loss_grad(X, Y, rows, cols, vals, pair_offsets, grad: bool = True, workspace=None,
              out=None):
    """Loss [B] and dL/dX [B,n,d] (float32) on the stored support of a row-sorted COO plan.
    ``out`` = (loss, dX) reuses buffers."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    rows, cols = rows.contiguous(), cols.contiguous()
    vals, offs = vals.contiguous(), pair_offsets.contiguous()
    if rows.dtype != torch.int32 or cols.dtype != torch.int32 or vals.dtype != torch.float32 \
            or offs.dtype != torch.int64 or offs.numel() != B + 1:
        raise TypeError("rows/cols int32, vals float32, pair_offsets int64[B+1]")
    if not (rows.numel() == cols.numel() == vals.numel()):
        raise ValueError("rows, cols and vals must have the same length (the offsets index them)")
    if rows.numel() == 0:   # the C ABI wants real pointers even for an empty plan
        rows = torch.zeros(1, dtype=torch.int32, device=dev)
        cols = torch.zeros(1, dtype=torch.int32, device=dev)
        vals = torch.zeros(1, dtype=torch.float32, device=dev)
    if out is not None:
        loss, dX = out
        if loss is None:
            raise ValueError("out needs a loss tensor")
        _check_out(((loss, (B,)), (dX, (B, n, d))), torch.float32, dev, "out")
    else:
        loss = torch.empty(B, dtype=torch.float32, device=dev)
        dX = torch.empty(B, n, d, dtype=torch.float32, device=dev) if grad else None
    ws = _workspace(SK_OP_LOSS_GRAD, B, n, m, d, dt, dev, workspace)
    rc = lib.sinkhorn_loss_grad(_ptr(X), _ptr(Y), dt, B, n, m, d, _ptr(rows), _ptr(cols),
                                _ptr(vals), _ptr(offs), _ptr(loss), _ptr(dX), _ptr(ws),
                                ws.numel(), _stream())
    _check(rc)
    return loss, dX


def dense_grad(X, Y, a, b, f, g, eps: float, sides: str = "xy", workspace=None, out=None):
    """Dense transport application at eps: (dX, TX, dY, TY), float32.

    dX[p,i] = sum_j 2 P_ij (x_i - y_j), TX[p,i] = sum_j P_ij y_j / sum_j P_ij, and
    the same for the Y side; ``sides`` picks "x", "y" or "xy" (the others are
    None).  ``out`` = (dX, TX, dY, TY) reuses buffers (entries may be None)."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    f = f.reshape(B, n).contiguous().float()
    g = g.reshape(B, m).contiguous().float()
    if out is not None:
        dX, TX, dY, TY = out
        _check_out(((dX, (B, n, d)), (TX, (B, n, d)), (dY, (B, m, d)), (TY, (B, m, d))),
                   torch.float32, dev, "out")
    else:
        def new(k, on):
            return torch.empty(B, k, d, dtype=torch.float32, device=dev) if on else None
        dX, TX = new(n, "x" in sides), new(n, "x" in sides)
        dY, TY = new(m, "y" in sides), new(m, "y" in sides)
    ws = _workspace(SK_OP_DENSE_GRAD, B, n, m, d, dt, dev, workspace)
    rc = lib.sinkhorn_dense_grad(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d, float(eps),
                                 _ptr(f), _ptr(g), _ptr(dX), _ptr(TX), _ptr(dY), _ptr(TY),
                                 _ptr(ws), ws.numel(), _stream())
    _check(rc)
    return dX, TX, dY, TY


def normalize(X):
    """(Xh, norms): points of X [B,n,d] (fp32 or bf16) scaled to unit length, float32.
    With the normalised clouds every other call works under the cosine cost."""
    lib = load_library()
    if not X.is_cuda:
        raise ValueError("X must be a CUDA tensor")
    X = X.contiguous()
    if X.dim() == 2:
        X = X[None]
    dt = {torch.float32: SK_F32, torch.bfloat16: SK_BF16}.get(X.dtype)
    if dt is None:
        raise TypeError("X must be float32 or bfloat16")
    B, n, d = X.shape
    Xh = torch.empty(B, n, d, dtype=torch.float32, device=X.device)
    norms = torch.empty(B, n, dtype=torch.float32, device=X.device)
    _check(lib.sinkhorn_normalize(_ptr(X), dt, B, n, d, _ptr(Xh), _ptr(norms), _stream()))
    return Xh, norms


def normalize_backward(Xh, norms, G):
    """Gradient with respect to the raw points from G, the gradient with respect to Xh."""
    lib = load_library()
    Xh, norms, G = Xh.contiguous(), norms.contiguous(), G.contiguous().float()
    B, n, d = Xh.shape
    dX = torch.empty_like(Xh)
    _check(lib.sinkhorn_normalize_backward(_ptr(Xh), _ptr(norms), _ptr(G), B, n, d, _ptr(dX),
                                           _stream()))
    return dX


def coo_normalize(plan, transpose, a, b, n, m, iters, err=True, workspace=None):
    """Sinkhorn normalisation of a sparse plan on its support, in place.

    plan = (rows, cols, vals, pair_offsets) as plan_coo returns it; transpose =
    the plan of the exchanged clouds (plan_coo(Y, X, b, a, g, f, ...)), which
    must hold the same entries and values; both value arrays are rescaled in
    place.  Returns err [B,2] (float32: sum |row sums - a| and
    sum |column sums - b| per pair) or None."""
    lib = load_library()
    rows, cols, vals, offs = plan
    t_rows, t_cols, t_vals, t_offs = transpose
    B = offs.numel() - 1
    dev = vals.device
    # both value arrays are rewritten in place through their pointers: refuse
    # buffers of the wrong dtype, layout, device or length before the call
    _check_plan_out(rows, cols, vals, offs, B, dev)
    _check_plan_out(t_rows, t_cols, t_vals, t_offs, B, dev)
    for what, o, k in (("plan", offs, rows.numel()), ("transpose", t_offs, t_rows.numel())):
        if int(o[-1]) > k:   # this call reads the counts back anyway
            raise ValueError(f"{what}: pair_offsets end at {int(o[-1])}, beyond its {k} entries")
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    nnz = int(rows.numel())
    if workspace is None:
        workspace = torch.empty(lib.sinkhorn_coo_workspace_bytes(B, n, m, nnz), dtype=torch.uint8,
                                device=dev)
    e = torch.empty(B, 2, dtype=torch.float32, device=dev) if err else None
    one = torch.zeros(1, dtype=torch.int32, device=dev)   # real pointers for an empty plan

    def p(t):
        return _ptr(t if t.numel() else one)

    rc = lib.sinkhorn_coo_normalize(B, n, m, p(rows), p(cols), p(vals), _ptr(offs), p(t_rows),
                                    p(t_cols), p(t_vals), _ptr(t_offs), _ptr(a), _ptr(b),
                                    int(iters), _ptr(e), _ptr(workspace), workspace.numel(),
                                    _stream())
    _check(rc)
    return e


def hvp(X, Y, a, b, f, g, eps: float, V, cg_iters: int = 100, workspace=None, out=None):
    """(HV, cg_residual): Hessian-vector product of the entropic OT value in X along V
    [B,n,d] (d <= 16, or bf16 points with d = 32 or 64 on the matrix cores), at the
    plan of potentials f, g; cg_residual [B] is the final conjugate-gradient residual
    relative to the right-hand side (NaN, with HV, for a pair whose potentials are
    too far from a solution for the matrix-core path)."""
    lib = load_library()
    X, Y, dt = _points(X, Y)
    B, n, d = X.shape
    m = Y.shape[1]
    dev = X.device
    a, b = _weights(a, B, n, dev), _weights(b, B, m, dev)
    f = f.reshape(B, n).contiguous().float()
    g = g.reshape(B, m).contiguous().float()
    V = V.reshape(B, n, d).contiguous().float()
    if out is not None:
        _check_out(((out, (B, n, d)),), torch.float32, dev, "out")
    HV = out if out is not None else torch.empty(B, n, d, dtype=torch.float32, device=dev)
    res = torch.empty(B, dtype=torch.float32, device=dev)
    ws = _workspace(SK_OP_HVP, B, n, m, d, dt, dev, workspace)
    rc = lib.sinkhorn_hvp(_ptr(X), _ptr(Y), dt, _ptr(a), _ptr(b), B, n, m, d, float(eps), _ptr(f),
                          _ptr(g), _ptr(V), int(cg_iters), _ptr(HV), _ptr(res), _ptr(ws),
                          ws.numel(), _stream())
    _check(rc)
    return HV, res
