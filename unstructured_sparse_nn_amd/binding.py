"""ctypes binding of libsnack.so (include/snack.h), argument marshalling only.

Every function has the name of the C entry point it calls.  Array arguments
are torch tensors on the GPU (their ``data_ptr()`` is passed), raw integer
device addresses, or ``None`` for a NULL pointer.  The element type of values
and activations is taken from the tensors (``torch.float32`` or
``torch.bfloat16``); ``stream=None`` means torch's current stream.  A
negative status raises :class:`SnackError`.  No arithmetic of the layer
happens here: every step runs in the HIP library, and importing this module
fails loudly when that library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SNACK_LIBRARY selects another build of the same ABI, e.g. the debug build
# libsnack_debug.so (device checks of plan arrays before every product).
LIB_PATH = os.environ.get("SNACK_LIBRARY") or os.path.join(HERE, "libsnack.so")

F32, BF16 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
CONV_NHWC, CONV_NCHW = 0, 1
FIXED_COMPILE_ONLY = 1
PLAN_NODE_MAJOR_ONLY = 1
PRUNE_SORT_PLAN = 1
HOST_WORDS_BYTES = 64
STATIC_WS_MAX = 32 << 20
BATCH_MAJOR, NODE_MAJOR = 0, 1
PLAN_SLOTS = 16

ARRAYS = {"row_ptr": 0, "rpart_seg": 1, "rpart_nz": 2, "rcut": 3, "col_ptr": 4, "perm": 5,
          "row_t": 6, "cpart_seg": 7, "cpart_nz": 8, "ccut": 9}

STATUS = {0: "SNACK_OK", -1: "SNACK_E_NULL", -2: "SNACK_E_SHAPE", -3: "SNACK_E_DTYPE",
          -4: "SNACK_E_LAYOUT", -5: "SNACK_E_COO_RANGE", -6: "SNACK_E_COO_ORDER",
          -7: "SNACK_E_NAN", -8: "SNACK_E_COUNT", -9: "SNACK_E_WORKSPACE",
          -10: "SNACK_E_OVERFLOW", -11: "SNACK_E_HIP", -12: "SNACK_E_NOT_PREPARED",
          -13: "SNACK_E_PLAN_CORRUPT"}


class SnackError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_str(status)})")


FOOTPRINT_FIELDS = ("coo", "value_grad", "col_values", "derived", "plan_scratch",
                    "restructure_ws",
                    "sparse_total", "dense_weight", "dense_grad", "dense_total", "mask",
                    "masked_total", "activations")


class SnackFootprint(ctypes.Structure):
    """Mirror of ``struct snack_footprint``."""
    _fields_ = [(f, ctypes.c_uint64) for f in FOOTPRINT_FIELDS]


class SnackAdam(ctypes.Structure):
    """Mirror of ``struct snack_adam``."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("step", ctypes.c_int32)]


class SnackPlan(ctypes.Structure):
    """Mirror of ``struct snack_plan``."""
    _fields_ = [("M", ctypes.c_int32), ("K", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("max_batch", ctypes.c_int32), ("tile_row", ctypes.c_int32),
                ("tile_col", ctypes.c_int32), ("P_row", ctypes.c_int32),
                ("P_col", ctypes.c_int32), ("has_split_row", ctypes.c_int32),
                ("has_split_col", ctypes.c_int32), ("prepared", ctypes.c_int32),
                ("row", ctypes.c_void_p), ("col", ctypes.c_void_p),
                ("arena", ctypes.c_void_p), ("arena_bytes", ctypes.c_size_t),
                ("off", ctypes.c_size_t * PLAN_SLOTS), ("host_words", ctypes.c_void_p),
                ("host_words_dev", ctypes.c_void_p), ("host_words_key", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                            ctypes.c_size_t)
    plan_p = ctypes.POINTER(SnackPlan)
    sig = {
        "snack_version": ([], i32),
        "snack_plan_sizeof": ([], sz),
        "snack_status_str": ([i32], ctypes.c_char_p),
        "snack_plan_init": ([plan_p, i32, i32, i64, i32, i32, ctypes.c_uint32], i32),
        "snack_coo_prepare": ([plan_p, P, P, P, sz, P], i32),
        "snack_plan_array": ([plan_p, i32, ctypes.POINTER(i64)], P),
        "snack_spmm_fwd": ([plan_p, P, i32, P, i32, i32, P, P], i32),
        "snack_spmm_fwd_act": ([plan_p, P, i32, P, i32, i32, P, i32, P], i32),
        "snack_graph_propagate": ([plan_p, P, i32, P, i32, i32, i32, i32, P, P, P], i32),
        "snack_spmm_bwd_input": ([plan_p, P, i32, P, i32, i32, P, P], i32),
        "snack_gather_vals_t": ([plan_p, P, i32, P, P], i32),
        "snack_spmm_bwd_input_t": ([plan_p, P, i32, P, i32, i32, P, P], i32),
        "snack_sddmm_grad_vals": ([plan_p, P, P, i32, i32, i32, P, P], i32),
        "snack_spmm_bwd_fused": ([plan_p, P, P, i32, P, P, i32, i32, P, P, ctypes.c_float, P],
                                 i32),
        "snack_spmm_bwd_fused_adam": ([plan_p, P, P, i32, P, P, i32, i32, P, P, P, P,
                                       ctypes.POINTER(SnackAdam), P], i32),
        "snack_drop_count": ([i64, i32], i64),
        "snack_prune_regrow_workspace": ([i32, i32, i64, i64, ctypes.POINTER(sz)], i32),
        "snack_prune_regrow_workspace_ex": ([i32, i32, i64, i64, ctypes.c_uint32,
                                             ctypes.POINTER(sz)], i32),
        "snack_prune_regrow": ([P, P, P, i32, i32, i32, i64, i64, u64, u64, P, P, P, sz, P], i32),
        "snack_prune_regrow_ex": ([P, P, P, i32, i32, i32, i64, i64, u64, u64, P, P, P, sz,
                                   ctypes.c_uint32, P], i32),
        "snack_prune_regrow_prepared": ([plan_p, P, P, P, P, i32, i64, u64, u64, P, P, P, sz,
                                         ctypes.c_uint32, P], i32),
        "snack_prune_regrow_static": ([P, P, P, i32, i32, i32, i64, i64, u64, u64, P, P, P],
                                      i32),
        "snack_memory_footprint": ([i32, i32, i64, i32, i32, i64, ctypes.c_uint32,
                                    ctypes.POINTER(SnackFootprint)], i32),
        "snack_fixed_build": ([P, P, P, i32, i32, i32, i64, ctypes.c_uint32, ctypes.POINTER(P)],
                              i32),
        "snack_fixed_fwd": ([P, P, i32, i32, P, P], i32),
        "snack_fixed_info": ([P, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(sz),
                              ctypes.POINTER(sz)], i32),
        "snack_fixed_code": ([P, ctypes.POINTER(sz)], P),
        "snack_fixed_free": ([P], None),
        "snack_conv1x1": ([plan_p, P, i32, P, i32, i32, i32, P, P], i32),
        "snack_gelu_fwd": ([P, P, i64, P], i32),
        "snack_gelu_bwd": ([P, P, P, i64, P], i32),
        "snack_dense_fwd": ([P, P, i32, i32, i32, P, i32, P, P], i32),
        "snack_calibrate": ([i32, P, sz, i64, P], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def status_str(status: int) -> str:
    return _lib.snack_status_str(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise SnackError(status, what)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _dtype(*cands, dtype=None) -> int:
    """Element type: explicit ``dtype``, else that of the first tensor given."""
    if dtype is not None:
        return dtype
    import torch
    for t in cands:
        if t is None or isinstance(t, int):
            continue
        if t.dtype == torch.float32:
            return F32
        if t.dtype == torch.bfloat16:
            return BF16
        raise TypeError(f"unsupported dtype {t.dtype}")
    raise TypeError("no tensor to take the dtype from; pass dtype=")


def _stream(stream):
    if stream is None:  # torch's current stream, as a raw handle (no Stream object built)
        import torch
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()) or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def snack_version() -> int:
    return _lib.snack_version()


def snack_plan_sizeof() -> int:
    return _lib.snack_plan_sizeof()


def snack_plan_init(M: int, K: int, nnz: int, max_batch: int, tile_items: int = 0,
                    flags: int = 0) -> SnackPlan:
    plan = SnackPlan()
    _check(_lib.snack_plan_init(ctypes.byref(plan), M, K, nnz, max_batch, tile_items, flags),
           "snack_plan_init")
    return plan


def snack_coo_prepare(plan: SnackPlan, row, col, arena, stream=None, arena_bytes=None):
    if arena_bytes is None:
        arena_bytes = arena.numel() * arena.element_size() if arena is not None and \
            not isinstance(arena, int) else 0
    _check(_lib.snack_coo_prepare(ctypes.byref(plan), _ptr(row), _ptr(col), _ptr(arena),
                                  arena_bytes, _stream(stream)), "snack_coo_prepare")


def snack_plan_array(plan: SnackPlan, which) -> tuple:
    """(device address, element count) of a derived array; which is a name or id."""
    w = ARRAYS[which] if isinstance(which, str) else int(which)
    n = ctypes.c_int64(0)
    addr = _lib.snack_plan_array(ctypes.byref(plan), w, ctypes.byref(n))
    return addr, n.value


def snack_spmm_fwd(plan, vals, X, layout, B, Y, stream=None, dtype=None):
    dt = _dtype(vals, X, Y, dtype=dtype)
    _check(_lib.snack_spmm_fwd(ctypes.byref(plan), _ptr(vals), dt, _ptr(X), layout, B, _ptr(Y),
                               _stream(stream)), "snack_spmm_fwd")


def snack_spmm_fwd_act(plan, vals, X, layout, B, Y, act, stream=None, dtype=None):
    dt = _dtype(vals, X, Y, dtype=dtype)
    _check(_lib.snack_spmm_fwd_act(ctypes.byref(plan), _ptr(vals), dt, _ptr(X), layout, B,
                                   _ptr(Y), act, _stream(stream)), "snack_spmm_fwd_act")


def snack_graph_propagate(plan, vals, X, layout, B, layers, act, Y, tmp=None, stream=None,
                          dtype=None):
    """Y = act(...act(act(X W^T) W^T)... W^T), `layers` propagations (tmp: B*M
    elements, needed when layers > 1)."""
    dt = _dtype(vals, X, Y, dtype=dtype)
    _check(_lib.snack_graph_propagate(ctypes.byref(plan), _ptr(vals), dt, _ptr(X), layout, B,
                                      layers, act, _ptr(Y), _ptr(tmp), _stream(stream)),
           "snack_graph_propagate")


def snack_spmm_bwd_input(plan, vals, dY, layout, B, dX, stream=None, dtype=None):
    dt = _dtype(vals, dY, dX, dtype=dtype)
    _check(_lib.snack_spmm_bwd_input(ctypes.byref(plan), _ptr(vals), dt, _ptr(dY), layout, B,
                                     _ptr(dX), _stream(stream)), "snack_spmm_bwd_input")


def snack_gather_vals_t(plan, vals, vals_t, stream=None, dtype=None):
    """vals_t[i] = vals[perm[i]]: the values in the plan's column order."""
    dt = _dtype(vals, vals_t, dtype=dtype)
    _check(_lib.snack_gather_vals_t(ctypes.byref(plan), _ptr(vals), dt, _ptr(vals_t),
                                    _stream(stream)), "snack_gather_vals_t")


def snack_spmm_bwd_input_t(plan, vals_t, dY, layout, B, dX, stream=None, dtype=None):
    """dX = dY W with the values given in column order (vals_t)."""
    dt = _dtype(vals_t, dY, dX, dtype=dtype)
    _check(_lib.snack_spmm_bwd_input_t(ctypes.byref(plan), _ptr(vals_t), dt, _ptr(dY), layout,
                                       B, _ptr(dX), _stream(stream)), "snack_spmm_bwd_input_t")


def snack_sddmm_grad_vals(plan, dY, X, layout, B, dvals, stream=None, dtype=None):
    dt = _dtype(dvals, dY, X, dtype=dtype)
    _check(_lib.snack_sddmm_grad_vals(ctypes.byref(plan), _ptr(dY), _ptr(X), dt, layout, B,
                                      _ptr(dvals), _stream(stream)), "snack_sddmm_grad_vals")


def snack_spmm_bwd_fused(plan, vals, X, dY, layout, B, dX, dvals=None, lr=0.0, stream=None,
                         dtype=None, vals_t=None):
    """dX = dY W, dvals = (dY^T X) at the nonzeros, and vals -= lr * dV in place, in one pass
    (vals_t: the values in column order, read instead of vals and updated with them)."""
    dt = _dtype(vals, X, dY, dX, dtype=dtype)
    _check(_lib.snack_spmm_bwd_fused(ctypes.byref(plan), _ptr(vals), _ptr(vals_t), dt, _ptr(X),
                                     _ptr(dY), layout, B, _ptr(dX), _ptr(dvals), float(lr),
                                     _stream(stream)), "snack_spmm_bwd_fused")


def snack_spmm_bwd_fused_adam(plan, vals, X, dY, layout, B, dX, dvals, m_t, v_t, lr, step,
                              beta1=0.9, beta2=0.999, eps=1e-8, stream=None, dtype=None,
                              vals_t=None):
    """dX, dV and an Adam step on the values in one pass (moments m_t, v_t: fp32,
    column order)."""
    dt = _dtype(vals, X, dY, dX, dtype=dtype)
    hp = SnackAdam(float(lr), float(beta1), float(beta2), float(eps), int(step))
    _check(_lib.snack_spmm_bwd_fused_adam(ctypes.byref(plan), _ptr(vals), _ptr(vals_t), dt,
                                          _ptr(X), _ptr(dY), layout, B, _ptr(dX), _ptr(dvals),
                                          _ptr(m_t), _ptr(v_t), ctypes.byref(hp),
                                          _stream(stream)), "snack_spmm_bwd_fused_adam")


def snack_drop_count(nnz: int, frac_ppm: int) -> int:
    return _lib.snack_drop_count(nnz, frac_ppm)


def snack_prune_regrow_workspace(M: int, K: int, nnz: int, n_drop: int, flags: int = 0) -> int:
    """Workspace bytes of a restructure (flags: PRUNE_SORT_PLAN forces the sort plan;
    the plain entry point when flags == 0)."""
    out = ctypes.c_size_t(0)
    if flags:
        _check(_lib.snack_prune_regrow_workspace_ex(M, K, nnz, n_drop, flags, ctypes.byref(out)),
               "snack_prune_regrow_workspace_ex")
    else:
        _check(_lib.snack_prune_regrow_workspace(M, K, nnz, n_drop, ctypes.byref(out)),
               "snack_prune_regrow_workspace")
    return out.value


def _nbytes(buf, given):
    if given is not None:
        return given
    return buf.numel() * buf.element_size() if buf is not None and not isinstance(buf, int) else 0


def snack_prune_regrow(row, col, vals, M, K, nnz, n_drop, seed, step, dropped_lin, grown_lin,
                       ws, stream=None, ws_bytes=None, dtype=None, flags: int = 0):
    dt = _dtype(vals, dtype=dtype)
    ws_bytes = _nbytes(ws, ws_bytes)
    args = (_ptr(row), _ptr(col), _ptr(vals), dt, M, K, nnz, n_drop, seed & (2**64 - 1),
            step & (2**64 - 1), _ptr(dropped_lin), _ptr(grown_lin), _ptr(ws), ws_bytes)
    if flags:
        _check(_lib.snack_prune_regrow_ex(*args, flags, _stream(stream)), "snack_prune_regrow_ex")
    else:
        _check(_lib.snack_prune_regrow(*args, _stream(stream)), "snack_prune_regrow")


def snack_prune_regrow_static(row, col, vals, M, K, nnz, n_drop, seed, step, dropped_lin,
                              grown_lin, stream=None, dtype=None):
    """snack_prune_regrow with the library's per-GPU workspace array (no allocation)."""
    dt = _dtype(vals, dtype=dtype)
    _check(_lib.snack_prune_regrow_static(_ptr(row), _ptr(col), _ptr(vals), dt, M, K, nnz,
                                          n_drop, seed & (2**64 - 1), step & (2**64 - 1),
                                          _ptr(dropped_lin), _ptr(grown_lin),
                                          _stream(stream)),
           "snack_prune_regrow_static")


def snack_prune_regrow_prepared(plan, row, col, vals, n_drop, seed, step, dropped_lin, grown_lin,
                                ws, stream=None, ws_bytes=None, dtype=None, vals_t=None,
                                flags: int = 0):
    """Restructure and re-prepare in one call; vals_t (optional) receives the new
    values in the new column order."""
    dt = _dtype(vals, dtype=dtype)
    _check(_lib.snack_prune_regrow_prepared(ctypes.byref(plan), _ptr(row), _ptr(col), _ptr(vals),
                                            _ptr(vals_t), dt, n_drop, seed & (2**64 - 1),
                                            step & (2**64 - 1), _ptr(dropped_lin),
                                            _ptr(grown_lin), _ptr(ws), _nbytes(ws, ws_bytes),
                                            flags, _stream(stream)),
           "snack_prune_regrow_prepared")


def snack_memory_footprint(M: int, K: int, nnz: int, max_batch: int, dtype: int, n_drop: int = 0,
                           plan_flags: int = 0) -> dict:
    """Device bytes of the sparse layer, the dense layer and Dense+Mask (a dict
    with the fields of ``struct snack_footprint``)."""
    out = SnackFootprint()
    _check(_lib.snack_memory_footprint(M, K, nnz, max_batch, dtype, n_drop, plan_flags,
                                       ctypes.byref(out)), "snack_memory_footprint")
    return {f: int(getattr(out, f)) for f in FOOTPRINT_FIELDS}


class SnackFixed:
    """Handle of a kernel generated for one fixed weight (snack_fixed_build);
    freed with the object or by ``free()``."""

    def __init__(self, handle):
        self.handle = handle

    def info(self) -> dict:
        g, nb = ctypes.c_int32(0), ctypes.c_int32(0)
        cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(_lib.snack_fixed_info(self.handle, ctypes.byref(g), ctypes.byref(nb),
                                     ctypes.byref(cb), ctypes.byref(sb)), "snack_fixed_info")
        return {"waves": g.value, "bands": nb.value, "code_bytes": cb.value,
                "source_bytes": sb.value}

    def code(self) -> bytes:
        """The compiled code object."""
        n = ctypes.c_size_t(0)
        p = _lib.snack_fixed_code(self.handle, ctypes.byref(n))
        return ctypes.string_at(p, n.value) if p else b""

    def free(self):
        if self.handle:
            _lib.snack_fixed_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def snack_fixed_build(row, col, vals, M: int, K: int, dtype=None, flags: int = 0) -> SnackFixed:
    """row, col (int32) and vals (float32, or uint16 bf16 bits with dtype=BF16)
    are HOST numpy arrays."""
    import numpy as np
    row = np.ascontiguousarray(row, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    vals = np.ascontiguousarray(vals)
    if dtype is None:
        dtype = F32 if vals.dtype == np.float32 else BF16
    out = ctypes.c_void_p(0)
    _check(_lib.snack_fixed_build(row.ctypes.data or None, col.ctypes.data or None,
                                  vals.ctypes.data or None, dtype, M, K, row.size, flags,
                                  ctypes.byref(out)), "snack_fixed_build")
    return SnackFixed(out.value)


def snack_fixed_fwd(f: SnackFixed, X, B: int, images: int, Y, stream=None):
    _check(_lib.snack_fixed_fwd(f.handle, _ptr(X), B, images, _ptr(Y), _stream(stream)),
           "snack_fixed_fwd")


def snack_conv1x1(plan, vals, X, N: int, HW: int, layout: int, Y, stream=None, dtype=None):
    dt = _dtype(vals, X, Y, dtype=dtype)
    _check(_lib.snack_conv1x1(ctypes.byref(plan), _ptr(vals), dt, _ptr(X), N, HW, layout,
                              _ptr(Y), _stream(stream)), "snack_conv1x1")


def snack_gelu_fwd(z, h, n=None, stream=None):
    n = z.numel() if n is None else n
    _check(_lib.snack_gelu_fwd(_ptr(z), _ptr(h), n, _stream(stream)), "snack_gelu_fwd")


def snack_gelu_bwd(z, dh, dz, n=None, stream=None):
    n = z.numel() if n is None else n
    _check(_lib.snack_gelu_bwd(_ptr(z), _ptr(dh), _ptr(dz), n, _stream(stream)),
           "snack_gelu_bwd")


def snack_dense_fwd(W, mask, M, K, X, B, Y, stream=None, dtype=None):
    dt = _dtype(W, X, Y, dtype=dtype)
    _check(_lib.snack_dense_fwd(_ptr(W), _ptr(mask), dt, M, K, _ptr(X), B, _ptr(Y),
                                _stream(stream)), "snack_dense_fwd")


CALIB_EMPTY, CALIB_READ, CALIB_WRITE, CALIB_CHAIN, CALIB_CHASE = 0, 1, 2, 3, 4


def snack_calibrate(kind: int, buf=None, nbytes: int = 0, n: int = 1, stream=None):
    """Launch one calibration kernel (empty, read, write, chain, chase)."""
    _check(_lib.snack_calibrate(kind, _ptr(buf), nbytes, n, _stream(stream)), "snack_calibrate")


def raw_status(name: str, *args) -> int:
    """Call an entry point with raw ctypes arguments and return its status
    (for tests of the host-side argument checks)."""
    return getattr(_lib, name)(*args)


lib = _lib
