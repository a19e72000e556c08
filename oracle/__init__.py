"""Serial fp64 CPU oracle of the truly sparse linear layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never imports, links or calls it, and it never calls the HIP
library: the two share nothing but the seeded inputs from ``synth``.

Every function follows a definition stated in ``oracle.c`` (forward
``Y = X W^T``, input gradient ``dX = dY W``, value gradient ``dV[k] =
sum_b dY[b,row_k] X[b,col_k]``, the derived index arrays, the load-balanced
partition and the prune/regrow rule).  Floats are widened exactly to fp64
before any arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# SNACK_ORACLE_SANITIZE=1 (set by the sanitizer test for its child process):
# load the AddressSanitizer + UndefinedBehaviorSanitizer build instead
_SANITIZE = os.environ.get("SNACK_ORACLE_SANITIZE") == "1"
_SO = os.path.join(_HERE, "liboracle_asan.so" if _SANITIZE else "liboracle.so")

_lib = None


def build(force: bool = True, sanitize: bool = _SANITIZE) -> str:
    """Compile oracle.c with gcc into liboracle.so (serial, no fast-math); with
    sanitize, into liboracle_asan.so with -fsanitize=address,undefined (no
    recovery: the first report aborts)."""
    so = os.path.join(_HERE, "liboracle_asan.so" if sanitize else "liboracle.so")
    if force or not os.path.exists(so):
        tmp = so + ".tmp"
        extra = (["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"] if sanitize else [])
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                        "-fno-fast-math", *extra, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, so)
    return so


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    lib.orc_validate_coo.argtypes = [i32, i32, i64, P, P]
    lib.orc_validate_coo.restype = ctypes.c_int
    lib.orc_spmm_fwd.argtypes = [i32, i32, i64, P, P, P, i32, P, ctypes.c_int, P, P]
    lib.orc_spmm_bwd_input.argtypes = [i32, i32, i64, P, P, P, i32, P, ctypes.c_int, P, P]
    lib.orc_sddmm.argtypes = [i32, i32, i64, P, P, i32, P, P, ctypes.c_int, P, P]
    lib.orc_gelu.argtypes = [i64, P, P]
    lib.orc_gelu_bwd.argtypes = [i64, P, P, P]
    lib.orc_row_ptr.argtypes = [i32, i64, P, P]
    lib.orc_csc.argtypes = [i32, i64, P, P, P, P, P]
    lib.orc_csc.restype = ctypes.c_int
    lib.orc_partition.argtypes = [i32, i64, P, i64, P, P, P, P, P, P]
    lib.orc_partition.restype = i64
    lib.orc_splitmix64.argtypes = [u64, u64]
    lib.orc_splitmix64.restype = u64
    lib.orc_drop_count.argtypes = [i64, ctypes.c_int32]
    lib.orc_drop_count.restype = i64
    lib.orc_prune_regrow.argtypes = [i32, i32, i64, P, P, P, ctypes.c_int, i64, u64, u64,
                                     P, P, P, P, P]
    lib.orc_prune_regrow.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


ERRORS = {0: "ok", -5: "coo index out of range", -6: "coo not strictly increasing",
          -7: "nan value", -8: "bad count", -12: "out of memory"}


def validate_coo(M, K, row, col) -> int:
    row, col = _i32(row), _i32(col)
    return _load().orc_validate_coo(M, K, row.size, _p(row), _p(col))


def spmm_fwd(M, K, row, col, v, B, X, node_major=False):
    """Y = X W^T in fp64; returns (Y, S) flat, same layout as X."""
    row, col, v, X = _i32(row), _i32(col), _f64(v), _f64(X)
    assert X.size == B * K
    Y = np.empty(B * M, dtype=np.float64)
    S = np.empty(B * M, dtype=np.float64)
    _load().orc_spmm_fwd(M, K, row.size, _p(row), _p(col), _p(v), B, _p(X), int(node_major),
                         _p(Y), _p(S))
    return Y, S


def spmm_bwd_input(M, K, row, col, v, B, dY, node_major=False):
    """dX = dY W in fp64; returns (dX, S) flat."""
    row, col, v, dY = _i32(row), _i32(col), _f64(v), _f64(dY)
    assert dY.size == B * M
    dX = np.empty(B * K, dtype=np.float64)
    S = np.empty(B * K, dtype=np.float64)
    _load().orc_spmm_bwd_input(M, K, row.size, _p(row), _p(col), _p(v), B, _p(dY),
                               int(node_major), _p(dX), _p(S))
    return dX, S


def sddmm(M, K, row, col, B, dY, X, node_major=False):
    """dV[k] = sum_b dY[b,row_k] X[b,col_k] in fp64; returns (dV, S)."""
    row, col, dY, X = _i32(row), _i32(col), _f64(dY), _f64(X)
    dV = np.empty(row.size, dtype=np.float64)
    S = np.empty(row.size, dtype=np.float64)
    _load().orc_sddmm(M, K, row.size, _p(row), _p(col), B, _p(dY), _p(X), int(node_major),
                      _p(dV), _p(S))
    return dV, S


def gelu(z):
    z = _f64(z)
    out = np.empty_like(z)
    _load().orc_gelu(z.size, _p(z), _p(out))
    return out


def gelu_bwd(z, dy):
    z, dy = _f64(z), _f64(dy)
    out = np.empty_like(z)
    _load().orc_gelu_bwd(z.size, _p(z), _p(dy), _p(out))
    return out


def row_ptr(M, row):
    row = _i32(row)
    out = np.empty(M + 1, dtype=np.int32)
    _load().orc_row_ptr(M, row.size, _p(row), _p(out))
    return out


def csc(K, row, col):
    """Returns (col_ptr[K+1], perm[nnz], row_t[nnz])."""
    row, col = _i32(row), _i32(col)
    n = row.size
    col_ptr = np.empty(K + 1, dtype=np.int32)
    perm = np.empty(n, dtype=np.int32)
    row_t = np.empty(n, dtype=np.int32)
    rc = _load().orc_csc(K, n, _p(row), _p(col), _p(col_ptr), _p(perm), _p(row_t))
    if rc:
        raise MemoryError
    return col_ptr, perm, row_t


def partition(ptr, T):
    """Merge-path tiles with short segments kept whole.

    Returns dict(P, part_seg[P+1], part_nz[P+1], split=(seg, first, last))."""
    ptr = _i32(ptr)
    S = ptr.size - 1
    nnz = int(ptr[-1])
    Pmax = (S + nnz + T - 1) // T
    part_seg = np.empty(Pmax + 1, dtype=np.int32)
    part_nz = np.empty(Pmax + 1, dtype=np.int32)
    ss = np.empty(max(Pmax, 1), dtype=np.int32)
    sf = np.empty(max(Pmax, 1), dtype=np.int32)
    sl = np.empty(max(Pmax, 1), dtype=np.int32)
    ns = ctypes.c_int64(0)
    P = _load().orc_partition(S, nnz, _p(ptr), T, _p(part_seg), _p(part_nz), _p(ss), _p(sf),
                              _p(sl), ctypes.byref(ns))
    n = ns.value
    return {"P": int(P), "part_seg": part_seg[:P + 1], "part_nz": part_nz[:P + 1],
            "split_seg": ss[:n].copy(), "split_first": sf[:n].copy(), "split_last": sl[:n].copy()}


def splitmix64(state: int, i: int) -> int:
    return int(_load().orc_splitmix64(state & (2**64 - 1), i))


def drop_count(nnz: int, ppm: int) -> int:
    return int(_load().orc_drop_count(nnz, ppm))


def prune_regrow(M, K, row, col, vals, dtype, n_drop, seed, step):
    """One prune/regrow step; returns dict(row, col, vals, dropped, grown, rc).

    ``vals`` are float32 values or bf16 bit patterns (uint16)."""
    row, col = _i32(row), _i32(col)
    n = row.size
    if dtype == "bf16":
        vb = np.asarray(vals, dtype=np.uint16).astype(np.uint32)
    else:
        vb = np.ascontiguousarray(vals, dtype=np.float32).view(np.uint32).copy()
    orow = np.empty(n, dtype=np.int32)
    ocol = np.empty(n, dtype=np.int32)
    ovb = np.empty(n, dtype=np.uint32)
    dl = np.empty(max(n_drop, 1), dtype=np.int64)
    gl = np.empty(max(n_drop, 1), dtype=np.int64)
    rc = _load().orc_prune_regrow(M, K, n, _p(row), _p(col), _p(vb), int(dtype == "bf16"),
                                  n_drop, seed & (2**64 - 1), step & (2**64 - 1), _p(orow),
                                  _p(ocol), _p(ovb), _p(dl), _p(gl))
    if rc:
        return {"rc": rc}
    ov = ovb.astype(np.uint16) if dtype == "bf16" else ovb.view(np.float32)
    return {"rc": 0, "row": orow, "col": ocol, "vals": ov, "dropped": dl[:n_drop].copy(),
            "grown": gl[:n_drop].copy()}


def adam_step(w, g, m, v, lr, beta1, beta2, eps, step):
    """One Adam step (Kingma & Ba, "Adam: A Method for Stochastic
    Optimization", ICLR 2015, Algorithm 1) in fp64 on flat arrays:
        m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2,
        w <- w - lr * (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps).
    Returns (w, m, v); nothing is rounded."""
    w, g, m, v = (np.asarray(a, dtype=np.float64) for a in (w, g, m, v))
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    return w - lr * mh / (np.sqrt(vh) + eps), m, v


def memory_by_definition(M: int, K: int, nnz: int, elem_bytes: int, max_batch: int) -> dict:
    """Bytes of the tensors whose size the layer's definition fixes (SNACK
    abstract: the sparse layer stores only its nonzero connections; the
    baselines store a dense weight, Dense+Mask adds a mask): element counts
    times element sizes.  The COO holds two int32 indices and one value per
    connection; the value gradient one value per connection; the dense layer
    a weight and a gradient of M*K values; the mask one byte per weight;
    the activations X (B x K), Y (B x M) and their gradients at B =
    max_batch.  Plan and workspace sizes belong to the implementation, not
    to the definition, and are not computed here.  Pinned against byte
    counts written out by hand and against numpy's nbytes of arrays of those
    shapes and dtypes."""
    mk = M * K
    return {
        "coo": nnz * (4 + 4 + elem_bytes),
        "value_grad": nnz * elem_bytes,
        "dense_weight": mk * elem_bytes,
        "dense_grad": mk * elem_bytes,
        "mask": mk,
        "activations": max_batch * (K + M) * elem_bytes * 2,
    }


def act_f64(x, act: int):
    """The nonlinearity of a propagation step in fp64: 0 identity, 1 ReLU
    (max(x, 0)), 2 exact GELU."""
    x = _f64(x)
    if act == 1:
        return np.where(x > 0, x, 0.0)
    if act == 2:
        return gelu(x)
    return x.copy()


def graph_propagate(M, K, row, col, v, B, X, layers: int, act: int, node_major=False):
    """Multi-layer propagation through one sparse adjacency (the SNACK
    abstract's graph-style inference, read as H_l = act(H_{l-1} W^T)), in fp64
    with no rounding between layers.  Returns [(H_l, S_l)] for l = 1..layers,
    S_l the per-output sum of |v| |H_{l-1}| of layer l (its error scale)."""
    out = []
    H = _f64(X)
    for _ in range(layers):
        Z, S = spmm_fwd(M, K, row, col, v, B, H, node_major)
        H = act_f64(Z, act)
        out.append((H, S))
    return out
