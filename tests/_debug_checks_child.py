"""Run by test_debug_build.py in a child process with SNACK_LIBRARY naming the
debug build (libsnack_debug.so): the products match the oracle, and a plan
array or COO index put out of range turns every product call into
SNACK_E_PLAN_CORRUPT before any product kernel runs (the check kernel reads
each array only within its size, so nothing is read out of bounds)."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import synth  # noqa: E402
import unstructured_sparse_nn_amd as snk  # noqa: E402
from unstructured_sparse_nn_amd import binding as B  # noqa: E402

assert os.path.basename(B.LIB_PATH) == "libsnack_debug.so", B.LIB_PATH
orc = oracle
M, K, Bsz = 96, 80, 8
w = synth.random_case(31, M, K, 2000, Bsz, "f32", "node")
wt = w.weights[0]
row = torch.from_numpy(wt.row).cuda()
col = torch.from_numpy(wt.col).cuda()
vals = torch.from_numpy(wt.vals).cuda()
X = torch.from_numpy(w.X[0].data).cuda()
dY = torch.from_numpy(w.dY[0].data).cuda()
topo = snk.Topology(row, col, M, K, Bsz)
NM = B.NODE_MAJOR


def within(got, ref, S, what):
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * S), what


def products():
    Y = topo.fwd(vals, X, Bsz, NM)
    dX = topo.bwd_input(vals, dY, Bsz, NM)
    dV = topo.grad_vals(dY, X, Bsz, NM)
    torch.cuda.synchronize()
    return Y, dX, dV


Y, dX, dV = products()
X64, dY64, v64 = w.X[0].f64(), w.dY[0].f64(), wt.vals_f64()
within(Y, *orc.spmm_fwd(M, K, wt.row, wt.col, v64, Bsz, X64, True), "fwd")
within(dX, *orc.spmm_bwd_input(M, K, wt.row, wt.col, v64, Bsz, dY64, True), "dX")
within(dV, *orc.sddmm(M, K, wt.row, wt.col, Bsz, dY64, X64, True), "dV")
print("products match the oracle", flush=True)


def corrupt(t, i, value, name):
    old = int(t[i].item())
    t[i] = value
    torch.cuda.synchronize()
    for call, out_len in ((lambda o: topo.fwd(vals, X, Bsz, NM, out=o), M * Bsz),
                          (lambda o: topo.bwd_input(vals, dY, Bsz, NM, out=o), K * Bsz)):
        out = torch.full((out_len,), float("nan"), device="cuda")
        try:
            call(out)
        except B.SnackError as e:
            assert e.status == -13, (name, e.status)
        else:
            raise AssertionError(f"{name}: no error")
        torch.cuda.synchronize()
        assert torch.isnan(out).all(), f"{name}: a product kernel ran"
    t[i] = old
    torch.cuda.synchronize()
    print(f"{name}: refused", flush=True)


nnz = wt.nnz
corrupt(col, 7, K + 3, "COO column past K")
corrupt(col, 0, -1, "negative COO column")
corrupt(topo.array("row_ptr"), 5, nnz + 50, "row offset past nnz")
corrupt(topo.array("row_ptr"), M, nnz - 1, "last row offset != nnz")
corrupt(topo.array("col_ptr"), 3, -4, "negative column offset")
corrupt(topo.array("perm"), 3, nnz, "perm past nnz")
corrupt(topo.array("row_t"), 11, M, "row_t past M")
corrupt(topo.array("rcut"), 1, 7, "cut flag not 0/1")
corrupt(topo.array("cpart_nz"), 1, nnz + 1, "column tile past nnz")
Y2, dX2, dV2 = products()  # restored: the same results again
assert torch.equal(Y, Y2) and torch.equal(dX, dX2) and torch.equal(dV, dV2)
print("DEBUG CHECKS OK", flush=True)
