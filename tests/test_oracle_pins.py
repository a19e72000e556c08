"""Pins of the CPU oracle against things other than itself.

The SNACK page defines the layer only in words (a layer that stores and
computes only its nonzeros, with gradients kept sparse); the pins therefore
come from mathematics: a dense masked product through numpy, the gradient
identities, the adjoint identity, exact finite differences of a bilinear map,
brute-force recounts, a full lexicographic sort, published SplitMix64 outputs
and the worked examples printed on the "Two Lotteries" page.
"""
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def dense_of(w):
    W = np.zeros((w.M, w.K), dtype=np.float64)
    W[w.row, w.col] = w.vals_f64()
    return W


def as_bf(a, layout, B, F):
    """flat activation -> (B, F) array"""
    return a.reshape(F, B).T if layout == "node" else a.reshape(B, F)


EDGE = [
    # (M, K, nnz, B, layout)
    (1, 1, 1, 1, "batch"),
    (1, 1, 0, 3, "batch"),
    (5, 7, 0, 2, "node"),
    (1, 64, 64, 4, "batch"),       # one fully dense row
    (64, 1, 64, 4, "node"),        # one fully dense column
    (13, 11, 143, 3, "batch"),     # full density: plain GEMM
    (37, 53, 200, 1, "batch"),     # B = 1: SpMV
    (200, 150, 900, 5, "node"),
    (300, 40, 30, 2, "batch"),     # many empty rows
]


@pytest.mark.parametrize("M,K,nnz,B,layout", EDGE)
def test_products_match_dense_masked_gemm(orc, M, K, nnz, B, layout):
    w = synth.random_case(11, M, K, nnz, B, "f32", layout)
    wt = w.weights[0]
    X, dY = w.X[0].f64(), w.dY[0].f64()
    nm = layout == "node"
    W = dense_of(wt)
    Xb, dYb = as_bf(X, layout, B, K), as_bf(dY, layout, B, M)
    Y, S = orc.spmm_fwd(M, K, wt.row, wt.col, wt.vals_f64(), B, X, nm)
    np.testing.assert_allclose(as_bf(Y, layout, B, M), Xb @ W.T, rtol=0, atol=1e-13)
    dX, S_dx = orc.spmm_bwd_input(M, K, wt.row, wt.col, wt.vals_f64(), B, dY, nm)
    np.testing.assert_allclose(as_bf(dX, layout, B, K), dYb @ W, rtol=0, atol=1e-13)
    dV, S_dw = orc.sddmm(M, K, wt.row, wt.col, B, dY, X, nm)
    np.testing.assert_allclose(dV, (dYb.T @ Xb)[wt.row, wt.col], rtol=0, atol=1e-13)
    # each error scale is the sum of its output's term magnitudes, i.e. the
    # same product taken over |W|, |X| and |dY|: S_y = |X| |W|^T,
    # S_dx = |dY| |W| and S_dw = (|dY|^T |X|) at the nonzeros.  These scales
    # gate every GPU tolerance, so a wrong one would silently loosen them.
    np.testing.assert_allclose(as_bf(S, layout, B, M), np.abs(Xb) @ np.abs(W).T, atol=1e-13)
    np.testing.assert_allclose(as_bf(S_dx, layout, B, K), np.abs(dYb) @ np.abs(W), atol=1e-13)
    np.testing.assert_allclose(S_dw, (np.abs(dYb).T @ np.abs(Xb))[wt.row, wt.col], atol=1e-13)
    # a scale bounds its output and is never negative
    for out, sc in ((Y, S), (dX, S_dx), (dV, S_dw)):
        assert (sc >= 0).all() and (np.abs(out) <= sc + 1e-13).all()


def test_diagonal_identity_is_exact(orc):
    n, B = 33, 4
    pos = np.arange(n) * n + np.arange(n)
    w = synth.random_case(1, n, n, n, B, positions=pos)
    X = w.X[0].f64()
    Y, _ = orc.spmm_fwd(n, n, w.weights[0].row, w.weights[0].col, np.ones(n), B, X)
    assert np.array_equal(Y, X)


def test_single_layer_config_against_dense(orc):
    w = synth.single_layer()
    wt = w.weights[0]
    assert wt.nnz == 6554
    X, dY = w.X[0].f64(), w.dY[0].f64()
    W = dense_of(wt)
    Y, _ = orc.spmm_fwd(wt.M, wt.K, wt.row, wt.col, wt.vals_f64(), 4, X)
    np.testing.assert_allclose(Y.reshape(4, 256), X.reshape(4, 256) @ W.T, atol=1e-13)
    dX, _ = orc.spmm_bwd_input(wt.M, wt.K, wt.row, wt.col, wt.vals_f64(), 4, dY)
    np.testing.assert_allclose(dX.reshape(4, 256), dY.reshape(4, 256) @ W, atol=1e-13)


def _adjoint(orc, wt, B, X, dY, nm):
    v = wt.vals_f64()
    Y, _ = orc.spmm_fwd(wt.M, wt.K, wt.row, wt.col, v, B, X, nm)
    dX, _ = orc.spmm_bwd_input(wt.M, wt.K, wt.row, wt.col, v, B, dY, nm)
    dV, _ = orc.sddmm(wt.M, wt.K, wt.row, wt.col, B, dY, X, nm)
    a, b, c = float(dY @ Y), float(dX @ X), float(v @ dV)
    scale = float(np.abs(dY) @ np.abs(Y)) + 1e-300
    assert abs(a - b) <= 1e-12 * scale and abs(a - c) <= 1e-12 * scale


@pytest.mark.parametrize("which", ["single", "square95", "square99", "gpt2_90", "gpt2_99",
                                   "llama_up", "llama_down"])
def test_adjoint_identity_at_config_sizes(orc, which):
    """<dY, X W^T> = <dY W, X> = <v, dV> holds for every bilinear product."""
    if which == "single":
        w = synth.single_layer()
    elif which.startswith("square"):
        w = synth.inference_layer(sparsity=0.95 if which == "square95" else 0.99, B=8)
    elif which.startswith("gpt2"):
        w = synth.gpt2_mlp(sparsity=0.9 if which == "gpt2_90" else 0.99, B=64)
        # second layer's X and first layer's dY are not drawn by the config
        rng = np.random.default_rng(5)
        w.X[1] = synth.Activation(rng.standard_normal(64 * 3072).astype(np.float32), "f32",
                                  64, 3072, "batch")
        w.dY[0] = synth.Activation(rng.standard_normal(64 * 3072).astype(np.float32), "f32",
                                   64, 3072, "batch")
    else:
        w = synth.llama_proj(which=which.split("_")[1], B=4)
    for i, wt in enumerate(w.weights):
        _adjoint(orc, wt, w.B, w.X[i].f64(), w.dY[i].f64(), w.X[i].layout == "node")


@pytest.mark.slow
def test_adjoint_identity_graph(orc):
    w = synth.graph_layer()
    wt = w.weights[0]
    assert wt.nnz == 2_400_000
    _adjoint(orc, wt, 128, w.X[0].f64(), w.dY[0].f64(), True)


def test_finite_differences_are_exact_for_bilinear_map(orc):
    """L(v, X) = <G, X W(v)^T> is linear in each v[k] and in X, so a central
    difference with step 1 equals the derivative up to rounding."""
    w = synth.random_case(3, 40, 30, 250, 3)
    wt = w.weights[0]
    v = wt.vals_f64()
    X, G = w.X[0].f64(), w.dY[0].f64()

    def L(vv, XX):
        Y, _ = orc.spmm_fwd(40, 30, wt.row, wt.col, vv, 3, XX)
        return float(G @ Y)

    dV, _ = orc.sddmm(40, 30, wt.row, wt.col, 3, G, X)
    dX, _ = orc.spmm_bwd_input(40, 30, wt.row, wt.col, v, 3, G)
    for k in [0, 7, 100, 249]:
        e = np.zeros_like(v)
        e[k] = 1.0
        fd = (L(v + e, X) - L(v - e, X)) / 2
        assert abs(fd - dV[k]) <= 1e-12 * (1 + abs(dV[k]))
    for j in [0, 5, 44, 89]:
        e = np.zeros_like(X)
        e[j] = 1.0
        fd = (L(v, X + e) - L(v, X - e)) / 2
        assert abs(fd - dX[j]) <= 1e-12 * (1 + abs(dX[j]))


def test_gelu_against_scipy_and_differences(orc):
    from scipy.special import erf
    z = np.linspace(-6, 6, 1001)
    np.testing.assert_allclose(orc.gelu(z), 0.5 * z * (1 + erf(z / np.sqrt(2))), rtol=1e-12,
                               atol=1e-22)
    h = 1e-5
    fd = (orc.gelu(z + h) - orc.gelu(z - h)) / (2 * h)
    np.testing.assert_allclose(orc.gelu_bwd(z, np.ones_like(z)), fd, atol=1e-9)
    # closed forms: gelu(0) = 0, gelu'(0) = 1/2
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    assert orc.gelu_bwd(np.array([0.0]), np.array([1.0]))[0] == 0.5


# ------------------------------------------------------------ index arrays
@pytest.mark.parametrize("M,K,nnz", [(1, 1, 0), (1, 1, 1), (300, 40, 30), (64, 1, 64),
                                     (256, 256, 6554), (4096, 4096, 167772)])
def test_row_ptr_and_csc_brute_force(orc, M, K, nnz):
    wt = synth.random_case(2, M, K, nnz, 1).weights[0]
    rp = orc.row_ptr(M, wt.row)
    assert np.array_equal(rp, np.concatenate(([0], np.cumsum(np.bincount(wt.row, minlength=M)))))
    cp, perm, rt = orc.csc(K, wt.row, wt.col)
    assert np.array_equal(cp, np.concatenate(([0], np.cumsum(np.bincount(wt.col, minlength=K)))))
    ref = np.lexsort((wt.row, wt.col))  # by column, then row: stable column order
    assert np.array_equal(perm, ref)
    assert np.array_equal(rt, wt.row[ref])


def _walk_partition(ptr, T):
    """Brute force: list every item of the merge path, read the point at each
    multiple of T, then keep short segments whole."""
    S = len(ptr) - 1
    pts = []          # point (s, z) before item i
    s = z = 0
    for seg in range(S):
        for _ in range(ptr[seg + 1] - ptr[seg]):
            pts.append((s, z))
            z += 1
        pts.append((s, z))
        s += 1
    I = len(pts)
    P = -(-I // T)
    seg_b, nz_b = [], []
    for p in range(P):
        s, z = pts[p * T]
        if z != ptr[s] and ptr[s + 1] - ptr[s] < T:
            z = ptr[s]
        seg_b.append(s)
        nz_b.append(z)
    seg_b.append(S)
    nz_b.append(int(ptr[-1]))
    return P, np.array(seg_b), np.array(nz_b)


@pytest.mark.parametrize("lengths,T", [
    ([0], 1), ([3], 1), ([3], 4), ([0, 0, 5, 0], 2), ([10, 10, 10, 90], 31),
    ([1] * 50 + [400] + [0] * 20 + [7] * 30, 16), ([64] * 10, 64), ([63, 64, 65], 64),
])
def test_partition_brute_force(orc, lengths, T):
    ptr = np.concatenate(([0], np.cumsum(lengths))).astype(np.int32)
    got = orc.partition(ptr, T)
    P, sb, zb = _walk_partition(list(ptr), T)
    assert got["P"] == P
    assert np.array_equal(got["part_seg"], sb) and np.array_equal(got["part_nz"], zb)
    # split list: segments holding an inner boundary, with first/last tiles
    exp = []
    for s in range(len(lengths)):
        inner = [p for p in range(1, P) if sb[p] == s and zb[p] > ptr[s]]
        if inner:
            exp.append((s, inner[0] - 1, inner[-1]))
    got_split = list(zip(got["split_seg"], got["split_first"], got["split_last"]))
    assert got_split == exp


def test_partition_invariants_on_skewed_rows(orc):
    w = synth.llama_proj(which="down", B=1)
    wt = w.weights[0]
    ptr = orc.row_ptr(wt.M, wt.row)
    T = 2048
    got = orc.partition(ptr, T)
    seg, nz = got["part_seg"].astype(np.int64), got["part_nz"].astype(np.int64)
    items = np.diff(seg + nz)
    assert (items > 0).all() and items.max() < 2 * T
    assert (np.diff(seg) >= 0).all() and (np.diff(nz) >= 0).all()
    inside = seg[:-1] < wt.M
    assert ((ptr[seg[:-1][inside]] <= nz[:-1][inside]) &
            (nz[:-1][inside] <= ptr[seg[:-1][inside] + 1])).all()
    lengths = np.diff(ptr)
    for s, f, l in zip(got["split_seg"], got["split_first"], got["split_last"]):
        assert lengths[s] >= T and l > f


def test_partition_fixes_page_imbalance_example(orc):
    """Page example: units left with 10, 10, 10 and 90 operations.  A fixed
    assignment finishes with the 90; the balanced tiles stay near the mean."""
    g = json.load(open(os.path.join(GOLD, "imbalance_example.json")))
    after = g["units_after"]
    assert 1 - sum(after) / sum(g["units_before"]) == pytest.approx(g["removed_fraction"])
    assert max(after) == g["static_completion"]
    ptr = np.concatenate(([0], np.cumsum(after))).astype(np.int32)
    n_units = len(after)
    T = -(-(sum(after) + n_units) // n_units)
    got = orc.partition(ptr, T)
    assert got["P"] == n_units
    loads = np.diff(got["part_seg"].astype(np.int64) + got["part_nz"])
    assert loads.max() < g["static_completion"] / 2
    assert loads.sum() == sum(after) + n_units


# ------------------------------------------------------------ prune / regrow
def test_splitmix64_published_vectors(orc):
    g = json.load(open(os.path.join(GOLD, "splitmix64_vectors.json")))
    for case in g["cases"]:
        outs = [orc.splitmix64(case["seed"], i) for i in range(len(case["outputs"]))]
        assert outs == [int(x) for x in case["outputs"]]


def test_drop_count_rounding(orc):
    assert orc.drop_count(6554, 100000) == 655
    assert orc.drop_count(235930, 300000) == 70779
    assert orc.drop_count(23593, 300000) == 7078
    assert orc.drop_count(5, 500000) == 3      # 2.5 rounds half up
    assert orc.drop_count(0, 300000) == 0


def _absbits(vals, dtype):
    if dtype == "bf16":
        return np.asarray(vals, np.uint16).astype(np.int64) & 0x7FFF
    return np.asarray(vals, np.float32).view(np.uint32).astype(np.int64) & 0x7FFFFFFF


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,nnz,ppm", [(256, 256, 6554, 100000), (64, 48, 700, 300000),
                                         (10, 10, 50, 1000000), (7, 9, 1, 1000000)])
def test_prune_regrow_against_sort_and_invariants(orc, dtype, M, K, nnz, ppm):
    wt = synth.random_case(4, M, K, nnz, 1, dtype).weights[0]
    vals = wt.vals.copy()
    # plant ties and signed zeros so the tie-break by linear index matters
    if nnz > 20:
        vals[5] = vals[9] = vals[13]
        vals[2] = np.float32(-0.0) if dtype == "f32" else np.uint16(0x8000)
        vals[3] = np.float32(0.0) if dtype == "f32" else np.uint16(0)
    n_drop = orc.drop_count(nnz, ppm)
    out = orc.prune_regrow(M, K, wt.row, wt.col, vals, dtype, n_drop, seed=7, step=3)
    assert out["rc"] == 0
    lin = wt.row.astype(np.int64) * K + wt.col
    order = np.lexsort((lin, _absbits(vals, dtype)))
    assert np.array_equal(out["dropped"], np.sort(lin[order[:n_drop]]))
    grown = out["grown"]
    assert np.array_equal(grown, np.unique(grown)) and grown.size == n_drop
    assert not np.isin(grown, lin).any()
    assert grown.min(initial=0) >= 0 and grown.max(initial=0) < M * K
    new_lin = out["row"].astype(np.int64) * K + out["col"]
    assert (np.diff(new_lin) > 0).all() and new_lin.size == nnz
    survivors = np.setdiff1d(lin, out["dropped"])
    assert np.array_equal(np.sort(np.concatenate((survivors, grown))), new_lin)
    # survivors keep their values, grown entries are zero
    old = dict(zip(lin.tolist(), np.asarray(vals).tolist()))
    newv = np.asarray(out["vals"])
    for l, vv in zip(new_lin.tolist(), newv.tolist()):
        assert vv == (old[l] if l in old else 0)
    # the layer's function is unchanged by growth: fwd(after) == fwd(before
    # with the dropped entries zeroed), exactly
    if dtype == "f32":
        rng = np.random.default_rng(0)
        X = rng.standard_normal(2 * K)
        vz = np.asarray(vals, np.float64).copy()
        vz[np.isin(lin, out["dropped"])] = 0
        Ya, _ = orc.spmm_fwd(M, K, out["row"], out["col"], newv.astype(np.float64), 2, X)
        Yb, _ = orc.spmm_fwd(M, K, wt.row, wt.col, vz, 2, X)
        assert np.array_equal(Ya, Yb)


def test_prune_regrow_grown_positions_follow_the_stream(orc):
    """The first accepted candidates of the SplitMix64 stream, recomputed
    here from the pinned generator outputs, are the grown positions."""
    M, K, nnz = 20, 30, 100
    wt = synth.random_case(9, M, K, nnz, 1).weights[0]
    lin = set((wt.row.astype(np.int64) * K + wt.col).tolist())
    out = orc.prune_regrow(M, K, wt.row, wt.col, wt.vals, "f32", 10, seed=123, step=4)
    s = orc.splitmix64(123, 4)
    acc, i = [], 0
    while len(acc) < 10:
        p = (orc.splitmix64(s, i) * (M * K)) >> 64
        if p not in lin and p not in acc:
            acc.append(p)
        i += 1
    assert sorted(acc) == out["grown"].tolist()


def test_prune_regrow_determinism_and_errors(orc):
    wt = synth.random_case(4, 64, 64, 400, 1).weights[0]
    a = orc.prune_regrow(64, 64, wt.row, wt.col, wt.vals, "f32", 40, 1, 1)
    b = orc.prune_regrow(64, 64, wt.row, wt.col, wt.vals, "f32", 40, 1, 1)
    c = orc.prune_regrow(64, 64, wt.row, wt.col, wt.vals, "f32", 40, 1, 2)
    assert np.array_equal(a["grown"], b["grown"]) and not np.array_equal(a["grown"], c["grown"])
    v = wt.vals.copy()
    v[3] = np.nan
    assert orc.prune_regrow(64, 64, wt.row, wt.col, v, "f32", 40, 1, 1)["rc"] == -7
    assert orc.prune_regrow(64, 64, wt.row, wt.col, wt.vals, "f32", 401, 1, 1)["rc"] == -8
    full = synth.random_case(4, 4, 4, 16, 1).weights[0]
    assert orc.prune_regrow(4, 4, full.row, full.col, full.vals, "f32", 1, 1, 1)["rc"] == -8


def test_regrow_is_roughly_uniform(orc):
    """Statistical only: grown rows over many steps pass a loose chi-square."""
    M, K, nnz = 32, 32, 200
    wt = synth.random_case(5, M, K, nnz, 1).weights[0]
    counts = np.zeros(M)
    for step in range(200):
        out = orc.prune_regrow(M, K, wt.row, wt.col, wt.vals, "f32", 20, 99, step)
        counts += np.bincount(out["grown"] // K, minlength=M)
    expected = counts.sum() * (K - np.bincount(wt.row, minlength=M)) / (M * K - nnz)
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    assert chi2 < 3 * M, chi2


def test_validate_coo(orc):
    assert orc.validate_coo(4, 4, [0, 0, 1], [1, 2, 0]) == 0
    assert orc.validate_coo(4, 4, [0, 0], [2, 2]) == -6
    assert orc.validate_coo(4, 4, [0, 1], [2, 1]) == 0
    assert orc.validate_coo(4, 4, [1, 0], [0, 3]) == -6
    assert orc.validate_coo(4, 4, [0, 4], [0, 0]) == -5
    assert orc.validate_coo(4, 4, [0], [-1]) == -5


def test_generator_counts_and_determinism():
    w1, w2 = synth.single_layer(), synth.single_layer()
    assert np.array_equal(w1.weights[0].row, w2.weights[0].row)
    assert np.array_equal(w1.X[0].data, w2.X[0].data)
    wt = w1.weights[0]
    lin = wt.row.astype(np.int64) * 256 + wt.col
    assert (np.diff(lin) > 0).all() and lin.size == 6554
    assert synth.nnz_for(4096, 4096, 0.95) == 838861
    assert synth.nnz_for(11008, 4096, 0.9) == 4508877
    d = synth.rank_profile(11008, 4096, 4508877, 1.2)
    assert d.sum() == 4508877 and (d == 4096).sum() == 310


def test_graph_propagation_composes_dense_steps(orc):
    """The oracle's multi-layer propagation equals repeated dense products
    (numpy) with the nonlinearity applied after each, for ReLU and GELU; and
    with a diagonal identity adjacency and ReLU it is ReLU of the input."""
    rng = np.random.default_rng(11)
    N, B, L = 9, 3, 3
    lin = np.sort(rng.choice(N * N, 30, replace=False))
    row, col = (lin // N).astype(np.int32), (lin % N).astype(np.int32)
    v = rng.standard_normal(lin.size)
    W = np.zeros((N, N))
    W[row, col] = v
    X = rng.standard_normal(B * N)
    for act in (1, 2):
        got = orc.graph_propagate(N, N, row, col, v, B, X, L, act)
        H = X.reshape(B, N)
        for l in range(L):
            scale = np.abs(H) @ np.abs(W).T  # layer l's error scale, from its input
            Z = H @ W.T
            H = np.maximum(Z, 0) if act == 1 else orc.gelu(Z.ravel()).reshape(B, N)
            assert np.allclose(got[l][0].reshape(B, N), H, rtol=1e-13, atol=1e-15)
            assert np.allclose(got[l][1].reshape(B, N), scale, rtol=1e-13, atol=1e-15)
    eye = np.arange(N, dtype=np.int32)
    out = orc.graph_propagate(N, N, eye, eye, np.ones(N), B, X, 2, 1)
    assert np.array_equal(out[-1][0], np.maximum(X, 0))


# ------------------------------------------------------------ memory by definition
# Byte counts of the definition-fixed tensors, written out by hand (not by
# the oracle's formula): int32 row and col plus one value per connection for
# the COO, one value per connection for the value gradient, M*K values for
# the dense weight and again for its gradient, one byte per weight for the
# Dense+Mask mask, and X, Y, dX, dY at the largest batch.  The SNACK
# abstract compares a 90%-sparse single layer's memory against dense; the
# second case is that point at 4096 x 4096 in fp32.
MEMORY_BY_HAND = [
    # 256 x 256 at 90%: 6,554 nnz, fp32, batch 4
    ((256, 256, 6554, 4, 4),
     {"coo": 78_648, "value_grad": 26_216, "dense_weight": 262_144, "dense_grad": 262_144,
      "mask": 65_536, "activations": 16_384}),
    # 4096 x 4096 at 90%: 1,677,722 nnz, fp32, batch 1
    ((4096, 4096, 1_677_722, 4, 1),
     {"coo": 20_132_664, "value_grad": 6_710_888, "dense_weight": 67_108_864,
      "dense_grad": 67_108_864, "mask": 16_777_216, "activations": 65_536}),
    # 4096 x 4096 at 95%: 838,861 nnz, bf16, batch 32
    ((4096, 4096, 838_861, 2, 32),
     {"coo": 8_388_610, "value_grad": 1_677_722, "dense_weight": 33_554_432,
      "dense_grad": 33_554_432, "mask": 16_777_216, "activations": 1_048_576}),
]


@pytest.mark.parametrize("args,expect", MEMORY_BY_HAND)
def test_memory_by_definition_hand_counts(orc, args, expect):
    assert orc.memory_by_definition(*args) == expect


@pytest.mark.parametrize("args,_", MEMORY_BY_HAND[:2])
def test_memory_by_definition_matches_allocated_arrays(orc, args, _):
    """The same counts as the nbytes of arrays of those shapes and dtypes
    (numpy's own bookkeeping; np.empty touches no memory)."""
    M, K, nnz, s, B = args
    ft = {4: np.float32, 2: np.uint16}[s]
    arrays = {"coo": [np.empty(nnz, np.int32), np.empty(nnz, np.int32), np.empty(nnz, ft)],
              "value_grad": [np.empty(nnz, ft)],
              "dense_weight": [np.empty((M, K), ft)], "dense_grad": [np.empty((M, K), ft)],
              "mask": [np.empty((M, K), np.uint8)],
              "activations": [np.empty((B, K), ft), np.empty((B, M), ft),
                              np.empty((B, K), ft), np.empty((B, M), ft)]}
    got = orc.memory_by_definition(M, K, nnz, s, B)
    assert got == {k: sum(a.nbytes for a in v) for k, v in arrays.items()}
    # by definition the sparse layer (COO + value gradient) at 10% density
    # with int32 indices and fp32 values holds 16 B per connection against 8 B
    # per dense weight: one fifth of the dense layer
    if (M, K, s) == (4096, 4096, 4):
        assert (got["coo"] + got["value_grad"]) * 5 == pytest.approx(
            got["dense_weight"] + got["dense_grad"], rel=1e-6)


# ------------------------------------------------------------ Adam
def test_adam_first_step_is_lr_times_sign(orc):
    """From zero moments the bias-corrected first step is g / (|g| + eps):
    lr * sign(g) when |g| >> eps (Kingma & Ba, Algorithm 1, at t = 1)."""
    rng = np.random.default_rng(3)
    g = rng.standard_normal(1000)
    w = rng.standard_normal(1000)
    z = np.zeros(1000)
    w1, m1, v1 = orc.adam_step(w, g, z, z, 1e-3, 0.9, 0.999, 1e-8, 1)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-13)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-13)
    np.testing.assert_allclose(w - w1, 1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_adam_constant_gradient_keeps_unit_steps(orc):
    """With a constant gradient the bias corrections make every step
    lr * g / (|g| + eps) (m_hat = g, v_hat = g^2 at every t)."""
    g = np.array([0.5, -2.0, 3e-3])
    w = np.zeros(3)
    m = np.zeros(3)
    v = np.zeros(3)
    for t in range(1, 8):
        w_new, m, v = orc.adam_step(w, g, m, v, 0.01, 0.9, 0.99, 1e-12, t)
        np.testing.assert_allclose(w - w_new, 0.01 * np.sign(g), rtol=1e-9)
        w = w_new
