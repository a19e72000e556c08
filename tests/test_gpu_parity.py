"""GPU parity: every entry point of the HIP library against the fp64 oracle.

Integer outputs (offsets, tiles, cut flags, column view, post-step COO,
dropped/grown lists) must be bit-exact; float outputs must satisfy
|gpu - oracle| <= tol * S per output, S = sum of |term| (tol 1e-5 for fp32,
1e-2 for bf16 values with fp32 accumulation).
"""
import functools

import numpy as np
import pytest

import synth
from gpuhelp import assert_within, from_dev, node_major, to_dev, topology, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only collection
    pytest.skip("no GPU", allow_module_level=True)

import unstructured_sparse_nn_amd as snk  # noqa: E402
from unstructured_sparse_nn_amd import binding as B  # noqa: E402


# ------------------------------------------------------------------ inputs
@functools.lru_cache(maxsize=None)
def workload(name):
    if name == "single":
        return synth.single_layer()
    if name.startswith("square"):
        _, sp, b = name.split("_")
        return synth.inference_layer(sparsity=float(sp), B=int(b))
    if name.startswith("gpt2"):
        return synth.gpt2_mlp(sparsity=float(name.split("_")[1]))
    if name.startswith("llama"):
        _, which, b = name.split("_")
        return synth.llama_proj(which=which, B=int(b))
    if name == "graph":
        return synth.graph_layer()
    raise KeyError(name)


def check_prepare(orc, w, topo):
    rp = orc.row_ptr(w.M, w.row)
    assert np.array_equal(topo.array("row_ptr").cpu().numpy(), rp)
    cp, perm, rt = orc.csc(w.K, w.row, w.col)
    assert np.array_equal(topo.array("col_ptr").cpu().numpy(), cp)
    if w.nnz:
        assert np.array_equal(topo.array("perm").cpu().numpy(), perm)
        assert np.array_equal(topo.array("row_t").cpu().numpy(), rt)
    for view, ptr, T in (("r", rp, topo.plan.tile_row), ("c", cp, topo.plan.tile_col)):
        ref = orc.partition(ptr, T)
        assert ref["P"] == (topo.plan.P_row if view == "r" else topo.plan.P_col)
        assert np.array_equal(topo.array(view + "part_seg").cpu().numpy(), ref["part_seg"])
        assert np.array_equal(topo.array(view + "part_nz").cpu().numpy(), ref["part_nz"])
        # cut flags: 1 where a cut lies inside a segment, i.e. the tiles
        # first+1 .. last of every split segment the oracle lists
        P = ref["P"]
        exp_cut = np.zeros(P + 1, dtype=np.int32)
        for f, l in zip(ref["split_first"], ref["split_last"]):
            exp_cut[f + 1:l + 1] = 1
        assert np.array_equal(topo.array(view + "cut").cpu().numpy(), exp_cut)
        has = topo.plan.has_split_row if view == "r" else topo.plan.has_split_col
        assert has == int(len(ref["split_seg"]) > 0)


def run_products(orc, w, X, dY, dt, layout, Bsz, tile=0, sddmm=True, repeat_check=False,
                 flags=0):
    nm = layout == "node"
    lay = B.NODE_MAJOR if nm else B.BATCH_MAJOR
    topo = topology(w, max(Bsz, 1), tile, flags)
    vals = to_dev(w.vals, dt)
    Xd, dYd = to_dev(X.data, dt), to_dev(dY.data, dt)
    v64 = w.vals_f64()
    Y = topo.fwd(vals, Xd, Bsz, lay)
    ref, S = orc.spmm_fwd(w.M, w.K, w.row, w.col, v64, Bsz, X.f64(), nm)
    assert_within(from_dev(Y, dt), ref, S, dt, "fwd")
    dX = topo.bwd_input(vals, dYd, Bsz, lay)
    ref, S = orc.spmm_bwd_input(w.M, w.K, w.row, w.col, v64, Bsz, dY.f64(), nm)
    assert_within(from_dev(dX, dt), ref, S, dt, "bwd_input")
    dV = None
    if sddmm:
        dV = topo.grad_vals(dYd, Xd, Bsz, lay)
        ref, S = orc.sddmm(w.M, w.K, w.row, w.col, Bsz, dY.f64(), X.f64(), nm)
        assert_within(from_dev(dV, dt), ref, S, dt, "sddmm")
    if repeat_check:  # bitwise reproducible: no order-dependent atomics
        assert torch.equal(topo.fwd(vals, Xd, Bsz, lay), Y)
        assert torch.equal(topo.bwd_input(vals, dYd, Bsz, lay), dX)
        if sddmm:
            assert torch.equal(topo.grad_vals(dYd, Xd, Bsz, lay), dV)
    return topo


# --------------------------------------------------------------- prepare
PREP_CASES = [
    ("single", 0), ("single", 16), ("single", 1), ("square_0.95_1", 0), ("square_0.99_1", 0),
    ("llama_up_1", 0), ("llama_down_1", 0), ("graph", 0),
]


@pytest.mark.parametrize("name,tile", PREP_CASES)
def test_prepare_matches_oracle(orc, name, tile):
    w = workload(name).weights[0]
    topo = topology(w, 1, tile)
    check_prepare(orc, w, topo)


EDGE = [  # (M, K, nnz, tile)
    (1, 1, 0, 0), (1, 1, 1, 0), (5, 7, 0, 2), (1, 64, 64, 0), (1, 64, 64, 5), (64, 1, 64, 3),
    (13, 11, 143, 4), (300, 40, 30, 7), (257, 255, 3000, 64), (1000, 3, 2500, 128),
]


@pytest.mark.parametrize("M,K,nnz,tile", EDGE)
def test_prepare_edge_cases(orc, M, K, nnz, tile):
    w = synth.random_case(21, M, K, nnz, 1).weights[0]
    check_prepare(orc, w, topology(w, 1, tile))


def test_prepare_rejects_bad_coo():
    row = to_dev(np.array([0, 0, 1], np.int32))
    for col, status in (([1, 1, 0], -6), ([2, 1, 0], -6), ([0, 5, 0], -5), ([-1, 1, 0], -5)):
        c = to_dev(np.array(col, np.int32))
        plan = snk.snack_plan_init(4, 4, 3, 1)
        arena = torch.empty(plan.arena_bytes, dtype=torch.uint8, device="cuda")
        with pytest.raises(snk.SnackError) as e:
            snk.snack_coo_prepare(plan, row, c, arena)
        assert e.value.status == status
    rowbad = to_dev(np.array([1, 0, 2], np.int32))
    c = to_dev(np.array([0, 1, 2], np.int32))
    plan = snk.snack_plan_init(4, 4, 3, 1)
    arena = torch.empty(plan.arena_bytes, dtype=torch.uint8, device="cuda")
    with pytest.raises(snk.SnackError) as e:
        snk.snack_coo_prepare(plan, rowbad, c, arena)
    assert e.value.status == -6


# --------------------------------------------------------------- products
SMALL = [  # (M, K, nnz, B, dtype, layout, tile)
    (1, 1, 1, 1, "f32", "batch", 0),
    (1, 1, 0, 3, "f32", "batch", 0),
    (5, 7, 0, 2, "bf16", "node", 2),
    (1, 64, 64, 4, "f32", "batch", 5),      # one dense row split over many tiles
    (64, 1, 64, 4, "f32", "node", 3),       # one dense column split over many tiles
    (13, 11, 143, 3, "f32", "batch", 4),    # full density, odd batch
    (37, 53, 200, 1, "bf16", "batch", 0),
    (300, 40, 30, 2, "f32", "batch", 7),    # mostly empty rows
    (257, 255, 3000, 8, "bf16", "batch", 64),
    (257, 255, 3000, 12, "bf16", "node", 0),
    (511, 129, 9000, 32, "bf16", "node", 256),
    (511, 129, 9000, 32, "f32", "batch", 256),
    (100, 333, 8000, 33, "f32", "node", 100),
    (100, 333, 8000, 64, "f32", "node", 0),
    (100, 333, 8000, 5, "bf16", "batch", 1),
    (1000, 3, 2500, 16, "bf16", "node", 128),
    # tiles of >= 256 items (column view with deferred values), columns split
    (2000, 2, 3000, 8, "bf16", "node", 256),
    (2000, 3, 5000, 5, "f32", "batch", 512),
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt,layout,tile", SMALL)
def test_products_small_and_ragged(orc, M, K, nnz, Bsz, dt, layout, tile):
    w = synth.random_case(5, M, K, nnz, Bsz, dt, layout)
    run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, layout, Bsz, tile, repeat_check=True)


def test_products_skewed_rows_with_splits(orc):
    """Rows of 1 .. 3000 entries, tiles of 64 items: many rows span several
    tiles; their tile pieces go through the carry slots and the fix-up (wide
    batches in several passes)."""
    M, K = 400, 3000
    deg = synth.rank_profile(M, K, 60000, 1.3)
    rng = np.random.default_rng(3)
    lin = np.concatenate([r * K + np.sort(rng.choice(K, d, replace=False))
                          for r, d in enumerate(rng.permutation(deg))])
    for dt, layout, Bsz in (("f32", "batch", 3), ("bf16", "node", 16), ("f32", "node", 32),
                            ("f32", "node", 100), ("bf16", "batch", 64)):
        w = synth.random_case(7, M, K, lin.size, Bsz, dt, layout, positions=lin)
        topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, layout, Bsz, tile=64,
                            repeat_check=True)
        assert topo.plan.has_split_row == 1


def test_products_skewed_columns_with_splits(orc):
    """Columns of 1 .. 3000 entries, tiles of 64 items: the input gradient's
    long columns are summed as tile pieces by the first workgroups of the
    launch that runs the short ones, in the die-contiguous block order (400
    columns), with piece workgroups past the last tile."""
    M, K = 3000, 400
    deg = synth.rank_profile(K, M, 60000, 1.3)
    rng = np.random.default_rng(4)
    lin = np.sort(np.concatenate([np.sort(rng.choice(M, d, replace=False)) * K + c
                                  for c, d in enumerate(rng.permutation(deg))]))
    for dt, layout, Bsz in (("f32", "batch", 3), ("bf16", "node", 16), ("f32", "node", 32),
                            ("bf16", "node", 1), ("f32", "node", 100)):
        w = synth.random_case(8, M, K, lin.size, Bsz, dt, layout, positions=lin)
        topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, layout, Bsz, tile=64,
                            repeat_check=True)
        assert topo.plan.has_split_col == 1


@pytest.mark.parametrize("name,B", [("single", 4)])
def test_single_layer_config(orc, name, B):
    w = workload(name)
    run_products(orc, w.weights[0], w.X[0], w.dY[0], "f32", "batch", B, repeat_check=True)


@pytest.mark.parametrize("sp", ["0.95", "0.99"])
@pytest.mark.parametrize("Bsz", [1, 8, 32])
def test_square_inference_configs(orc, sp, Bsz):
    w = workload(f"square_{sp}_{Bsz}")
    run_products(orc, w.weights[0], w.X[0], w.dY[0], "bf16", "batch", Bsz, repeat_check=True)


@pytest.mark.parametrize("sp", ["0.95", "0.99"])
@pytest.mark.parametrize("Bsz", [1, 8, 32])
def test_square_node_major_benchmarked_path(orc, sp, Bsz):
    """The layer and launch configuration the benchmark times: 4096^2,
    node-major activations, a plan without batch-major scratch."""
    w = workload(f"square_{sp}_{Bsz}")
    topo = run_products(orc, w.weights[0], node_major(w.X[0]), node_major(w.dY[0]), "bf16",
                        "node", Bsz, repeat_check=True, flags=B.PLAN_NODE_MAJOR_ONLY)
    assert topo.plan.has_split_row == 0 and topo.plan.has_split_col == 0


LDS_CASES = [
    # M, K, nnz, B, dtype: layers with >= 16,384 segments whose whole
    # node-major input fits in LDS take the LDS-staged wave kernel
    (16384, 3001, 200000, 1, "bf16"),    # forward staged; 6,002-byte input (ragged tail)
    (3001, 20000, 300000, 4, "f32"),     # input gradient staged (dY: 3,001 x 4 fp32, 48 KB)
    (32768, 2048, 1000000, 16, "bf16"),  # forward staged, exactly 64 KB, two lanes per entry
    (32768, 32768, 10737418, 1, "bf16"),  # 32768^2 at 99%: the size sweep's largest layer
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt", LDS_CASES)
def test_wave_lds_staged_inputs(orc, M, K, nnz, Bsz, dt):
    w = synth.random_case(24, M, K, nnz, Bsz, dt, "node")
    topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, "node", Bsz, repeat_check=True,
                        flags=B.PLAN_NODE_MAJOR_ONLY)
    assert topo.plan.has_split_row == 0


LDS_MID_CASES = [
    # M, K, nnz, B, dtype: 2,048-16,383 segments averaging >= 256 entries with
    # inputs of 16-160 KB also take the LDS-staged kernels: rows (forward and
    # value gradient) stage 32-64 KB, columns (input gradient) stage 128 KB,
    # one workgroup per CU with one lane per entry
    (8192, 2048, 2_200_000, 8, "bf16"),
    (8192, 4096, 2_200_000, 4, "f32"),
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt", LDS_MID_CASES)
def test_wave_lds_staged_mid_sized_views(orc, M, K, nnz, Bsz, dt):
    w = synth.random_case(26, M, K, nnz, Bsz, dt, "node")
    wt = w.weights[0]
    topo = run_products(orc, wt, w.X[0], w.dY[0], dt, "node", Bsz, repeat_check=True,
                        flags=B.PLAN_NODE_MAJOR_ONLY)
    assert topo.plan.has_split_row == 0 and topo.plan.has_split_col == 0
    vals = to_dev(wt.vals, dt)
    dX = topo.bwd_input_t(topo.gather_vals_t(vals), to_dev(w.dY[0].data, dt), Bsz, B.NODE_MAJOR)
    ref, S = orc.spmm_bwd_input(M, K, wt.row, wt.col, wt.vals_f64(), Bsz, w.dY[0].f64(), True)
    assert_within(from_dev(dX, dt), ref, S, dt, "bwd_input_t")


LARGE_CASES = [  # (M, K, nnz, B, dtype, layout): >= 16,384 segments, inputs over 64 KB
    (16500, 20000, 1_300_000, 8, "bf16", "node"),
    (16384, 16384, 1_000_000, 32, "bf16", "node"),
    (16384, 16384, 800_000, 4, "f32", "node"),
    (16390, 16500, 500_000, 16, "bf16", "batch"),   # batch-major in and out
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt,layout", LARGE_CASES)
def test_large_layers_small_batches(orc, M, K, nnz, Bsz, dt, layout):
    """Large layers at batches 4 to 32, whose node-major input does not fit
    LDS: the gather kernels (forward, input gradient through perm and from
    column-ordered values, forward with ReLU)."""
    w = synth.random_case(28, M, K, nnz, Bsz, dt, layout)
    wt = w.weights[0]
    topo = run_products(orc, wt, w.X[0], w.dY[0], dt, layout, Bsz, sddmm=False,
                        repeat_check=True)
    assert topo.plan.has_split_row == 0 and topo.plan.has_split_col == 0
    nm = layout == "node"
    lay = B.NODE_MAJOR if nm else B.BATCH_MAJOR
    vals = to_dev(wt.vals, dt)
    dYd, Xd = to_dev(w.dY[0].data, dt), to_dev(w.X[0].data, dt)
    dX = topo.bwd_input_t(topo.gather_vals_t(vals), dYd, Bsz, lay)
    ref, S = orc.spmm_bwd_input(M, K, wt.row, wt.col, wt.vals_f64(), Bsz, w.dY[0].f64(), nm)
    assert_within(from_dev(dX, dt), ref, S, dt, "bwd_input_t")
    Y = torch.empty(Bsz * M, dtype=Xd.dtype, device="cuda")
    snk.snack_spmm_fwd_act(topo.plan, vals, Xd, lay, Bsz, Y, snk.ACT_RELU)
    ref, S = orc.spmm_fwd(M, K, wt.row, wt.col, wt.vals_f64(), Bsz, w.X[0].f64(), nm)
    assert_within(from_dev(Y, dt), np.maximum(ref, 0.0), S, dt, "fwd relu")


WIDE_CASES = [  # (M, K, nnz, B, dtype, layout): batches of several 64-column passes
    (300, 700, 21000, 128, "f32", "node"),
    (300, 700, 21000, 192, "f32", "batch"),    # batch-major through the node-major copy
    (96, 3000, 28800, 256, "bf16", "node"),    # rows of ~300 entries kept whole (wide tiles)
    (2000, 1500, 30000, 128, "bf16", "node"),
    (5000, 40, 20000, 256, "bf16", "node"),    # columns of ~500 entries kept whole
    (64, 64, 0, 128, "f32", "node"),           # no entries: zeros
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt,layout", WIDE_CASES)
def test_wide_batches(orc, M, K, nnz, Bsz, dt, layout):
    """Batches of 128 or more run in 64-column passes on plans whose wide
    tiles keep uniform segments whole (no split, no fix-up); also the input
    gradient from column-ordered values."""
    w = synth.random_case(27, M, K, nnz, Bsz, dt, layout)
    wt = w.weights[0]
    topo = run_products(orc, wt, w.X[0], w.dY[0], dt, layout, Bsz, repeat_check=True)
    assert topo.plan.has_split_row == 0 and topo.plan.has_split_col == 0
    lay = B.NODE_MAJOR if layout == "node" else B.BATCH_MAJOR
    vals = to_dev(wt.vals, dt)
    dX = topo.bwd_input_t(topo.gather_vals_t(vals), to_dev(w.dY[0].data, dt), Bsz, lay)
    ref, S = orc.spmm_bwd_input(M, K, wt.row, wt.col, wt.vals_f64(), Bsz, w.dY[0].f64(),
                                layout == "node")
    assert_within(from_dev(dX, dt), ref, S, dt, "bwd_input_t")


@pytest.mark.parametrize("which", ["up", "down"])
@pytest.mark.parametrize("Bsz", [1, 4, 16])
def test_llama_projection_configs(orc, which, Bsz):
    w = workload(f"llama_{which}_{Bsz}")
    topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], "bf16", "batch", Bsz,
                        repeat_check=True)
    assert topo.plan.has_split_row == 1  # dense rows longer than a tile


@pytest.mark.parametrize("which", ["up", "down"])
@pytest.mark.parametrize("Bsz", [1, 4, 16])
def test_llama_projection_node_major(orc, which, Bsz):
    """The LLaMA-shaped layers as the benchmark runs them: node-major, no
    batch-major scratch, split rows through the tile pieces and the fix-up."""
    w = workload(f"llama_{which}_{Bsz}")
    topo = run_products(orc, w.weights[0], node_major(w.X[0]), node_major(w.dY[0]), "bf16",
                        "node", Bsz, repeat_check=True, flags=B.PLAN_NODE_MAJOR_ONLY)
    assert topo.plan.has_split_row == 1


def test_graph_config(orc):
    w = workload("graph")
    topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], "f32", "node", 128, sddmm=True)
    assert topo.plan.has_split_row == 1


@pytest.mark.parametrize("sp", ["0.9", "0.99"])
def test_gpt2_mlp_chain(orc, sp):
    """fwd W1 -> GELU -> fwd W2, then the full backward, each op gated on the
    oracle with the GPU's own intermediates as inputs."""
    w = workload(f"gpt2_{sp}")
    W1, W2 = w.weights
    Bsz = w.B
    X, G = w.X[0], w.dY[1]
    t1, t2 = topology(W1, Bsz), topology(W2, Bsz)
    v1, v2 = to_dev(W1.vals), to_dev(W2.vals)
    Xd, Gd = to_dev(X.data), to_dev(G.data)
    Z = t1.fwd(v1, Xd, Bsz)
    ref, S = orc.spmm_fwd(W1.M, W1.K, W1.row, W1.col, W1.vals_f64(), Bsz, X.f64())
    assert_within(from_dev(Z, "f32"), ref, S, "f32", "fwd W1")
    H = torch.empty_like(Z)
    snk.snack_gelu_fwd(Z, H)
    z64 = from_dev(Z, "f32")
    np.testing.assert_allclose(from_dev(H, "f32"), orc.gelu(z64), rtol=2e-6, atol=1e-7)
    Y = t2.fwd(v2, H, Bsz)
    h64 = from_dev(H, "f32")
    ref, S = orc.spmm_fwd(W2.M, W2.K, W2.row, W2.col, W2.vals_f64(), Bsz, h64)
    assert_within(from_dev(Y, "f32"), ref, S, "f32", "fwd W2")
    dH = t2.bwd_input(v2, Gd, Bsz)
    ref, S = orc.spmm_bwd_input(W2.M, W2.K, W2.row, W2.col, W2.vals_f64(), Bsz, G.f64())
    assert_within(from_dev(dH, "f32"), ref, S, "f32", "dX W2")
    dV2 = t2.grad_vals(Gd, H, Bsz)
    ref, S = orc.sddmm(W2.M, W2.K, W2.row, W2.col, Bsz, G.f64(), h64)
    assert_within(from_dev(dV2, "f32"), ref, S, "f32", "dW W2")
    dZ = torch.empty_like(Z)
    snk.snack_gelu_bwd(Z, dH, dZ)
    dh64 = from_dev(dH, "f32")
    np.testing.assert_allclose(from_dev(dZ, "f32"), orc.gelu_bwd(z64, dh64), rtol=4e-6,
                               atol=1e-6 * np.abs(dh64).max())
    dX = t1.bwd_input(v1, dZ, Bsz)
    dz64 = from_dev(dZ, "f32")
    ref, S = orc.spmm_bwd_input(W1.M, W1.K, W1.row, W1.col, W1.vals_f64(), Bsz, dz64)
    assert_within(from_dev(dX, "f32"), ref, S, "f32", "dX W1")
    dV1 = t1.grad_vals(dZ, Xd, Bsz)
    ref, S = orc.sddmm(W1.M, W1.K, W1.row, W1.col, Bsz, dz64, X.f64())
    assert_within(from_dev(dV1, "f32"), ref, S, "f32", "dW W1")


def test_node_major_only_plan(orc):
    w = synth.random_case(3, 200, 300, 5000, 8, "bf16", "node")
    wt = w.weights[0]
    topo = snk.Topology(to_dev(wt.row), to_dev(wt.col), wt.M, wt.K, 8, flags=1)
    vals = to_dev(wt.vals, "bf16")
    Y = topo.fwd(vals, to_dev(w.X[0].data, "bf16"), 8, B.NODE_MAJOR)
    ref, S = orc.spmm_fwd(wt.M, wt.K, wt.row, wt.col, wt.vals_f64(), 8, w.X[0].f64(), True)
    assert_within(from_dev(Y, "bf16"), ref, S, "bf16", "fwd node-major-only plan")
    with pytest.raises(snk.SnackError) as e:
        topo.fwd(vals, to_dev(w.X[0].data, "bf16"), 8, B.BATCH_MAJOR)
    assert e.value.status == -9
    # B == 1: both layouts are the same vector, no scratch needed
    topo.fwd(vals, to_dev(w.X[0].data[:wt.K], "bf16"), 1, B.BATCH_MAJOR)


def test_zero_batch_and_empty_weight(orc):
    w = synth.random_case(2, 30, 20, 50, 1).weights[0]
    topo = topology(w, 4)
    vals = to_dev(w.vals)
    dV = torch.full((w.nnz,), 7.0, device="cuda")
    topo.grad_vals(torch.empty(0, device="cuda"), torch.empty(0, device="cuda"), 0, out=dV)
    assert torch.count_nonzero(dV) == 0
    Y = torch.full((0,), 1.0, device="cuda")
    topo.fwd(vals, torch.empty(0, device="cuda"), 0, out=Y)
    e = synth.random_case(2, 30, 20, 0, 3)
    topo = topology(e.weights[0], 3)
    Y = torch.full((3 * 30,), 5.0, device="cuda")
    topo.fwd(torch.empty(0, device="cuda"), to_dev(e.X[0].data), 3, out=Y)
    assert torch.count_nonzero(Y) == 0
    with pytest.raises(snk.SnackError) as ex:
        topo.fwd(torch.empty(0, device="cuda"), to_dev(e.X[0].data), 4, out=Y)
    assert ex.value.status == -2


# ------------------------------------------------- values in column order
def bits_of(t, dt):
    """Raw bits of a float tensor (bitwise comparisons)."""
    return (t.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16"
            else t.view(torch.int32).cpu().numpy().view(np.uint32))


VALS_T_CASES = [
    # name, dtype, layout, batch, tile, flags
    ("square_0.95_32", "bf16", "node", 32, 0, B.PLAN_NODE_MAJOR_ONLY),
    ("square_0.99_1", "bf16", "node", 1, 0, B.PLAN_NODE_MAJOR_ONLY),
    ("llama_up_1", "bf16", "node", 1, 0, B.PLAN_NODE_MAJOR_ONLY),
    ("llama_down_4", "bf16", "node", 4, 0, B.PLAN_NODE_MAJOR_ONLY),
    ("single", "f32", "batch", 4, 0, 0),
    ("ragged", "f32", "node", 5, 64, 0),      # split columns: tile pieces and the fix-up
    ("ragged", "bf16", "batch", 33, 0, 0),    # odd batch above 16: the merge-path kernel
    ("ragged", "f32", "node", 100, 64, 0),    # wide batch in passes, split columns
]


@pytest.mark.parametrize("name,dt,layout,Bsz,tile,flags", VALS_T_CASES)
def test_bwd_input_from_column_ordered_values(orc, name, dt, layout, Bsz, tile, flags):
    """snack_gather_vals_t is vals[perm] bit for bit, and the input gradient
    from it matches the oracle and equals, bit for bit, the one that reads the
    values through perm (same entries, same order, same reduction tree)."""
    if name == "ragged":
        w = synth.random_case(19, 300, 200, 9000, Bsz, dt, layout)
        wt, dY = w.weights[0], w.dY[0]
    else:
        w = workload(name)
        wt = w.weights[0]
        dY = node_major(w.dY[0]) if layout == "node" else w.dY[0]
    nm = layout == "node"
    lay = B.NODE_MAJOR if nm else B.BATCH_MAJOR
    topo = topology(wt, Bsz, tile, flags)
    vals = to_dev(wt.vals, dt)
    vt = topo.gather_vals_t(vals)
    _, perm, _ = orc.csc(wt.K, wt.row, wt.col)
    assert np.array_equal(bits_of(vt, dt), bits_of(vals, dt)[perm])
    dYd = to_dev(dY.data, dt)
    dX = topo.bwd_input_t(vt, dYd, Bsz, lay)
    ref, S = orc.spmm_bwd_input(wt.M, wt.K, wt.row, wt.col, wt.vals_f64(), Bsz, dY.f64(), nm)
    assert_within(from_dev(dX, dt), ref, S, dt, "bwd_input_t")
    assert torch.equal(topo.bwd_input(vals, dYd, Bsz, lay), dX)
    assert torch.equal(topo.bwd_input_t(vt, dYd, Bsz, lay), dX)


@pytest.mark.parametrize("dt,layout,Bsz,tile,lr", [
    ("bf16", "node", 32, 0, 0.05), ("f32", "batch", 4, 0, 0.1), ("bf16", "batch", 8, 0, 0.0),
    ("f32", "node", 5, 64, 0.1),   # split columns: merge-path form, copy refreshed by a gather
])
def test_bwd_fused_keeps_column_ordered_values(orc, dt, layout, Bsz, tile, lr):
    """With vals_t, the fused backward reads the column-ordered values and its
    SGD step updates both copies; results equal those of the call without it,
    bit for bit, over two steps."""
    w = synth.random_case(20, 512, 384, 20000, Bsz, dt, layout)
    wt = w.weights[0]
    lay = B.NODE_MAJOR if layout == "node" else B.BATCH_MAJOR
    topo = topology(wt, Bsz, tile)
    X, dY = to_dev(w.X[0].data, dt), to_dev(w.dY[0].data, dt)
    v1, v2 = to_dev(wt.vals, dt), to_dev(wt.vals, dt)
    vt = topo.gather_vals_t(v2)
    _, perm, _ = orc.csc(wt.K, wt.row, wt.col)
    for _ in range(2):
        outs = []
        for v, t in ((v1, None), (v2, vt)):
            dX = torch.empty(Bsz * wt.K, dtype=torch_dtype(dt), device="cuda")
            dV = torch.empty(wt.nnz, dtype=torch_dtype(dt), device="cuda")
            snk.snack_spmm_bwd_fused(topo.plan, v, X, dY, lay, Bsz, dX, dV, lr, vals_t=t)
            outs.append((dX, dV))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
        assert torch.equal(v1, v2)
        assert np.array_equal(bits_of(vt, dt), bits_of(v2, dt)[perm])
    ref, S = orc.spmm_bwd_input(wt.M, wt.K, wt.row, wt.col, wt.vals_f64(), Bsz, w.dY[0].f64(),
                                layout == "node")
    if lr == 0.0:
        assert_within(from_dev(outs[1][0], dt), ref, S, dt, "fused dX with vals_t")


# --------------------------------------------------------------- prune / regrow
@pytest.fixture(params=["auto", "sort"])
def prune_plan(request):
    """Restructure flags of a prune test: the library's own plan choice (the
    bitmap plan for every layer density <= 1/4 here), and again forced onto
    the sort plan."""
    return B.PRUNE_SORT_PLAN if request.param == "sort" else 0


def gpu_prune(w, dt, n_drop, seed, step, vals=None, flags=0):
    row, col = to_dev(w.row), to_dev(w.col)
    v = to_dev(w.vals if vals is None else vals, dt)
    ws = torch.empty(snk.snack_prune_regrow_workspace(w.M, w.K, w.nnz, n_drop, flags),
                     dtype=torch.uint8, device="cuda")
    dl = torch.empty(max(n_drop, 1), dtype=torch.int64, device="cuda")
    gl = torch.empty(max(n_drop, 1), dtype=torch.int64, device="cuda")
    snk.snack_prune_regrow(row, col, v, w.M, w.K, w.nnz, n_drop, seed, step, dl, gl, ws,
                           flags=flags)
    return row, col, v, dl[:n_drop], gl[:n_drop]


def check_prune(orc, w, dt, ppm, seed, step, vals=None, flags=0):
    n_drop = orc.drop_count(w.nnz, ppm)
    vals = w.vals if vals is None else vals
    ref = orc.prune_regrow(w.M, w.K, w.row, w.col, vals, dt, n_drop, seed, step)
    assert ref["rc"] == 0
    row, col, v, dl, gl = gpu_prune(w, dt, n_drop, seed, step, vals, flags)
    assert np.array_equal(row.cpu().numpy(), ref["row"])
    assert np.array_equal(col.cpu().numpy(), ref["col"])
    if dt == "bf16":
        got = v.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = v.cpu().numpy().view(np.uint32)
        ref["vals"] = np.asarray(ref["vals"], np.float32).view(np.uint32)
    assert np.array_equal(got, ref["vals"])
    assert np.array_equal(dl.cpu().numpy(), ref["dropped"])
    assert np.array_equal(gl.cpu().numpy(), ref["grown"])
    return row, col


def test_prune_regrow_single_layer(orc, prune_plan):
    w = workload("single").weights[0]
    check_prune(orc, w, "f32", 100000, 0, 1, flags=prune_plan)


@pytest.mark.parametrize("sp", ["0.9", "0.99"])
def test_prune_regrow_gpt2(orc, sp, prune_plan):
    for W in workload(f"gpt2_{sp}").weights:
        row, col = check_prune(orc, W, "f32", 300000, 0, 5, flags=prune_plan)
        # the restructured COO prepares exactly as the oracle says
        w2 = synth.SparseWeight(W.M, W.K, row.cpu().numpy(), col.cpu().numpy(), W.vals, "f32")
        check_prepare(orc, w2, topology(w2, 1))


def test_prune_regrow_bf16_ties_and_signed_zero(orc, prune_plan):
    w = synth.random_case(8, 300, 200, 5000, 1, "bf16").weights[0]
    vals = w.vals.copy()
    vals[::7] = vals[3]                    # many exact ties
    vals[1::11] = np.uint16(0x8000)        # -0
    vals[2::13] = np.uint16(0)             # +0
    check_prune(orc, w, "bf16", 250000, 42, 9, vals, flags=prune_plan)


def test_prune_regrow_square_bf16(orc, prune_plan):
    w = workload("square_0.95_1").weights[0]
    check_prune(orc, w, "bf16", 300000, 3, 1, flags=prune_plan)


def test_prune_regrow_nearly_full_needs_several_chunks(orc, prune_plan):
    """Only a few free positions: the candidate stream runs over many chunks."""
    M, K = 40, 60
    nnz = M * K - 30
    w = synth.random_case(9, M, K, nnz, 1).weights[0]
    check_prune(orc, w, "f32", 10000, 5, 2, flags=prune_plan)


def test_prune_regrow_rejects_nan_and_keeps_coo(prune_plan):
    w = synth.random_case(4, 64, 64, 400, 1).weights[0]
    vals = w.vals.copy()
    vals[17] = np.nan
    row, col = to_dev(w.row), to_dev(w.col)
    v = to_dev(vals)
    ws = torch.empty(snk.snack_prune_regrow_workspace(64, 64, 400, 40, prune_plan),
                     dtype=torch.uint8, device="cuda")
    with pytest.raises(snk.SnackError) as e:
        snk.snack_prune_regrow(row, col, v, 64, 64, 400, 40, 1, 1, None, None, ws,
                               flags=prune_plan)
    assert e.value.status == -7
    assert np.array_equal(row.cpu().numpy(), w.row) and np.array_equal(col.cpu().numpy(), w.col)


def test_prune_regrow_huge_sparse_grid_takes_sort_plan(orc):
    """A 100,000 x 100,000 grid with 2,000 entries: a support bitmap would be
    far larger than the COO, so the sort plan runs by itself."""
    w = synth.random_case(11, 100000, 100000, 2000, 1, "bf16").weights[0]
    check_prune(orc, w, "bf16", 300000, 7, 3)


def test_prune_regrow_without_lists_and_second_step(orc, prune_plan):
    """Nullable dropped/grown outputs, then a second step on the result."""
    w = workload("single").weights[0]
    n_drop = orc.drop_count(w.nnz, 100000)
    row, col, v = to_dev(w.row), to_dev(w.col), to_dev(w.vals)
    ws = torch.empty(snk.snack_prune_regrow_workspace(w.M, w.K, w.nnz, n_drop, prune_plan),
                     dtype=torch.uint8, device="cuda")
    snk.snack_prune_regrow(row, col, v, w.M, w.K, w.nnz, n_drop, 0, 1, None, None, ws,
                           flags=prune_plan)
    ref = orc.prune_regrow(w.M, w.K, w.row, w.col, w.vals, "f32", n_drop, 0, 1)
    assert np.array_equal(row.cpu().numpy(), ref["row"])
    assert np.array_equal(col.cpu().numpy(), ref["col"])
    snk.snack_prune_regrow(row, col, v, w.M, w.K, w.nnz, n_drop, 0, 2, None, None, ws,
                           flags=prune_plan)
    ref2 = orc.prune_regrow(w.M, w.K, ref["row"], ref["col"],
                            np.asarray(ref["vals"], np.float32), "f32", n_drop, 0, 2)
    assert np.array_equal(row.cpu().numpy(), ref2["row"])
    assert np.array_equal(col.cpu().numpy(), ref2["col"])
    assert np.array_equal(v.cpu().numpy().view(np.uint32),
                          np.asarray(ref2["vals"], np.float32).view(np.uint32))


def test_prune_regrow_rejects_invalid_coo_on_bitmap_plan():
    """The bitmap plan validates the COO while building the support bitmap:
    a repeated entry is reported and the COO is left as it was."""
    w = synth.random_case(4, 64, 64, 400, 1).weights[0]
    r, c = w.row.copy(), w.col.copy()
    r[10], c[10] = r[9], c[9]
    row, col, v = to_dev(r), to_dev(c), to_dev(w.vals)
    ws = torch.empty(snk.snack_prune_regrow_workspace(64, 64, 400, 40), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(snk.SnackError) as e:
        snk.snack_prune_regrow(row, col, v, 64, 64, 400, 40, 1, 1, None, None, ws)
    assert e.value.status == -6
    assert np.array_equal(row.cpu().numpy(), r) and np.array_equal(col.cpu().numpy(), c)


PREPARED_CASES = [
    ("single", "f32", 100000, 0, 1, 0),          # 256 x 256: fused
    ("gpt2_0.9", "f32", 300000, 0, 5, 0),        # 3072 x 768: fused
    ("square_0.95_32", "bf16", 300000, 3, 2, 0),  # 4096 x 4096: fused
    ("ragged", "bf16", 250000, 4, 7, 0),         # 300 x 200: not multiples of 32, two calls
    ("single", "f32", 100000, 2, 3, 64),         # small tiles: rows and columns split
    # density 1/4, every entry dropped: acceptance near 1/2.  bf16 (3 chunks
    # on the entry kernels) needs stand-alone chunk launches and the finisher;
    # fp32 (5 chunks) ends in the drop kernel's tail
    ("quarter_all", "bf16", 1000000, 6, 1, 0),
    ("quarter_all", "f32", 1000000, 6, 1, 0),
    # 8192 x 8448 at 2.9%: past 2^26 positions, so regrow chunk 0 takes the
    # grid-wide atomic path instead of the per-region buckets
    ("wide_grid", "bf16", 300000, 5, 3, 0),
    # 4096 x 4096 at 10%: 503,316 draws in chunk 0, more bucketing slices
    # than half the region workgroup's threads, so the region pass maps its
    # candidates by scan and search (at 5% each slice gets two threads)
    ("square_0.9_many_slices", "bf16", 300000, 10, 1, 0),
    # without the dropped and grown lists (the emitter instance the training
    # step runs)
    ("square_0.95_32_nolists", "bf16", 300000, 3, 2, 0),
    # 12288 rows: the most the column emitter stages; 3 column words, so each
    # workgroup writes 1,025 row pointers (more than its threads)
    ("rows_at_max", "bf16", 300000, 8, 1, 0),
    # 12320 rows: past it, so the transposed bitmap and its emitter run
    ("rows_past_max", "bf16", 300000, 9, 1, 0),
    ("rows_past_max_nolists", "f32", 300000, 9, 2, 0),
]


@pytest.mark.parametrize("name,dt,ppm,seed,step,tile", PREPARED_CASES)
def test_prune_regrow_prepared(orc, prune_plan, name, dt, ppm, seed, step, tile):
    """The fused restructure leaves exactly the COO of the oracle's step and
    the plan snack_coo_prepare would build for it, and the products on that
    plan match the oracle."""
    if name == "ragged":
        w = synth.random_case(12, 300, 200, 6000, 1, dt).weights[0]
    elif name == "quarter_all":
        w = synth.random_case(12, 512, 512, 512 * 512 // 4, 1, dt).weights[0]
    elif name == "wide_grid":
        w = synth.random_case(12, 8192, 8448, 2000000, 1, dt).weights[0]
    elif name == "square_0.9_many_slices":
        w = synth.random_case(15, 4096, 4096, 4096 * 4096 // 10, 1, dt).weights[0]
    elif name == "rows_at_max":
        w = synth.random_case(13, 12288, 96, 12288 * 96 // 20, 1, dt).weights[0]
    elif name.startswith("rows_past_max"):
        w = synth.random_case(14, 12320, 256, 12320 * 256 // 20, 1, dt).weights[0]
    else:
        w = workload(name.replace("_nolists", "")).weights[0]
    lists = not name.endswith("_nolists")
    n_drop = orc.drop_count(w.nnz, ppm)
    ref = orc.prune_regrow(w.M, w.K, w.row, w.col, w.vals, dt, n_drop, seed, step)
    assert ref["rc"] == 0
    topo = topology(w, 4, tile)
    v = to_dev(w.vals, dt)
    ws = torch.empty(snk.snack_prune_regrow_workspace(w.M, w.K, w.nnz, n_drop, prune_plan),
                     dtype=torch.uint8, device="cuda")
    dl = torch.empty(n_drop, dtype=torch.int64, device="cuda") if lists else None
    gl = torch.empty(n_drop, dtype=torch.int64, device="cuda") if lists else None
    vt = torch.full_like(v, 3.0)  # receives the new values in the new column order
    snk.snack_prune_regrow_prepared(topo.plan, topo.row, topo.col, v, n_drop, seed, step, dl, gl,
                                    ws, vals_t=vt, flags=prune_plan)
    assert np.array_equal(topo.row.cpu().numpy(), ref["row"])
    assert np.array_equal(topo.col.cpu().numpy(), ref["col"])
    if lists:
        assert np.array_equal(dl.cpu().numpy(), ref["dropped"])
        assert np.array_equal(gl.cpu().numpy(), ref["grown"])
    w2 = synth.SparseWeight(w.M, w.K, ref["row"], ref["col"], ref["vals"], dt)
    check_prepare(orc, w2, topo)
    _, perm, _ = orc.csc(w.K, ref["row"], ref["col"])
    assert np.array_equal(bits_of(vt, dt), bits_of(v, dt)[perm])
    xf = np.random.default_rng(14).standard_normal(4 * w.K).astype(np.float32)
    Xa = synth.Activation(xf if dt == "f32" else synth.f32_to_bf16_bits(xf), dt, 4, w.K,
                          "batch")
    Y = topo.fwd(v, to_dev(Xa.data, dt), 4, B.BATCH_MAJOR)
    r, S = orc.spmm_fwd(w.M, w.K, ref["row"], ref["col"], w2.vals_f64(), 4, Xa.f64(), False)
    assert_within(from_dev(Y, dt), r, S, dt, "fwd after restructure")


def test_prune_regrow_prepared_rejects_unprepared_plan():
    plan = snk.snack_plan_init(64, 64, 400, 1)
    row = torch.zeros(400, dtype=torch.int32, device="cuda")
    with pytest.raises(snk.SnackError) as e:
        snk.snack_prune_regrow_prepared(plan, row, row, torch.zeros(400, device="cuda"), 40, 1, 1,
                                        None, None, None)
    assert e.value.status == -12


FUSED_BWD = [
    # name, dtype, layout, batch, tile, lr
    ("single", "f32", "batch", 4, 0, 0.0),
    ("single", "f32", "batch", 4, 0, 0.05),
    ("square_0.95_32", "bf16", "batch", 32, 0, 0.0),
    ("square_0.95_1", "bf16", "batch", 1, 0, 0.01),
    ("square_0.99_8", "bf16", "batch", 8, 0, 0.01),
    ("ragged", "f32", "node", 5, 64, 0.1),    # small tiles: split columns and the fix-up
    ("ragged", "bf16", "batch", 3, 64, 0.1),
    ("ragged", "bf16", "node", 32, 0, 0.2),
    ("skewed", "f32", "batch", 16, 64, 0.1),   # one dense column spanning many tiles
    # columns of ~750 entries kept whole (wave path over several load batches)
    ("long", "bf16", "node", 32, 2048, 0.1),
    ("long", "f32", "batch", 7, 2048, 0.0),
    # larger layers: 2,048-4,096 columns of ~500-1,100 entries, 2.2 M values
    # updated in place through perm
    ("wide", "bf16", "node", 8, 0, 0.05),
    ("wide_f32", "f32", "node", 4, 0, 0.0),
]


@pytest.mark.parametrize("name,dt,layout,Bsz,tile,lr", FUSED_BWD)
def test_bwd_fused(orc, name, dt, layout, Bsz, tile, lr):
    """One pass gives the input gradient and the value gradient of the
    separate products, and the SGD step of their definition."""
    if name == "ragged":
        w = synth.random_case(15, 300, 200, 9000, Bsz, dt, layout)
    elif name == "long":
        w = synth.random_case(18, 1500, 40, 30000, Bsz, dt, layout)
    elif name == "wide":
        w = synth.random_case(26, 8192, 2048, 2_200_000, Bsz, dt, layout)
    elif name == "wide_f32":
        w = synth.random_case(26, 8192, 4096, 2_200_000, Bsz, dt, layout)
    elif name == "skewed":
        lin = np.concatenate([np.arange(64) * 40 + 7, np.arange(3000) + 64 * 40])
        lin = np.unique(lin[lin < 80 * 40])
        w = synth.random_case(16, 80, 40, lin.size, Bsz, dt, layout, positions=lin)
    else:
        w = workload(name)
    wt, X, dY = w.weights[0], w.X[0], w.dY[0]
    nm = layout == "node"
    topo = topology(wt, Bsz, tile)
    vals = to_dev(wt.vals, dt)
    dX = torch.empty(Bsz * wt.K, dtype=torch_dtype(dt), device="cuda")
    dV = torch.empty(wt.nnz, dtype=torch_dtype(dt), device="cuda")
    snk.snack_spmm_bwd_fused(topo.plan, vals, to_dev(X.data, dt), to_dev(dY.data, dt),
                             B.NODE_MAJOR if nm else B.BATCH_MAJOR, Bsz, dX, dV, lr)
    v64 = wt.vals_f64()
    ref, S = orc.spmm_bwd_input(wt.M, wt.K, wt.row, wt.col, v64, Bsz, dY.f64(), nm)
    assert_within(from_dev(dX, dt), ref, S, dt, "fused dX")
    refv, Sv = orc.sddmm(wt.M, wt.K, wt.row, wt.col, Bsz, dY.f64(), X.f64(), nm)
    assert_within(from_dev(dV, dt), refv, Sv, dt, "fused dV")
    new = from_dev(vals, dt)
    if lr == 0.0:
        assert np.array_equal(new, v64)
    else:
        exp = v64 - lr * refv
        ulp = 2.0 ** (-8 if dt == "bf16" else -23)
        tol = 1e-2 if dt == "bf16" else 1e-5
        assert np.all(np.abs(new - exp) <= lr * tol * Sv + ulp * np.abs(exp) + 1e-30)


SMALL_ADAM = (512, 384, 20000)


@pytest.mark.parametrize("dt,layout,Bsz,use_vt,shape", [
    ("f32", "node", 8, True, SMALL_ADAM),
    ("f32", "batch", 5, False, SMALL_ADAM),
    ("bf16", "node", 32, True, SMALL_ADAM),
    ("bf16", "node", 8, True, (8192, 2048, 2_200_000)),  # 2.2 M values and moments
])
def test_bwd_fused_adam(orc, dt, layout, Bsz, use_vt, shape):
    """Three Adam steps through the fused backward against the oracle's step
    (Kingma & Ba, Algorithm 1).  fp32: the returned dV is the fp32 gradient
    sum itself, so the oracle steps from it and the moments and values must
    agree to fp32 rounding; bf16: the moments against the oracle's exact
    gradient within the products' tolerance carried through the step."""
    w = synth.random_case(25, *shape, Bsz, dt, layout)
    wt = w.weights[0]
    lay = B.NODE_MAJOR if layout == "node" else B.BATCH_MAJOR
    topo = topology(wt, Bsz)
    assert topo.plan.has_split_col == 0
    X, dY = to_dev(w.X[0].data, dt), to_dev(w.dY[0].data, dt)
    vals = to_dev(wt.vals, dt)
    vt = topo.gather_vals_t(vals) if use_vt else None
    m_t = torch.zeros(wt.nnz, device="cuda")
    v_t = torch.zeros(wt.nnz, device="cuda")
    _, perm, _ = orc.csc(wt.K, wt.row, wt.col)
    # the ABI takes the hyperparameters as fp32: the oracle steps with those values
    lr, b1, b2, eps = (float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8))
    m64, v64 = np.zeros(wt.nnz), np.zeros(wt.nnz)
    gref, Sg = orc.sddmm(wt.M, wt.K, wt.row, wt.col, Bsz, w.dY[0].f64(), w.X[0].f64(),
                         layout == "node")
    for t in (1, 2, 3):
        dX = torch.empty(Bsz * wt.K, dtype=torch_dtype(dt), device="cuda")
        dV = torch.empty(wt.nnz, dtype=torch_dtype(dt), device="cuda")
        prev = from_dev(vals, dt)
        snk.snack_spmm_bwd_fused_adam(topo.plan, vals, X, dY, lay, Bsz, dX, dV, m_t, v_t, lr, t,
                                      b1, b2, eps, vals_t=vt)
        got_v, got_m = from_dev(vals, dt), m_t.cpu().numpy().astype(np.float64)[np.argsort(perm)]
        got_s = v_t.cpu().numpy().astype(np.float64)[np.argsort(perm)]
        assert_within(from_dev(dV, dt), gref, Sg, dt, f"adam step {t} dV")
        if use_vt:
            assert np.array_equal(bits_of(vt, dt), bits_of(vals, dt)[perm])
        if dt == "f32":  # step the oracle from the GPU's own fp32 gradient
            w_ref, m64, v64 = orc.adam_step(prev, from_dev(dV, dt), m64, v64, lr, b1, b2, eps, t)
            np.testing.assert_allclose(got_m, m64, rtol=4e-6, atol=1e-12)
            np.testing.assert_allclose(got_s, v64, rtol=4e-6, atol=1e-15)
            assert np.all(np.abs(got_v - w_ref) <= 4 * 2.0 ** -24 * np.abs(w_ref) + lr * 1e-4)
        else:  # the moments against the exact gradient, errors carried through the step
            w_ref, m64, v64 = orc.adam_step(prev, gref, m64, v64, lr, b1, b2, eps, t)
            tol_g = 1e-2 * Sg
            assert np.all(np.abs(got_m - m64) <= tol_g + 1e-6 * np.abs(m64) + 1e-30)
            assert np.all(np.abs(got_s - v64) <= 2 * np.abs(gref) * tol_g + tol_g ** 2
                          + 1e-6 * v64 + 1e-30)
            assert np.all(np.abs(got_v - w_ref) <= 2.0 ** -7 * np.abs(w_ref) + 3 * lr)
            m64, v64 = got_m, got_s  # continue from the GPU's moments


def test_bwd_fused_adam_rejections():
    w = synth.random_case(26, 80, 40, 900, 4, "f32")
    wt = w.weights[0]
    X, dY = to_dev(w.X[0].data, "f32"), to_dev(w.dY[0].data, "f32")
    dX = torch.empty(4 * 40, device="cuda")
    m = torch.zeros(wt.nnz, device="cuda")
    vals = to_dev(wt.vals, "f32")
    split = topology(wt, 4, tile=8)  # columns of ~22 entries over 8-item tiles
    assert split.plan.has_split_col == 1
    for topo, kw, status in ((split, {}, -2),
                             (topology(wt, 4), {"step": 0}, -2),
                             (topology(wt, 4), {"lr": float("nan")}, -7)):
        args = dict(lr=1e-3, step=1)
        args.update(kw)
        before = vals.clone()
        with pytest.raises(snk.SnackError) as e:
            snk.snack_spmm_bwd_fused_adam(topo.plan, vals, X, dY, B.BATCH_MAJOR, 4, dX, None, m,
                                          m.clone(), args["lr"], args["step"])
        assert e.value.status == status
        assert torch.equal(vals, before)


def test_bwd_fused_rejects_wide_batch_and_bad_lr():
    w = synth.random_case(17, 64, 48, 500, 33, "f32")
    wt = w.weights[0]
    topo = topology(wt, 33)
    vals = to_dev(wt.vals, "f32")
    X, dY = to_dev(w.X[0].data, "f32"), to_dev(w.dY[0].data, "f32")
    dX = torch.empty(33 * 48, device="cuda")
    with pytest.raises(snk.SnackError) as e:
        snk.snack_spmm_bwd_fused(topo.plan, vals, X, dY, B.BATCH_MAJOR, 33, dX, None, 0.1)
    assert e.value.status == -2
    with pytest.raises(snk.SnackError) as e:
        snk.snack_spmm_bwd_fused(topo.plan, vals, X, dY, B.BATCH_MAJOR, 8, dX, None,
                                 float("nan"))
    assert e.value.status == -7


# --------------------------------------------------------------- aux
def test_gelu_matches_oracle(orc):
    z = torch.linspace(-8, 8, 100003, device="cuda")
    h = torch.empty_like(z)
    snk.snack_gelu_fwd(z, h)
    z64 = z.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(h.cpu().numpy(), orc.gelu(z64), rtol=2e-6, atol=1e-7)
    dh = torch.ones_like(z)
    dz = torch.empty_like(z)
    snk.snack_gelu_bwd(z, dh, dz)
    np.testing.assert_allclose(dz.cpu().numpy(), orc.gelu_bwd(z64, np.ones_like(z64)),
                               rtol=4e-6, atol=1e-6)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("Bsz,K", [(1, 1000), (1, 4096), (1, 4104), (5, 1000), (16, 4096),
                                   (32, 1024), (40, 997)])
def test_dense_baseline(orc, dt, masked, Bsz, K):
    """Dense and Dense+Mask reference kernels against a numpy product, on
    every batch-tile path (batch 1 with X held in registers up to K = 4096,
    the weight stream beyond it and for batches up to 8, the 16-row matrix
    core tiles from 16 on), aligned and ragged K."""
    w = synth.random_case(6, 300, K, 30000, Bsz, dt)
    wt = w.weights[0]
    rng = np.random.default_rng(1)
    Wd = (rng.standard_normal(300 * K) * 0.02).astype(np.float32)
    if dt == "bf16":
        Wd = synth.f32_to_bf16_bits(Wd)
    mask = np.zeros(300 * K, np.uint8)
    mask[wt.row.astype(np.int64) * K + wt.col] = 1
    Y = torch.empty(Bsz * 300, dtype=torch_dtype(dt), device="cuda")
    snk.snack_dense_fwd(to_dev(Wd, dt), to_dev(mask) if masked else None, 300, K,
                        to_dev(w.X[0].data, dt), Bsz, Y)
    Wf = (synth.bf16_bits_to_f32(Wd) if dt == "bf16" else Wd).astype(np.float64)
    Wf = Wf * (mask if masked else 1)
    Xb = w.X[0].f64().reshape(Bsz, K)
    Wm = Wf.reshape(300, K)
    assert_within(from_dev(Y, dt), Xb @ Wm.T, np.abs(Xb) @ np.abs(Wm).T, dt, "dense")


def test_sparse_linear_column_values_follow_updates(orc):
    """The layer's column-ordered values follow a restructure (written by it)
    and a torch optimiser step (the version counter moves: gathered again);
    the input gradient read from them matches the oracle each time."""
    w = synth.random_case(22, 256, 320, 8000, 8, "f32")
    wt = w.weights[0]
    layer = snk.SparseLinear(320, 256, to_dev(wt.row), to_dev(wt.col), to_dev(wt.vals), 8)
    x = to_dev(w.X[0].data).view(8, 320)
    g = to_dev(w.dY[0].data).view(8, 256)
    opt = torch.optim.SGD([layer.vals], lr=0.5)

    def check(what):
        xr = x.clone().requires_grad_(True)
        layer.zero_grad()
        layer(xr).backward(g)
        row, col = layer.topo.row.cpu().numpy(), layer.topo.col.cpu().numpy()
        v = layer.vals.detach().cpu().numpy().astype(np.float64)
        ref, S = orc.spmm_bwd_input(256, 320, row, col, v, 8, w.dY[0].f64())
        assert_within(from_dev(xr.grad, "f32"), ref, S, "f32", what)
        _, perm, _ = orc.csc(320, row, col)
        assert np.array_equal(bits_of(layer.vals_t(), "f32"), bits_of(layer.vals.data, "f32")[perm])

    check("dX, first step")
    opt.step()                      # torch changes the values: the copy is gathered again
    check("dX after an optimiser step")
    layer.prune_regrow(200000, 1)   # the restructure writes the copy itself
    check("dX after a restructure")
    opt.step()
    check("dX after a restructure and an optimiser step")


def test_sparse_linear_autograd(orc):
    w = workload("single")
    wt = w.weights[0]
    layer = snk.SparseLinear(256, 256, to_dev(wt.row), to_dev(wt.col), to_dev(wt.vals), 40)
    x = to_dev(w.X[0].data).view(4, 256).requires_grad_(True)
    y = layer(x)
    g = to_dev(w.dY[0].data).view(4, 256)
    y.backward(g)
    ref, S = orc.spmm_fwd(256, 256, wt.row, wt.col, wt.vals_f64(), 4, w.X[0].f64())
    assert_within(from_dev(y, "f32"), ref, S, "f32", "SparseLinear fwd")
    ref, S = orc.spmm_bwd_input(256, 256, wt.row, wt.col, wt.vals_f64(), 4, w.dY[0].f64())
    assert_within(from_dev(x.grad, "f32"), ref, S, "f32", "SparseLinear dX")
    ref, S = orc.sddmm(256, 256, wt.row, wt.col, 4, w.dY[0].f64(), w.X[0].f64())
    assert_within(from_dev(layer.vals.grad, "f32"), ref, S, "f32", "SparseLinear dV")
    # 256 columns: the two separate calls (as for a batch above the fused limit)
    assert not snk.layer.fused_backward_pays(256, wt.nnz, 4, 4)
    xw = torch.randn(40, 256, device="cuda", requires_grad=True)
    layer(xw).backward(torch.ones(40, 256, device="cuda"))
    ref, S = orc.spmm_bwd_input(256, 256, wt.row, wt.col, wt.vals_f64(), 40,
                                np.ones(40 * 256))
    assert_within(from_dev(xw.grad, "f32"), ref, S, "f32", "SparseLinear dX, batch 40")
    dropped, grown = layer.prune_regrow(100000, 1)
    ref = orc.prune_regrow(256, 256, wt.row, wt.col, wt.vals, "f32", 655, 0, 1)
    assert np.array_equal(grown.cpu().numpy(), ref["grown"])
    assert np.array_equal(layer.topo.row.cpu().numpy(), ref["row"])


def test_sparse_linear_autograd_fused_path(orc):
    """A layer wide enough for the fused backward (2,048 columns, batch 32):
    both gradients from one snack_spmm_bwd_fused call, against the oracle."""
    w = synth.random_case(33, 2048, 2048, 200000, 32, "f32")
    wt = w.weights[0]
    assert snk.layer.fused_backward_pays(2048, wt.nnz, 4, 32)
    layer = snk.SparseLinear(2048, 2048, to_dev(wt.row), to_dev(wt.col), to_dev(wt.vals), 32)
    x = to_dev(w.X[0].data).view(32, 2048).requires_grad_(True)
    layer(x).backward(to_dev(w.dY[0].data).view(32, 2048))
    ref, S = orc.spmm_bwd_input(2048, 2048, wt.row, wt.col, wt.vals_f64(), 32, w.dY[0].f64())
    assert_within(from_dev(x.grad, "f32"), ref, S, "f32", "SparseLinear fused dX")
    ref, S = orc.sddmm(2048, 2048, wt.row, wt.col, 32, w.dY[0].f64(), w.X[0].f64())
    assert_within(from_dev(layer.vals.grad, "f32"), ref, S, "f32", "SparseLinear fused dV")


# ------------------------------------------------------------ memory footprint
@pytest.mark.parametrize("dt,n_drop_ppm,flags", [("f32", 0, 0), ("bf16", 300000, 1)])
def test_memory_footprint_matches_device_allocations(dt, n_drop_ppm, flags):
    """The sparse layer's reported bytes are what its device tensors take:
    COO, value gradient, plan arena and restructuring workspace, allocated the
    way the layer allocates them.  The tensors' own sizes must add up to the
    report; the caching allocator's count (each allocation rounded up to 512
    bytes, and a large segment's tail under 1 MiB left unsplit) can only be
    larger."""
    N, sp, Bsz = 2048, 0.9, 8
    M = K = N
    w = synth.inference_layer(N=N, sparsity=sp, B=Bsz, dtype=dt).weights[0]
    d = snk.F32 if dt == "f32" else snk.BF16
    n_drop = snk.snack_drop_count(w.nnz, n_drop_ppm)
    f = snk.snack_memory_footprint(M, K, w.nnz, Bsz, d, n_drop, flags)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    row, col = to_dev(w.row), to_dev(w.col)
    vals = to_dev(w.vals, dt)
    dV = torch.empty_like(vals)
    topo = snk.Topology(row, col, M, K, Bsz, flags=flags)
    vt = topo.gather_vals_t(vals)
    ws = torch.empty(f["restructure_ws"], dtype=torch.uint8, device="cuda") if n_drop else None
    torch.cuda.synchronize()
    used = torch.cuda.memory_allocated() - before
    tensors = [row, col, vals, dV, vt, topo.arena] + ([ws] if n_drop else [])
    held = sum(t.untyped_storage().nbytes() for t in tensors)
    assert held == f["sparse_total"]
    r512 = lambda n: -(-n // 512) * 512  # noqa: E731
    assert used >= sum(r512(t.untyped_storage().nbytes()) for t in tensors)
    assert (f["coo"] + f["value_grad"] + f["col_values"]
            == 4 * w.nnz * 2 + vals.element_size() * w.nnz * 3)
    assert topo.arena.numel() == f["derived"] + f["plan_scratch"]
    if n_drop:  # the workspace suffices for the restructure it was sized for
        topo.restructure(vals, n_drop, 0, 1, ws=ws, vals_t=vt)
    del row, col, vals, dV, topo, ws, vt


# ------------------------------------- fused activation and multi-layer propagation
LACT = {0: 1.0, 1: 1.0, 2: 1.13}  # slope bound of each nonlinearity (GELU's is ~1.129)
UNIT = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8}


def propagation_reference(orc, w, Bsz, X64, layers, act, dt, nm):
    """The oracle's output after `layers` steps and an elementwise bound on the
    GPU's distance from it: each step adds its accumulation tolerance
    (tol * S_l), a few roundings of its stored output in dt (8 u |H_l|), and
    carries the previous bound through |W| and the nonlinearity's slope."""
    ref = orc.graph_propagate(w.M, w.K, w.row, w.col, w.vals_f64(), Bsz, X64, layers, act, nm)
    E = np.zeros(Bsz * w.K)
    absv = np.abs(w.vals_f64())
    for H, S in ref:
        prop, _ = orc.spmm_fwd(w.M, w.K, w.row, w.col, absv, Bsz, E, nm)
        E = LACT[act] * (prop + TOL_DT[dt] * S) + 8 * UNIT[dt] * np.abs(H)
    return ref[-1][0], E


TOL_DT = {"f32": 1e-5, "bf16": 1e-2}


def assert_bound(got, ref, E, what):
    err = np.abs(got - ref)
    bad = err > E
    assert np.isfinite(got).all(), what
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {got.size} out of bound; worst "
                           f"{float(np.max(err - E))}")


ACT_CASES = [  # (M, K, nnz, B, dtype, layout, tile)
    (257, 255, 3000, 8, "bf16", "batch", 64),
    (1, 64, 64, 4, "f32", "batch", 5),       # one dense row split over many tiles
    (300, 40, 30, 2, "f32", "batch", 7),     # mostly empty rows: act(0) = 0
    (511, 129, 9000, 32, "f32", "node", 256),
    (100, 333, 8000, 5, "bf16", "node", 0),
]


@pytest.mark.parametrize("M,K,nnz,Bsz,dt,layout,tile", ACT_CASES)
def test_spmm_fwd_fused_activation(orc, M, K, nnz, Bsz, dt, layout, tile):
    wl = synth.random_case(9, M, K, nnz, Bsz, dt, layout)
    w, X = wl.weights[0], wl.X[0]
    nm = layout == "node"
    lay = B.NODE_MAJOR if nm else B.BATCH_MAJOR
    topo = topology(w, Bsz, tile)
    vals, Xd = to_dev(w.vals, dt), to_dev(X.data, dt)
    plain = topo.fwd(vals, Xd, Bsz, lay)
    for act in (B.ACT_NONE, B.ACT_RELU, B.ACT_GELU):
        Y = torch.empty_like(plain)
        B.snack_spmm_fwd_act(topo.plan, vals, Xd, lay, Bsz, Y, act)
        if act == B.ACT_NONE:
            assert torch.equal(Y, plain)
        ref, E = propagation_reference(orc, w, Bsz, X.f64(), 1, act, dt, nm)
        assert_bound(from_dev(Y, dt), ref, E, f"act {act}")
        Y2 = torch.empty_like(plain)
        B.snack_spmm_fwd_act(topo.plan, vals, Xd, lay, Bsz, Y2, act)
        assert torch.equal(Y, Y2)  # bitwise reproducible


@pytest.mark.parametrize("dt,layout,Bsz,act", [("f32", "node", 16, 1), ("f32", "node", 16, 2),
                                               ("bf16", "batch", 5, 1), ("f32", "batch", 3, 2)])
def test_graph_propagate_small(orc, dt, layout, Bsz, act):
    nm = layout == "node"
    lay = B.NODE_MAJOR if nm else B.BATCH_MAJOR
    if dt == "f32" and nm:
        wl = synth.graph_layer(seed=4, n=3000, nnz=40000, B=Bsz)
    else:
        wl = synth.random_case(4, 700, 700, 20000, Bsz, dt, layout)
    w, X = wl.weights[0], wl.X[0]
    topo = topology(w, Bsz, 0)
    vals, Xd = to_dev(w.vals, dt), to_dev(X.data, dt)
    for layers in (1, 2, 3):
        Y = torch.empty_like(Xd)
        tmp = torch.empty_like(Xd)
        B.snack_graph_propagate(topo.plan, vals, Xd, lay, Bsz, layers, act, Y, tmp)
        ref, E = propagation_reference(orc, w, Bsz, X.f64(), layers, act, dt, nm)
        assert_bound(from_dev(Y, dt), ref, E, f"layers {layers}")
        if layers == 1:
            Z = torch.empty_like(Xd)
            B.snack_spmm_fwd_act(topo.plan, vals, Xd, lay, Bsz, Z, act)
            assert torch.equal(Y, Z)


def test_graph_propagate_power_law_graph_full_size(orc):
    """200,000 nodes, 2,400,000 power-law edges with random-walk weights, 128
    fp32 node-major features, three ReLU propagation steps, every output."""
    wl = workload("graph")
    w, X = wl.weights[0], wl.X[0]
    topo = topology(w, 128, 0)
    vals, Xd = to_dev(w.vals, "f32"), to_dev(X.data, "f32")
    Y, tmp = torch.empty_like(Xd), torch.empty_like(Xd)
    B.snack_graph_propagate(topo.plan, vals, Xd, B.NODE_MAJOR, 128, 3, B.ACT_RELU, Y, tmp)
    ref, E = propagation_reference(orc, w, 128, X.f64(), 3, B.ACT_RELU, "f32", True)
    assert_bound(from_dev(Y, "f32"), ref, E, "graph 3 layers")


# ------------------------------------ fixed-pattern kernels and 1x1 convolutions
FIXED_CASES = [  # (M, K, sparsity, B, images, dtype)
    (48, 40, 0.8, 100, 1, "f32"),       # ragged batch (not a multiple of 64)
    (300, 7, 0.5, 64, 3, "f32"),        # several images, narrow input
    (1, 256, 0.9, 33, 2, "bf16"),       # one output row
    (256, 256, 0.9, 200, 2, "bf16"),
    (200, 1, 0.0, 70, 1, "f32"),        # dense single column
    (64, 64, 1.0, 65, 1, "f32"),        # no entries: Y = 0
    (96, 1000, 0.95, 40, 2, "bf16"),    # four staged tiles, two bands
    (768, 3072, 0.99, 64, 1, "f32"),    # GPT-2 W2 shape at 99%: twelve tiles
    (3072, 768, 0.99, 100, 1, "bf16"),  # GPT-2 W1 shape at 99%: many bands
]


@pytest.mark.parametrize("M,K,sp,Bsz,images,dt", FIXED_CASES)
def test_fixed_pattern_kernel(orc, M, K, sp, Bsz, images, dt):
    nnz = synth.nnz_for(M, K, sp)
    wl = synth.random_case(13, M, K, nnz, Bsz * images, dt, "node")
    w = wl.weights[0]
    f = snk.snack_fixed_build(w.row, w.col, w.vals, M, K,
                              dtype=snk.F32 if dt == "f32" else snk.BF16)
    rng = np.random.default_rng(5)
    X32 = rng.standard_normal(images * K * Bsz).astype(np.float32)
    Xh = synth.f32_to_bf16_bits(X32) if dt == "bf16" else X32
    Xd = to_dev(Xh, dt)
    Y = torch.full((images * M * Bsz,), float("nan"), dtype=Xd.dtype, device="cuda")
    snk.snack_fixed_fwd(f, Xd, Bsz, images, Y)
    got = from_dev(Y, dt).reshape(images, M * Bsz)
    X64 = (synth.bf16_bits_to_f32(Xh) if dt == "bf16" else X32).astype(np.float64)
    X64 = X64.reshape(images, K * Bsz)
    for i in range(images):
        ref, S = orc.spmm_fwd(M, K, w.row, w.col, w.vals_f64(), Bsz, X64[i], True)
        assert_within(got[i], ref, S, dt, f"image {i}")
    Y2 = torch.empty_like(Y)
    snk.snack_fixed_fwd(f, Xd, Bsz, images, Y2)
    assert torch.equal(Y, Y2)
    f.free()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_conv1x1_layouts_and_fixed_kernel(orc, dt):
    """A 1x1 convolution (C_out = 96, C_in = 128, 90% sparse) over 2 images of
    7 x 9 pixels: NHWC as one batch-major product, NCHW as one node-major
    product per image and through the generated kernel, all against the
    oracle on the same pixels."""
    M, K, N, HW = 96, 128, 2, 63
    wl = synth.random_case(17, M, K, synth.nnz_for(M, K, 0.9), N * HW, dt, "batch")
    w = wl.weights[0]
    pix = wl.X[0]  # N*HW pixels x K channels (batch-major = NHWC)
    X64 = pix.f64().reshape(N, HW, K)
    topo = topology(w, N * HW, 0)
    vals = to_dev(w.vals, dt)
    Xn = to_dev(pix.data, dt)
    Yn = torch.empty(N * HW * M, dtype=Xn.dtype, device="cuda")
    snk.snack_conv1x1(topo.plan, vals, Xn, N, HW, snk.CONV_NHWC, Yn)
    ref, S = orc.spmm_fwd(M, K, w.row, w.col, w.vals_f64(), N * HW, X64.reshape(-1), False)
    assert_within(from_dev(Yn, dt), ref, S, dt, "NHWC")
    # NCHW: the same pixels, channel-major per image
    raw = pix.data.reshape(N, HW, K).transpose(0, 2, 1).copy().reshape(-1)
    Xc = to_dev(raw, dt)
    Yc = torch.empty_like(Yn)
    snk.snack_conv1x1(topo.plan, vals, Xc, N, HW, snk.CONV_NCHW, Yc)
    refc = ref.reshape(N, HW, M).transpose(0, 2, 1).reshape(-1)
    Sc = S.reshape(N, HW, M).transpose(0, 2, 1).reshape(-1)
    assert_within(from_dev(Yc, dt), refc, Sc, dt, "NCHW")
    f = snk.snack_fixed_build(w.row, w.col, w.vals, M, K,
                              dtype=snk.F32 if dt == "f32" else snk.BF16)
    Yf = torch.empty_like(Yn)
    snk.snack_fixed_fwd(f, Xc, HW, N, Yf)
    assert_within(from_dev(Yf, dt), refc, Sc, dt, "NCHW fixed kernel")


# ---------------------------------------------------- wave-per-segment path
# Views with no split segment run one wave per segment (wave.hip); a tile of
# 2048 items keeps rows of up to 2047 entries whole, so these cases exercise
# segments spanning several 256-entry load batches, partial gather rounds and
# the batch passes of wide batches.
WAVE = [  # (M, K, row degrees lo..hi, Bsz, dt, layout)
    (40, 1500, (0, 1200), 1, "f32", "node"),
    (40, 1500, (0, 1200), 3, "bf16", "batch"),
    (40, 1500, (0, 1200), 8, "bf16", "node"),
    (40, 1500, (0, 1200), 16, "f32", "batch"),
    (40, 1500, (0, 1200), 32, "bf16", "node"),
    (40, 1500, (0, 1200), 32, "f32", "node"),
    (40, 1500, (0, 1200), 64, "bf16", "node"),
    (40, 1500, (0, 1200), 64, "f32", "batch"),
    (40, 1500, (0, 1200), 100, "f32", "node"),
    (33, 700, (1, 300), 12, "bf16", "batch"),
    (33, 700, (1, 300), 6, "f32", "node"),
]


@pytest.mark.parametrize("M,K,deg,Bsz,dt,layout", WAVE)
def test_wave_products_long_segments_and_batches(orc, M, K, deg, Bsz, dt, layout):
    rng = np.random.default_rng(M * 1000 + Bsz)
    d = rng.integers(deg[0], deg[1] + 1, size=M)
    d[:3] = (0, deg[1], 257)  # an empty row, the longest row, one past a load batch
    lin = np.concatenate([r * K + np.sort(rng.choice(K, n, replace=False))
                          for r, n in enumerate(d)])
    w = synth.random_case(11, M, K, lin.size, Bsz, dt, layout, positions=lin)
    topo = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, layout, Bsz, tile=2048,
                        repeat_check=True)
    assert topo.plan.has_split_row == 0 and topo.plan.has_split_col == 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wave_products_match_merge_path(orc, dt):
    """The same layer through both kernels (default tiles: no split, wave
    path; 16-item tiles: splits, merge path) agrees with the oracle."""
    w = synth.random_case(13, 200, 300, 9000, 8, dt, "node")
    a = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, "node", 8, tile=0)
    b = run_products(orc, w.weights[0], w.X[0], w.dY[0], dt, "node", 8, tile=16)
    assert a.plan.has_split_row == 0 and b.plan.has_split_row == 1


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wave_inf_at_segment_end_stays_inf(dt):
    """Lanes past a segment's end gather at its last entry's index; that row
    holding Inf must not turn the row's result into NaN (0 * Inf)."""
    M, K, Bsz = 4, 64, 8
    lin = np.array([0 * K + 5, 0 * K + 9, 1 * K + 9, 2 * K + 1, 2 * K + 2, 2 * K + 63],
                   dtype=np.int64)
    w = synth.random_case(17, M, K, lin.size, Bsz, dt, "node", positions=lin).weights[0]
    topo = topology(w, Bsz)
    assert topo.plan.has_split_row == 0
    vals = torch.ones(lin.size, dtype=torch_dtype(dt), device="cuda")
    X = torch.ones(K * Bsz, dtype=torch_dtype(dt), device="cuda")
    X.view(K, Bsz)[9] = float("inf")  # column 9 ends rows 0 and 1
    Y = topo.fwd(vals, X, Bsz, B.NODE_MAJOR).float().view(M, Bsz).cpu().numpy()
    assert np.isposinf(Y[0]).all() and np.isposinf(Y[1]).all()
    assert (Y[2] == 3.0).all() and (Y[3] == 0.0).all()
    dY = torch.ones(M * Bsz, dtype=torch_dtype(dt), device="cuda")
    dY.view(M, Bsz)[2] = float("inf")  # row 2 ends column 63 and holds columns 1, 2
    dX = topo.bwd_input(vals, dY, Bsz, B.NODE_MAJOR).float().view(K, Bsz).cpu().numpy()
    for c in (1, 2, 63):
        assert np.isposinf(dX[c]).all()
    assert (dX[5] == 1.0).all() and (dX[9] == 2.0).all() and (dX[0] == 0.0).all()
