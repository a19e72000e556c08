"""Host-side tests of the C-ABI library (no GPU needed).

The library must load, export every entry point include/snack.h declares,
agree with the binding on the plan struct, and reject bad arguments on the
host before any HIP call is made.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "snack.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"SNACK_API\s+[\w\s\*]*?\b(snack_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def snk():
    import unstructured_sparse_nn_amd as m
    return m


def test_library_exports_every_declared_symbol(snk):
    from unstructured_sparse_nn_amd import binding
    names = declared_symbols()
    assert len(names) >= 15
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_plan_struct_matches(snk):
    assert ctypes.sizeof(snk.SnackPlan) == snk.snack_plan_sizeof()
    assert snk.snack_version() >= 100


def test_plan_init_sizes(snk):
    p = snk.snack_plan_init(4096, 4096, 838861, 32)
    assert p.tile_row == 512 and p.P_row == -(-(4096 + 838861) // 512)
    assert p.P_row <= 2048 and p.arena_bytes > 0
    p = snk.snack_plan_init(200000, 200000, 2400000, 128)
    assert p.tile_row == 2048
    # batches wider than 32: tiles of at least twice the mean segment length
    # (GPT-2 W1 3072 x 768 at 90%: rows of ~77, columns of ~307 entries)
    p = snk.snack_plan_init(3072, 768, 235930, 1024)
    assert (p.tile_row, p.tile_col) == (256, 1024)
    p = snk.snack_plan_init(3072, 768, 235930, 32)
    assert (p.tile_row, p.tile_col) == (128, 128)
    p = snk.snack_plan_init(7, 5, 0, 1, tile_items=3)
    assert p.tile_row == 3 and p.P_row == 3 and p.P_col == 2
    offs = list(p.off)[:10]
    assert offs == sorted(offs)
    # node-major-only plans skip the activation transpose scratch
    a = snk.snack_plan_init(4096, 4096, 838861, 32)
    b = snk.snack_plan_init(4096, 4096, 838861, 32, flags=1)
    assert a.arena_bytes - b.arena_bytes >= 4 * 32 * 8192


@pytest.mark.parametrize("args,status", [
    ((0, 4, 1, 1, 0), -2), ((4, 0, 1, 1, 0), -2), ((4, 4, -1, 1, 0), -2),
    ((4, 4, 17, 1, 0), -2), ((4, 4, 1, 0, 0), -2), ((4, 4, 1, 1, 4096), -2),
    ((2**31 - 1, 1, 1, 1, 0), -10), ((4, 4, 1, 1, 0, 2), -4),
])
def test_plan_init_rejects(snk, args, status):
    with pytest.raises(snk.SnackError) as e:
        snk.snack_plan_init(*args)
    assert e.value.status == status


def test_products_reject_unprepared_plan(snk):
    from unstructured_sparse_nn_amd import binding as b
    p = snk.snack_plan_init(8, 8, 4, 2)
    for fn in (b.snack_spmm_fwd, b.snack_spmm_bwd_input):
        with pytest.raises(snk.SnackError) as e:
            fn(p, 0x1000, 0x2000, 0, 1, 0x3000, stream=0, dtype=b.F32)
        assert e.value.status == -12
    with pytest.raises(snk.SnackError) as e:
        b.snack_sddmm_grad_vals(p, 0x1000, 0x2000, 0, 1, 0x3000, stream=0, dtype=b.F32)
    assert e.value.status == -12
    assert b.raw_status("snack_spmm_fwd", None, 1, 0, 1, 0, 1, 1, None) == -1


def test_column_order_value_calls_reject_bad_arguments(snk):
    from unstructured_sparse_nn_amd import binding as b
    p = snk.snack_plan_init(8, 8, 4, 2)
    with pytest.raises(snk.SnackError) as e:
        b.snack_gather_vals_t(p, 0x1000, 0x2000, stream=0, dtype=b.F32)
    assert e.value.status == -12
    with pytest.raises(snk.SnackError) as e:
        b.snack_spmm_bwd_input_t(p, 0x1000, 0x2000, 0, 1, 0x3000, stream=0, dtype=b.F32)
    assert e.value.status == -12
    assert b.raw_status("snack_gather_vals_t", None, 1, 0, 1, None) == -1
    assert b.raw_status("snack_spmm_bwd_input_t", None, 1, 0, 1, 0, 1, 1, None) == -1


def test_restructure_flags_and_workspaces(snk):
    from unstructured_sparse_nn_amd import binding as b
    auto = b.snack_prune_regrow_workspace(256, 256, 6554, 655)
    assert b.snack_prune_regrow_workspace(256, 256, 6554, 655, flags=b.PRUNE_SORT_PLAN) > 0
    assert auto == b.snack_prune_regrow_workspace(256, 256, 6554, 655, flags=0)
    sz = ctypes.c_size_t(0)
    assert b.raw_status("snack_prune_regrow_workspace_ex", 256, 256, 6554, 655, 2,
                        ctypes.byref(sz)) == -4
    with pytest.raises(snk.SnackError) as e:
        b.snack_prune_regrow(0x10, 0x20, 0x30, 4, 4, 3, 1, 0, 0, None, None, 0x40, stream=0,
                             ws_bytes=1 << 20, dtype=b.F32, flags=6)
    assert e.value.status == -4
    p = snk.snack_plan_init(8, 8, 4, 2)
    with pytest.raises(snk.SnackError) as e:  # never prepared: no arena
        b.snack_prune_regrow_prepared(p, 0x10, 0x20, 0x30, 1, 0, 0, None, None, 0x40, stream=0,
                                      ws_bytes=1 << 20, dtype=b.F32)
    assert e.value.status == -12


def test_library_allocates_nothing_and_reads_no_environment():
    """The boundary's promise, checked in the sources: no device or pinned
    allocation outside the fixed-pattern generator's code object, no
    environment switches, no thread-local or function-static state."""
    csrc = os.path.join(ROOT, "unstructured_sparse_nn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        text = re.sub(r"//[^\n]*", "", open(os.path.join(csrc, name)).read())
        for bad in ("getenv", "hipMalloc", "hipHostMalloc", "hipFree", "thread_local"):
            assert bad not in text, (name, bad)
        assert not re.search(r"\bstatic\s+(const\s+)?(bool|int|int32_t|int64_t|size_t|char)\b"
                             r"[^(;]*=", text), name


def test_prepare_rejects_small_arena_before_any_launch(snk):
    from unstructured_sparse_nn_amd import binding as b
    p = snk.snack_plan_init(8, 8, 4, 2)
    with pytest.raises(snk.SnackError) as e:
        b.snack_coo_prepare(p, 0x1000, 0x2000, 0x3000, stream=0, arena_bytes=16)
    assert e.value.status == -9
    with pytest.raises(snk.SnackError) as e:
        b.snack_coo_prepare(p, None, 0x2000, 0x3000, stream=0, arena_bytes=p.arena_bytes)
    assert e.value.status == -1


def test_drop_count_and_prune_argument_checks(snk, orc):
    from unstructured_sparse_nn_amd import binding as b
    for nnz, ppm in [(6554, 100000), (235930, 300000), (23593, 300000), (5, 500000), (0, 7),
                     (838861, 300000), (4508877, 100000)]:
        assert snk.snack_drop_count(nnz, ppm) == orc.drop_count(nnz, ppm)
    assert snk.snack_drop_count(-1, 5) == -1
    # n_drop larger than nnz, or than the free positions: rejected on the host
    with pytest.raises(snk.SnackError) as e:
        b.snack_prune_regrow(0x10, 0x20, 0x30, 4, 4, 3, 4, 0, 0, None, None, 0x40, stream=0,
                             ws_bytes=1 << 20, dtype=b.F32)
    assert e.value.status == -8
    with pytest.raises(snk.SnackError) as e:
        b.snack_prune_regrow(0x10, 0x20, 0x30, 4, 4, 15, 2, 0, 0, None, None, 0x40, stream=0,
                             ws_bytes=1 << 20, dtype=b.F32)
    assert e.value.status == -8
    # n_drop == 0 is a no-op that touches nothing
    b.snack_prune_regrow(None, None, None, 4, 4, 3, 0, 0, 0, None, None, None, stream=0,
                         ws_bytes=0, dtype=b.F32)
    with pytest.raises(snk.SnackError) as e:
        b.snack_prune_regrow(0x10, 0x20, 0x30, 4, 4, 3, 1, 0, 0, None, None, 0x40, stream=0,
                             ws_bytes=0, dtype=7)
    assert e.value.status == -3
    assert snk.snack_prune_regrow_workspace(256, 256, 6554, 655) > 0


def test_status_strings(snk):
    from unstructured_sparse_nn_amd import binding as b
    for code in b.STATUS:
        assert snk.status_str(code) and snk.status_str(code) != "unknown status"


# ---------------------------------------------------------------- footprint
FOOTPRINT_CASES = [  # (M, K, nnz, max_batch, dtype, n_drop, flags)
    (4096, 4096, 1677722, 1, "f32", 0, 0),        # 90%: the abstract's single-layer point
    (4096, 4096, 838861, 32, "bf16", 251658, 1),  # 95%, restructuring 30%
    (3072, 768, 235930, 1024, "f32", 70779, 0),   # GPT-2 MLP projection at 90%
    (256, 256, 6554, 4, "f32", 655, 0),
    (1, 1, 0, 1, "bf16", 0, 0),
]


@pytest.mark.parametrize("M,K,nnz,B,dt,n_drop,flags", FOOTPRINT_CASES)
def test_memory_footprint_matches_definitions_and_allocations(snk, M, K, nnz, B, dt, n_drop,
                                                              flags):
    import oracle
    d = snk.F32 if dt == "f32" else snk.BF16
    s = 4 if dt == "f32" else 2
    f = snk.snack_memory_footprint(M, K, nnz, B, d, n_drop, flags)
    ref = oracle.memory_by_definition(M, K, nnz, s, B)
    for k, v in ref.items():
        assert f[k] == v, k
    # the implementation's parts are exactly what the library asks callers for
    plan = snk.snack_plan_init(M, K, nnz, B, 0, flags)
    assert f["derived"] + f["plan_scratch"] == plan.arena_bytes
    assert f["derived"] == plan.off[10]  # derived arrays precede the scratch
    ws = snk.snack_prune_regrow_workspace(M, K, nnz, n_drop) if n_drop else 0
    assert f["restructure_ws"] == ws
    assert f["col_values"] == f["value_grad"]  # one value per connection, column order
    assert f["sparse_total"] == (f["coo"] + f["value_grad"] + f["col_values"] + f["derived"]
                                 + f["plan_scratch"] + f["restructure_ws"])
    assert f["dense_total"] == f["dense_weight"] + f["dense_grad"]
    assert f["masked_total"] == f["dense_total"] + f["mask"]


def test_memory_footprint_rejects_bad_arguments(snk):
    from unstructured_sparse_nn_amd import binding as B
    st = B.raw_status
    out = B.SnackFootprint()
    ref = ctypes.byref(out)
    assert st("snack_memory_footprint", 64, 64, 10, 1, 0, 0, 0, None) == -1
    assert st("snack_memory_footprint", 64, 64, 10, 1, 7, 0, 0, ref) == -3
    assert st("snack_memory_footprint", 0, 64, 10, 1, 0, 0, 0, ref) == -2
    assert st("snack_memory_footprint", 64, 64, 10, 0, 0, 0, 0, ref) == -2
    assert st("snack_memory_footprint", 64, 64, 10, 1, 0, -1, 0, ref) == -2
    assert st("snack_memory_footprint", 64, 64, 10, 1, 0, 11, 0, ref) == -8
    assert st("snack_memory_footprint", 4, 4, 10, 1, 0, 7, 0, ref) == -8
    assert st("snack_memory_footprint", 64, 64, 10, 1, 0, 0, 8, ref) == -4


def test_fused_activation_and_propagation_argument_checks(snk):
    from unstructured_sparse_nn_amd import binding as b
    p = snk.snack_plan_init(8, 8, 4, 2)
    q = snk.snack_plan_init(8, 6, 4, 2)
    cases = [  # (call, status) -- all rejected on the host, nothing launched
        (lambda: b.snack_spmm_fwd_act(p, 0x1000, 0x2000, 0, 1, 0x3000, 3, stream=0, dtype=0), -2),
        (lambda: b.snack_spmm_fwd_act(p, 0x1000, 0x2000, 0, 1, 0x3000, -1, stream=0, dtype=0), -2),
        (lambda: b.snack_spmm_fwd_act(p, 0x1000, 0x2000, 0, 1, 0x3000, 1, stream=0, dtype=0), -12),
        (lambda: b.snack_graph_propagate(p, 0x1000, 0x2000, 0, 1, 0, 1, 0x3000, 0x4000,
                                         stream=0, dtype=0), -2),   # no layers
        (lambda: b.snack_graph_propagate(q, 0x1000, 0x2000, 0, 1, 2, 1, 0x3000, 0x4000,
                                         stream=0, dtype=0), -2),   # not square
        (lambda: b.snack_graph_propagate(p, 0x1000, 0x2000, 0, 1, 2, 1, 0x3000, None,
                                         stream=0, dtype=0), -1),   # tmp missing
        (lambda: b.snack_graph_propagate(p, 0x1000, 0x2000, 0, 1, 2, 1, 0x2000, 0x4000,
                                         stream=0, dtype=0), -2),   # Y aliases X
        (lambda: b.snack_graph_propagate(p, 0x1000, 0x2000, 0, 1, 2, 5, 0x3000, 0x4000,
                                         stream=0, dtype=0), -2),   # unknown act
        (lambda: b.snack_graph_propagate(p, 0x1000, 0x2000, 0, 1, 2, 1, 0x3000, 0x4000,
                                         stream=0, dtype=0), -12),  # unprepared plan
    ]
    for call, status in cases:
        with pytest.raises(snk.SnackError) as e:
            call()
        assert e.value.status == status
    assert b.raw_status("snack_graph_propagate", None, 1, 0, 0, 0, 1, 1, 1, 1, 1, None) == -1


# ------------------------------------------------ fixed-pattern kernels (hipRTC)
def _fixed_case(M, K, sp, dt="f32", seed=3):
    import synth
    return synth.random_case(seed, M, K, synth.nnz_for(M, K, sp), 4, dt, "node").weights[0]


def test_fixed_pattern_kernel_compiles_for_gfx950_without_spills(snk):
    """The generated kernel compiles for gfx950 on the host, also with K over
    one staged tile of 256 inputs.  Its code object has one FMA per entry
    (the value an operand), no scratch and no packed fp32 instructions, and
    reads the staged inputs from LDS (ds_ instructions, no flat loads of
    them)."""
    import shutil
    import subprocess
    import tempfile
    for M, K, sp, dt in ((48, 40, 0.8, "f32"), (96, 64, 0.6, "bf16"), (40, 700, 0.9, "bf16")):
        w = _fixed_case(M, K, sp, dt)
        f = snk.snack_fixed_build(w.row, w.col, w.vals, M, K,
                                  dtype=snk.F32 if dt == "f32" else snk.BF16,
                                  flags=snk.FIXED_COMPILE_ONLY)
        info = f.info()
        assert 1 <= info["waves"] <= 16 and info["code_bytes"] > 0
        # bands: waves of at most 32 rows each, at most 16 waves per band
        assert info["bands"] >= -(-M // (32 * 16))
        code = f.code()
        assert len(code) == info["code_bytes"]
        objdump = "/opt/rocm/llvm/bin/llvm-objdump"
        readelf = "/opt/rocm/llvm/bin/llvm-readelf"
        if not (shutil.which(objdump) and shutil.which(readelf)):
            continue
        with tempfile.NamedTemporaryFile(suffix=".co") as t:
            t.write(code)
            t.flush()
            asm = subprocess.run([objdump, "-d", "--mcpu=gfx950", t.name], capture_output=True,
                                 text=True).stdout
            notes = subprocess.run([readelf, "--notes", t.name], capture_output=True,
                                   text=True).stdout
        assert "v_pk_fma_f32" not in asm and "v_pk_mul_f32" not in asm
        assert "scratch_" not in asm
        fmas = sum(asm.count(op) for op in ("v_fmamk_f32", "v_fmac_f32", "v_fma_f32",
                                            "v_mul_f32"))
        assert fmas >= w.nnz
        assert ".private_segment_fixed_size: 0" in notes.replace("  ", " ").replace("  ", " ")
        assert asm.count("ds_read") + asm.count("ds_load") > 0


def test_fixed_pattern_build_rejects_bad_arguments(snk):
    import numpy as np
    from unstructured_sparse_nn_amd import binding as b
    r = np.array([0, 0, 1], np.int32)
    c = np.array([1, 3, 0], np.int32)
    v = np.ones(3, np.float32)
    CO = snk.FIXED_COMPILE_ONLY
    cases = [
        (lambda: snk.snack_fixed_build(r, c, v, 0, 4, flags=CO), -2),
        (lambda: snk.snack_fixed_build(r, c, v, 2, 0, flags=CO), -2),
        (lambda: snk.snack_fixed_build(r, np.array([3, 1, 0], np.int32), v, 2, 4, flags=CO), -6),
        (lambda: snk.snack_fixed_build(r, np.array([1, 4, 0], np.int32), v, 2, 4, flags=CO), -5),
        (lambda: snk.snack_fixed_build(r, c, v, 2, 4, dtype=5, flags=CO), -3),
        (lambda: snk.snack_fixed_build(r, c, v, 2, 4, flags=8), -4),
    ]
    for call, status in cases:
        with pytest.raises(snk.SnackError) as e:
            call()
        assert e.value.status == status
    import ctypes
    out = ctypes.c_void_p(0)
    # more than 2^23 entries: refused before the arrays are read
    assert b.raw_status("snack_fixed_build", r.ctypes.data, c.ctypes.data, v.ctypes.data, 0,
                        4096, 4096, (1 << 23) + 1, CO, ctypes.byref(out)) == -2
    assert out.value is None
    f = snk.snack_fixed_build(r, c, v, 2, 4, flags=CO)
    with pytest.raises(snk.SnackError) as e:  # compile-only handles cannot run
        snk.snack_fixed_fwd(f, 0x1000, 8, 1, 0x2000, stream=0)
    assert e.value.status == -12
    assert b.raw_status("snack_fixed_build", None, None, None, 0, 2, 4, 0, 0, None) == -1
    p = snk.snack_plan_init(8, 8, 4, 2)
    with pytest.raises(snk.SnackError) as e:
        snk.snack_conv1x1(p, 0x1000, 0x2000, 1, 2, 7, 0x3000, stream=0, dtype=0)
    assert e.value.status == -4
