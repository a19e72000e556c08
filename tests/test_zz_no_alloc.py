"""snack_prune_regrow_static (the restructure with the library's per-GPU
workspace array, for callers that cannot allocate) against
snack_prune_regrow with a caller's workspace: bit-exact COO, values and
dropped/grown lists, on two calls in a row, the second on a smaller layer."""
import numpy as np
import pytest

import synth
from gpuhelp import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only collection
    pytest.skip("no GPU", allow_module_level=True)

import unstructured_sparse_nn_amd as snk  # noqa: E402


def restructure(w, dt, n_drop, seed, step, static):
    row, col, v = to_dev(w.row), to_dev(w.col), to_dev(w.vals, dt)
    dl = torch.empty(max(n_drop, 1), dtype=torch.int64, device="cuda")
    gl = torch.empty(max(n_drop, 1), dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    if static:
        before = torch.cuda.memory_allocated()
        snk.snack_prune_regrow_static(row, col, v, w.M, w.K, w.nnz, n_drop, seed, step, dl, gl)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before  # nothing allocated through torch
    else:
        ws = torch.empty(snk.snack_prune_regrow_workspace(w.M, w.K, w.nnz, n_drop),
                         dtype=torch.uint8, device="cuda")
        snk.snack_prune_regrow(row, col, v, w.M, w.K, w.nnz, n_drop, seed, step, dl, gl, ws)
    torch.cuda.synchronize()
    vb = v.view(torch.int16) if dt == "bf16" else v.view(torch.int32)
    return [t.cpu().numpy() for t in (row, col, vb, dl[:n_drop], gl[:n_drop])]


def test_static_workspace_matches_caller_workspace(orc):
    big = synth.inference_layer(N=4096, sparsity=0.95, B=1).weights[0]   # bf16, 15.5 MiB ws
    small = synth.single_layer().weights[0]                               # f32, 0.3 MiB ws
    for w, dt, ppm, seed, step in ((big, "bf16", 300000, 3, 2), (small, "f32", 100000, 0, 1)):
        n_drop = snk.snack_drop_count(w.nnz, ppm)
        assert snk.snack_prune_regrow_workspace(w.M, w.K, w.nnz, n_drop) <= snk.binding.STATIC_WS_MAX
        got = restructure(w, dt, n_drop, seed, step, static=True)
        ref = restructure(w, dt, n_drop, seed, step, static=False)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
    # the smaller layer against the oracle as well
    o = orc.prune_regrow(small.M, small.K, small.row, small.col, small.vals, "f32", 655, 0, 1)
    assert np.array_equal(got[0], o["row"]) and np.array_equal(got[4], o["grown"])


def test_static_workspace_rejects_layers_over_its_limit():
    # an 11008 x 4096 layer at 90% needs ~50 MiB of workspace: refused on the
    # host before any pointer is used
    with pytest.raises(snk.SnackError) as e:
        snk.snack_prune_regrow_static(None, None, None, 11008, 4096, 4508877, 450888, 0, 1,
                                      None, None, dtype=snk.BF16)
    assert e.value.status == -9
