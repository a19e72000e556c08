"""Shared helpers of the GPU parity tests: moving seeded inputs to the GPU,
reading results back, and the tolerance check against the fp64 oracle."""
import numpy as np

import synth

TOL = {"f32": 1e-5, "bf16": 1e-2}


def torch_dtype(dt):
    import torch
    return torch.float32 if dt == "f32" else torch.bfloat16


def to_dev(arr, dt=None):
    """numpy -> cuda tensor; bf16 inputs arrive as uint16 bit patterns."""
    import torch
    a = np.ascontiguousarray(arr)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.copy()).cuda()


def from_dev(t, dt):
    """cuda tensor -> float64 numpy (exact widening)."""
    import torch
    if dt == "bf16":
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def assert_within(got, ref, S, dt, what=""):
    """|got - ref| <= tol * S element by element; S == 0 demands exactly 0."""
    got, ref, S = (np.asarray(x, dtype=np.float64).ravel() for x in (got, ref, S))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL[dt] * S
    bad = err > bound
    if bad.any():
        i = int(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} outputs out of tolerance; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r} S {S[i]!r}")


def topology(w, max_batch, tile=0):
    import unstructured_sparse_nn_amd as snk
    return snk.Topology(to_dev(w.row), to_dev(w.col), w.M, w.K, max_batch, tile)
