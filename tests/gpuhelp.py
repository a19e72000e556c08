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


# bf16 outputs: fp32 accumulation plus one round-to-nearest-even to bf16 (8
# significant bits, unit roundoff 2^-8) must land within 2^-8 |ref| of the
# exact result, plus the accumulation error, which stays below the fp32
# tolerance 1e-5 S (per-lane runs of at most a few hundred terms, summed by a
# fixed tree).  This is about 5x tighter than 1e-2 S on typical outputs, so it
# catches an accumulation carried out in bf16.
BF16_ROUND = 2.0 ** -8
BF16_ACC = 1e-5


def _check(err, bound, got, ref, S, what, kind):
    bad = err > bound
    if bad.any():
        i = int(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} outputs out of {kind}; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r} S {S[i]!r}")


def assert_within(got, ref, S, dt, what=""):
    """|got - ref| <= tol * S element by element; S == 0 demands exactly 0.
    bf16 outputs must also meet |got - ref| <= 2^-8 |ref| + 1e-5 S."""
    got, ref, S = (np.asarray(x, dtype=np.float64).ravel() for x in (got, ref, S))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    _check(err, TOL[dt] * S, got, ref, S, what, "tolerance")
    if dt == "bf16":
        _check(err, BF16_ROUND * np.abs(ref) + BF16_ACC * S, got, ref, S, what,
               "the fp32-accumulate + one-rounding bound")


def node_major(act):
    """The same activations stored feature-major (F x B)."""
    if act.layout == "node":
        return act
    data = np.ascontiguousarray(act.data.reshape(act.B, act.F).T).ravel()
    return synth.Activation(data, act.dtype, act.B, act.F, "node")


def topology(w, max_batch, tile=0, flags=0):
    import unstructured_sparse_nn_amd as snk
    return snk.Topology(to_dev(w.row), to_dev(w.col), w.M, w.K, max_batch, tile, flags=flags)
