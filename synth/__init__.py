"""Seeded synthetic inputs for the truly sparse linear layer.

This module only draws inputs: sparsity patterns, weight values, activations
and upstream gradients.  It holds none of the layer's arithmetic (no
products, no reductions, no pruning), so that both the serial CPU oracle and
the HIP path can consume exactly the same bits without sharing any code of
the method itself.

Workloads follow the shapes the SNACK abstract describes ("Beyond Masked
Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU", Abstract): a
single layer, GPT-2- and LLaMA-shaped projections and a graph-style layer,
all in the small-batch, high-sparsity regime.  There is no dataset; every
tensor is drawn from a seeded ``numpy.random.Generator``.

Conventions
-----------
* A sparse weight W is ``M x K`` (out_features x in_features) stored as COO:
  ``row``/``col`` int32, strictly increasing in ``row*K + col``.
* ``nnz`` for a sparsity ``s`` is ``round_half_up((1 - s) * M * K)`` computed
  exactly with rationals.
* bf16 tensors are carried as their raw ``uint16`` bit patterns, obtained
  from float32 draws by round-to-nearest-even.
* Batch-major activations are ``B x K`` (``X[b*K + k]``); node-major ones are
  ``K x B`` (``X[k*B + b]``).
* Per-tensor random streams come from ``numpy.random.SeedSequence(seed)
  .spawn(6)`` in the fixed order: positions, values, X, dY, row permutation,
  columns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

STREAMS = ("positions", "values", "x", "dy", "rowperm", "columns")


def _streams(seed: int) -> dict:
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(STREAMS, kids)}


def nnz_for(M: int, K: int, sparsity) -> int:
    """Round-half-up of (1 - sparsity) * M * K, computed exactly."""
    dens = Fraction(1) - Fraction(str(sparsity))
    q = dens * M * K
    return int((q + Fraction(1, 2)).__floor__())


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (input preparation)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# sparsity patterns
# --------------------------------------------------------------------------
def uniform_positions(rng, M: int, K: int, nnz: int) -> np.ndarray:
    """nnz distinct linear positions, uniform without replacement, sorted."""
    total = M * K
    if nnz > total:
        raise ValueError("nnz exceeds M*K")
    if nnz == 0:
        return np.zeros(0, dtype=np.int64)
    if nnz * 2 > total:
        keep = rng.permutation(total)[:nnz]
        return np.sort(keep).astype(np.int64)
    out = np.zeros(0, dtype=np.int64)
    while out.size < nnz:
        need = nnz - out.size
        draw = rng.integers(0, total, size=int(need * 1.1) + 16, dtype=np.int64)
        out = np.union1d(out, draw)
    if out.size > nnz:
        # drop a uniformly chosen surplus so the kept set stays uniform
        drop = rng.choice(out.size, out.size - nnz, replace=False)
        out = np.delete(out, drop)
    return out


def rank_profile(n_rows: int, cap: int, total: int, s: float, lo: int = 1) -> np.ndarray:
    """Deterministic power-law row degrees d_i ~ c * i^-s (ranks i = 1..n).

    c is found by bisection so that sum(clip(c*i^-s, lo, cap)) equals
    ``total``; the real profile is then made integral by flooring and
    handing the deficit out by largest remainder (ties to the lower rank),
    never above ``cap``.  Returned in rank order (largest first).
    """
    if not (n_rows * lo <= total <= n_rows * cap):
        raise ValueError("total nnz not reachable with these bounds")
    ranks = np.arange(1, n_rows + 1, dtype=np.float64)
    base = ranks ** (-float(s))
    lo_c, hi_c = 0.0, cap / base[-1] * 2.0
    for _ in range(300):
        mid = 0.5 * (lo_c + hi_c)
        if np.clip(mid * base, lo, cap).sum() < total:
            lo_c = mid
        else:
            hi_c = mid
    d = np.clip(hi_c * base, lo, cap)
    fl = np.floor(d)
    deficit = int(total - fl.sum())
    if deficit < 0:
        raise RuntimeError("rank profile bisection overshot")
    rem = d - fl
    eligible = np.nonzero(fl < cap)[0]
    order = eligible[np.lexsort((eligible, -rem[eligible]))]
    fl[order[:deficit]] += 1
    out = fl.astype(np.int64)
    assert out.sum() == total and out.max() <= cap and out.min() >= lo
    return out


def skewed_positions(streams, M: int, K: int, total: int, s: float, lo: int = 1):
    """Rows get degrees from ``rank_profile`` (ranks assigned to rows by a
    seeded permutation); columns are uniform without replacement within a
    row.  Returns sorted linear positions."""
    deg_rank = rank_profile(M, K, total, s, lo)
    perm = streams["rowperm"].permutation(M)
    deg = np.empty(M, dtype=np.int64)
    deg[perm] = deg_rank
    crng = streams["columns"]
    rows = np.repeat(np.arange(M, dtype=np.int64), deg)
    cols = np.empty(total, dtype=np.int64)
    starts = np.concatenate(([0], np.cumsum(deg)))
    one = np.nonzero(deg == 1)[0]
    cols[starts[one]] = crng.integers(0, K, size=one.size, dtype=np.int64)
    for r in np.nonzero(deg > 1)[0]:
        d = int(deg[r])
        cols[starts[r]:starts[r + 1]] = np.sort(crng.choice(K, d, replace=False))
    return rows * K + cols


# --------------------------------------------------------------------------
# layer / workload containers
# --------------------------------------------------------------------------
@dataclass
class SparseWeight:
    M: int
    K: int
    row: np.ndarray          # int32 [nnz]
    col: np.ndarray          # int32 [nnz]
    vals: np.ndarray         # float32 or uint16 (bf16 bits) [nnz]
    dtype: str               # "f32" | "bf16"

    @property
    def nnz(self) -> int:
        return int(self.row.size)

    def vals_f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.vals).astype(np.float64)
        return self.vals.astype(np.float64)


@dataclass
class Activation:
    data: np.ndarray         # float32 or uint16 (bf16 bits), flat
    dtype: str
    B: int
    F: int                   # features (K for X, M for dY)
    layout: str              # "batch" (B x F) | "node" (F x B)

    def f64(self) -> np.ndarray:
        a = bf16_bits_to_f32(self.data) if self.dtype == "bf16" else self.data
        return a.astype(np.float64)


@dataclass
class Workload:
    name: str
    weights: list
    B: int
    X: list                  # one Activation per weight (input of that weight)
    dY: list                 # one Activation per weight (gradient of its output)
    meta: dict = field(default_factory=dict)


def weight_from_positions(lin, M, K, vals_f32, dtype) -> SparseWeight:
    lin = np.asarray(lin, dtype=np.int64)
    row = (lin // K).astype(np.int32)
    col = (lin % K).astype(np.int32)
    v = np.asarray(vals_f32, dtype=np.float32)
    if dtype == "bf16":
        v = f32_to_bf16_bits(v)
    return SparseWeight(M, K, row, col, v, dtype)


def normal_weight(streams, M, K, nnz, dtype, std=0.02) -> SparseWeight:
    lin = uniform_positions(streams["positions"], M, K, nnz)
    v = (streams["values"].standard_normal(nnz) * std).astype(np.float32)
    return weight_from_positions(lin, M, K, v, dtype)


def activation(rng, B, F, dtype, layout="batch") -> Activation:
    a = rng.standard_normal(B * F).astype(np.float32)
    if dtype == "bf16":
        a = f32_to_bf16_bits(a)
    return Activation(a, dtype, B, F, layout)


# --------------------------------------------------------------------------
# the five workloads (shapes from the layer's benchmark table) and extras
# --------------------------------------------------------------------------
def single_layer(seed=0, M=256, K=256, sparsity=0.9, B=4, dtype="f32") -> Workload:
    """256x256 layer at 90% (6,554 nnz), fp32, batch 4, plus dY."""
    st = _streams(seed)
    w = normal_weight(st, M, K, nnz_for(M, K, sparsity), dtype)
    X = activation(st["x"], B, K, dtype)
    dY = activation(st["dy"], B, M, dtype)
    return Workload("single_layer", [w], B, [X], [dY],
                    {"sparsity": sparsity, "drop_ppm": 100000})


def inference_layer(seed=0, N=4096, sparsity=0.95, B=8, dtype="bf16", with_dy=True) -> Workload:
    """4096x4096 at 95% (838,861 nnz), bf16 values and activations."""
    st = _streams(seed)
    w = normal_weight(st, N, N, nnz_for(N, N, sparsity), dtype)
    X = activation(st["x"], B, N, dtype)
    dY = activation(st["dy"], B, N, dtype) if with_dy else None
    return Workload(f"square{N}_s{sparsity}_B{B}_{dtype}", [w], B, [X], [dY],
                    {"sparsity": sparsity})


def gpt2_mlp(seed=0, sparsity=0.9, B=1024, d_model=768, d_ff=3072, dtype="f32") -> Workload:
    """GPT-2-small MLP: W1 d_ff x d_model, GELU, W2 d_model x d_ff."""
    st = _streams(seed)
    w1 = normal_weight(st, d_ff, d_model, nnz_for(d_ff, d_model, sparsity), dtype)
    w2 = normal_weight(st, d_model, d_ff, nnz_for(d_model, d_ff, sparsity), dtype)
    X = activation(st["x"], B, d_model, dtype)
    dY = activation(st["dy"], B, d_model, dtype)
    return Workload(f"gpt2_mlp_s{sparsity}", [w1, w2], B, [X, None], [None, dY],
                    {"sparsity": sparsity, "drop_ppm": 300000})


def llama_proj(seed=0, which="up", B=4, sparsity=0.9, dtype="bf16", zipf=1.2) -> Workload:
    """LLaMA-7B projections with power-law row degrees (same total nnz)."""
    st = _streams(seed)
    M, K = (11008, 4096) if which == "up" else (4096, 11008)
    nnz = nnz_for(M, K, sparsity)
    lin = skewed_positions(st, M, K, nnz, zipf, lo=1)
    v = (st["values"].standard_normal(nnz) * 0.02).astype(np.float32)
    w = weight_from_positions(lin, M, K, v, dtype)
    X = activation(st["x"], B, K, dtype)
    dY = activation(st["dy"], B, M, dtype)
    return Workload(f"llama_{which}_B{B}", [w], B, [X], [dY], {"sparsity": sparsity})


def graph_layer(seed=0, n=200_000, nnz=2_400_000, B=128, zipf=1.1) -> Workload:
    """Power-law adjacency (row degrees >= 1), random-walk normalised
    values, node-major fp32 features n x B."""
    st = _streams(seed)
    lin = skewed_positions(st, n, n, nnz, zipf, lo=1)
    u = st["values"].random(nnz)
    rows = lin // n
    rs = np.bincount(rows, weights=u, minlength=n)
    v = (u / rs[rows]).astype(np.float32)
    w = weight_from_positions(lin, n, n, v, "f32")
    X = activation(st["x"], B, n, "f32", layout="node")
    dY = activation(st["dy"], B, n, "f32", layout="node")
    return Workload("graph200k", [w], B, [X], [dY], {"nnz": nnz})


def random_case(seed, M, K, nnz, B, dtype="f32", layout="batch", positions=None) -> Workload:
    """Small generic case for parity sweeps and edge cases."""
    st = _streams(seed)
    lin = (uniform_positions(st["positions"], M, K, nnz) if positions is None
           else np.asarray(positions, dtype=np.int64))
    v = (st["values"].standard_normal(lin.size) * 0.02).astype(np.float32)
    w = weight_from_positions(lin, M, K, v, dtype)
    X = activation(st["x"], B, K, dtype, layout)
    dY = activation(st["dy"], B, M, dtype, layout)
    return Workload(f"case_{M}x{K}_{lin.size}_B{B}_{dtype}_{layout}", [w], B, [X], [dY])
