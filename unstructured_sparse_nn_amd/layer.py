"""Torch-facing wrappers: a prepared sparse topology and the SparseLinear
module, the torch API for sparse training and restructuring ("Beyond Masked
Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU", Abstract).

Torch allocates the device buffers (and the small pinned host buffer through
which prepare and the restructure read their result words) and supplies the
stream; every product, gradient and restructuring step is a call into the
HIP library.
"""
from __future__ import annotations

import torch

from . import binding as B

# Widest batch of snack_spmm_bwd_fused (one workgroup column covers the batch).
FUSED_MAX_BATCH = 32


def fused_backward_pays(K: int, nnz: int, elem_bytes: int, batch: int) -> bool:
    """Whether one snack_spmm_bwd_fused call beats the two separate gradient
    calls.  The fused pass reads the index stream once, but it runs one wave
    per column and writes dV through perm, scattered over the row-ordered
    array.  Measured on MI355X (cold, graph-timed): it pays with >= 2,048
    columns and a batch of 32 (4096^2 at 80-95%: 9-15% faster), a batch of
    8 with dV <= 2 MB, or dV <= 1 MB (2048^2 at 90%: 8-28% faster); larger
    dV at small batches costs up to twice the separate calls (8192^2 at 95%,
    batch 1: 33.7 against 17.1 us; LLaMA-shaped layers 40-70% slower), and 768
    columns leave too few waves (GPT-2 W1, batch 32: 22.1 against 14.0 us)."""
    if batch < 1 or batch > FUSED_MAX_BATCH or K < 2048:
        return False
    dv = nnz * elem_bytes
    return batch >= 32 or (batch >= 8 and dv <= 2 << 20) or dv <= 1 << 20


class Topology:
    """COO pattern (row, col int32 on the GPU) plus its prepared plan."""

    def __init__(self, row: torch.Tensor, col: torch.Tensor, M: int, K: int, max_batch: int,
                 tile_items: int = 0, stream=None, flags: int = 0):
        assert row.dtype == torch.int32 and col.dtype == torch.int32 and row.is_cuda
        self.row, self.col, self.M, self.K = row, col, M, K
        self.max_batch, self.tile_items, self.flags = max_batch, tile_items, flags
        self.prepare(stream)

    @property
    def nnz(self) -> int:
        return int(self.row.numel())

    def prepare(self, stream=None):
        self.plan = B.snack_plan_init(self.M, self.K, self.nnz, self.max_batch, self.tile_items,
                                      self.flags)
        self.arena = torch.empty(self.plan.arena_bytes, dtype=torch.uint8, device=self.row.device)
        # pinned host words: prepare and the restructure read their few result
        # words from here with no copy (without them: a copy and a sync)
        self.host_words = torch.zeros(B.HOST_WORDS_BYTES // 4, dtype=torch.int32,
                                      pin_memory=True)
        self.plan.host_words = self.host_words.data_ptr()
        try:
            B.snack_coo_prepare(self.plan, self.row, self.col, self.arena, stream)
        except B.SnackError as e:
            if e.status != -9:  # SNACK_E_WORKSPACE: the pinned words are not device-mapped
                raise
            self.plan.host_words = None
            B.snack_coo_prepare(self.plan, self.row, self.col, self.arena, stream)

    def restructure(self, vals, n_drop: int, seed: int, step: int, dropped=None, grown=None,
                    ws=None, stream=None, vals_t=None, flags: int = 0):
        """One prune/regrow step on (row, col, vals) in place, re-preparing this
        plan in the same call (snack_prune_regrow_prepared); vals_t, if given,
        receives the new values in the new column order."""
        if ws is None:
            ws = torch.empty(B.snack_prune_regrow_workspace(self.M, self.K, self.nnz, n_drop,
                                                            flags),
                             dtype=torch.uint8, device=self.row.device)
        B.snack_prune_regrow_prepared(self.plan, self.row, self.col, vals, n_drop, seed, step,
                                      dropped, grown, ws, stream, vals_t=vals_t, flags=flags)

    def array(self, name: str) -> torch.Tensor:
        """A derived array of the plan as an int32 view into the arena."""
        _, n = B.snack_plan_array(self.plan, name)
        off = self.plan.off[B.ARRAYS[name]]
        return self.arena[off:off + 4 * n].view(torch.int32)

    # products ------------------------------------------------------------
    def fwd(self, vals, X, Bsz, layout=B.BATCH_MAJOR, out=None):
        Y = out if out is not None else torch.empty(Bsz * self.M, dtype=X.dtype, device=X.device)
        B.snack_spmm_fwd(self.plan, vals, X, layout, Bsz, Y)
        return Y

    def bwd_input(self, vals, dY, Bsz, layout=B.BATCH_MAJOR, out=None):
        dX = out if out is not None else torch.empty(Bsz * self.K, dtype=dY.dtype,
                                                     device=dY.device)
        B.snack_spmm_bwd_input(self.plan, vals, dY, layout, Bsz, dX)
        return dX

    def gather_vals_t(self, vals, out=None):
        """The values in this plan's column order (vals_t[i] = vals[perm[i]])."""
        vt = out if out is not None else torch.empty_like(vals)
        B.snack_gather_vals_t(self.plan, vals, vt)
        return vt

    def bwd_input_t(self, vals_t, dY, Bsz, layout=B.BATCH_MAJOR, out=None):
        """dX = dY W from the values in column order."""
        dX = out if out is not None else torch.empty(Bsz * self.K, dtype=dY.dtype,
                                                     device=dY.device)
        B.snack_spmm_bwd_input_t(self.plan, vals_t, dY, layout, Bsz, dX)
        return dX

    def grad_vals(self, dY, X, Bsz, layout=B.BATCH_MAJOR, out=None):
        dV = out if out is not None else torch.empty(self.nnz, dtype=X.dtype, device=X.device)
        B.snack_sddmm_grad_vals(self.plan, dY, X, layout, Bsz, dV)
        return dV


class _SparseLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, vals, layer):
        topo = layer.topo
        Bsz = x.shape[0]
        xc = x.contiguous()
        ctx.layer = layer
        ctx.save_for_backward(xc, vals)
        return topo.fwd(vals, xc.view(-1), Bsz).view(Bsz, topo.M)

    @staticmethod
    def backward(ctx, gy):
        xc, vals = ctx.saved_tensors
        layer = ctx.layer
        topo = layer.topo
        Bsz = xc.shape[0]
        g = gy.contiguous().view(-1)
        vt = layer.vals_t()  # the values in column order: read coalesced by the input gradient
        if (ctx.needs_input_grad[0] and ctx.needs_input_grad[1]
                and fused_backward_pays(topo.K, topo.nnz, vals.element_size(), Bsz)):
            # both gradients from one pass over the column view (snack_spmm_bwd_fused)
            gx = torch.empty(Bsz * topo.K, dtype=g.dtype, device=g.device)
            gv = torch.empty(topo.nnz, dtype=g.dtype, device=g.device)
            B.snack_spmm_bwd_fused(topo.plan, vals, xc.view(-1), g, B.BATCH_MAJOR, Bsz, gx, gv,
                                   vals_t=vt)
            return gx.view(Bsz, topo.K), gv, None
        gx = topo.bwd_input_t(vt, g, Bsz).view(Bsz, topo.K) if ctx.needs_input_grad[0] else None
        gv = topo.grad_vals(g, xc.view(-1), Bsz) if ctx.needs_input_grad[1] else None
        return gx, gv, None


class SparseLinear(torch.nn.Module):
    """y = x W^T with W held only as its nonzeros (no bias).

    ``prune_regrow(frac_ppm, step)`` drops the smallest-magnitude fraction of
    the connections and regrows as many at seeded random free positions
    (value 0), then re-prepares the topology.

    The layer keeps a second copy of the values in the topology's column
    order, which the input gradient reads coalesced.  It is refreshed by one
    gather whenever the values tensor is replaced or changed by torch (its
    version counter moves, as with an optimiser step), and written directly by
    the restructure."""

    def __init__(self, in_features: int, out_features: int, row, col, vals, max_batch: int,
                 seed: int = 0, tile_items: int = 0):
        super().__init__()
        self.in_features, self.out_features, self.seed = in_features, out_features, seed
        self.topo = Topology(row, col, out_features, in_features, max_batch, tile_items)
        self.vals = torch.nn.Parameter(vals)
        self._vals_t = None
        self._vals_t_key = None

    def _key(self):
        v = self.vals
        return (v.data_ptr(), v._version, v.dtype, v.numel())

    def vals_t(self) -> torch.Tensor:
        """The values in column order, gathered again only if they changed."""
        key = self._key()
        if self._vals_t is None or self._vals_t_key != key:
            if self._vals_t is None or self._vals_t.dtype != self.vals.dtype or \
                    self._vals_t.numel() != self.vals.numel():
                self._vals_t = torch.empty_like(self.vals.data)
            self.topo.gather_vals_t(self.vals.data, out=self._vals_t)
            self._vals_t_key = key
        return self._vals_t

    def forward(self, x):
        return _SparseLinearFn.apply(x, self.vals, self)

    @torch.no_grad()
    def prune_regrow(self, frac_ppm: int, step: int):
        t = self.topo
        n_drop = B.snack_drop_count(t.nnz, frac_ppm)
        dropped = torch.empty(max(n_drop, 1), dtype=torch.int64, device=t.row.device)
        grown = torch.empty(max(n_drop, 1), dtype=torch.int64, device=t.row.device)
        if self._vals_t is None or self._vals_t.dtype != self.vals.dtype:
            self._vals_t = torch.empty_like(self.vals.data)
        t.restructure(self.vals.data, n_drop, self.seed, step, dropped, grown,
                      vals_t=self._vals_t)
        self._vals_t_key = self._key()  # written by the restructure itself
        return dropped[:n_drop], grown[:n_drop]
