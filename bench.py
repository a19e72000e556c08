"""Benchmark of the truly sparse layer's hot path on one MI355X.

One step = one dynamic-sparse-training step of a 4096 x 4096 layer at 95%
sparsity (838,861 nnz, bf16 values and activations, fp32 accumulation) on a
batch of 32:
    forward Y = X W^T  ->  input gradient dX = dY W (values read in column
    order)  ->  value gradient dV = (dY^T X) at the nonzeros  ->  prune/regrow
    of 30% of the connections  ->  re-prepare the topology (offsets, tiles,
    column view, column-ordered values); the last two are one call
    (snack_prune_regrow_prepared) unless --restructure separate.
The metric is the fwd+bwd SpMM bandwidth: algorithmic bytes of the three
products (values + indices + offsets + activations read + outputs written)
per second of whole-step time.  Inputs are resident in HBM before timing;
the step rotates over 20 independent layer instances (~1.2 GB touched per
rotation) so that each step reads from HBM rather than the 256 MB Infinity
Cache.

Per-op kernel times (``ops``, ``grid``, ``sweep``, ``baselines``) are cold:
each op rotates over enough distinct instances that at least 512 MB of the
data it touches lies between two uses of one instance.  ``ops_warm`` repeats
one instance (cache-resident) for comparison.  ``calibration`` holds the
machine floors measured in the same run (empty kernel, streaming read and
write, dependent-load latency).

Prints one JSON line (see --help).  --gpus > 1 is not supported: the layer
runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd SpMM GB/s and % HBM roofline at 95%/99% sparsity, batch 1–32"
HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def algo_bytes(op: str, M: int, K: int, nnz: int, B: int, s_w: int, s_a: int,
               s_idx: int = 4) -> int:
    """Minimum bytes an op must move: every stored value and its index once,
    the segment offsets, the activations read and the output written."""
    if op == "fwd":
        return nnz * (s_idx + s_w) + s_idx * (M + 1) + B * K * s_a + B * M * s_a
    if op == "bwd_input":
        return nnz * (s_idx + s_w) + s_idx * (K + 1) + B * M * s_a + B * K * s_a
    if op == "sddmm":  # reads indices, writes one value per nonzero
        return nnz * (s_idx + s_w) + s_idx * (M + 1) + B * K * s_a + B * M * s_a
    if op == "bwd_fused":  # one index stream: reads v, writes dV; reads dY and X, writes dX
        return nnz * (s_idx + 2 * s_w) + s_idx * (K + 1) + B * M * s_a + 2 * B * K * s_a
    raise KeyError(op)


def restructure_bytes(M: int, K: int, nnz: int, s_w: int, P_row: int, P_col: int) -> int:
    """Minimum bytes of one restructure with the re-prepared plan: the COO
    read and written back (two int32 indices and a value per connection,
    each way), the plan's derived arrays written (row and column offsets,
    perm and row_t, the tiles and cut flags of both views) and the
    column-ordered values written."""
    coo = nnz * (8 + s_w)
    plan = 4 * (M + 1) + 4 * (K + 1) + 8 * nnz + 12 * (P_row + 1) + 12 * (P_col + 1)
    return 2 * coo + plan + nnz * s_w


COLD_BYTES = 512e6  # data an op touches between two uses of one instance (> 256 MB MALL)


def rotation_for(op_bytes: int, cap: int = 600) -> int:
    """Instances to rotate so that >= COLD_BYTES of an op's data lies between
    two uses of one instance."""
    return max(2, min(cap, int(-(-COLD_BYTES // op_bytes)) + 1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--sparsity", type=float, default=0.95)
    ap.add_argument("--size", type=int, default=4096)
    ap.add_argument("--drop-ppm", type=int, default=300000)
    ap.add_argument("--layout", choices=("node", "batch"), default="node",
                    help="activation layout in HBM: node = feature-major K x B (the "
                         "layer's native layout), batch = B x K (adds transposes)")
    ap.add_argument("--rotate", type=int, default=20,
                    help="layer instances cycled through (1 = cache-warm)")
    ap.add_argument("--grid", action=argparse.BooleanOptionalAction, default=True,
                    help="also time fwd/dX/dV at 95/99%% x B in {1,8,32} (cold)")
    ap.add_argument("--sizes", default="8192,16384,32768",
                    help="square sizes of the cold size sweep of fwd/dX/dV at 95/99%% x B in "
                         "{1,8,32} ('' = none)")
    ap.add_argument("--calibrate", action=argparse.BooleanOptionalAction, default=True,
                    help="measure the machine floors (empty kernel, stream read/write, latency)")
    ap.add_argument("--cpu-baseline", action=argparse.BooleanOptionalAction, default=True)
    ap.add_argument("--conv", action=argparse.BooleanOptionalAction, default=True,
                    help="time a sparse 1x1 convolution (generated kernel, generic, dense)")
    ap.add_argument("--fixed-full", action="store_true",
                    help="also generate fixed-pattern kernels for full-size layers (GPT-2 "
                         "W1/W2 at 90%%, 4096^2 at 99%%; minutes of compilation) and time them "
                         "against the generic forward")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="time multi-layer graph inference (power-law graphs, fused GELU)")
    ap.add_argument("--configs", action=argparse.BooleanOptionalAction, default=True,
                    help="also time fwd/dX/dV on the other layer configurations (one instance "
                         "each, graph-timed)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--restructure", choices=("fused", "separate"), default="fused",
                    help="prune/regrow + prepare as one call (snack_prune_regrow_prepared) or "
                         "as two")
    ap.add_argument("--products-only", action="store_true",
                    help="time only fwd/dX/dV (for profiling the product kernels)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this size (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a, bf16=False):
    import torch
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.copy()).cuda()


def layout_data(act, layout):
    """Synthetic activations are drawn batch-major (B x F); node-major keeps
    the same values feature-major (F x B)."""
    if layout == "node" and act.B > 1:
        return np.ascontiguousarray(act.data.reshape(act.B, act.F).T)
    return act.data


class Instance:
    """One layer: COO + values (+ column-ordered copy) + activations + prepared
    topology + outputs; with ``restructure`` also a restructuring workspace.
    ``like`` clones another instance's host-side inputs on the device (distinct
    buffers, same contents) instead of copying them from the host again."""

    def __init__(self, w, X, dY, B, bf16, drop_ppm, layout="node", restructure=True, like=None):
        import torch
        import unstructured_sparse_nn_amd as snk
        wt = w
        self.M, self.K, self.B, self.nnz = wt.M, wt.K, B, wt.nnz
        self.lay = snk.NODE_MAJOR if layout == "node" else snk.BATCH_MAJOR
        if like is None:
            self.row, self.col = to_dev(wt.row), to_dev(wt.col)
            self.vals = to_dev(wt.vals, bf16)
            self.X = to_dev(layout_data(X, layout), bf16)
            self.dY = to_dev(layout_data(dY, layout), bf16)
        else:
            self.row, self.col, self.vals = like.row.clone(), like.col.clone(), like.vals.clone()
            self.X, self.dY = like.X.clone(), like.dY.clone()
        dt = self.vals.dtype
        self.Y = torch.empty(B * wt.M, dtype=dt, device="cuda")
        self.dX = torch.empty(B * wt.K, dtype=dt, device="cuda")
        self.dV = torch.empty(wt.nnz, dtype=dt, device="cuda")
        self.topo = snk.Topology(self.row, self.col, wt.M, wt.K, B,
                                 flags=snk.binding.PLAN_NODE_MAJOR_ONLY if layout == "node" else 0)
        # the values in column order, read coalesced by the input gradient;
        # kept in step by the restructure, which writes them
        self.vals_t = self.topo.gather_vals_t(self.vals)
        self.n_drop = snk.snack_drop_count(wt.nnz, drop_ppm)
        self.ws = None
        if restructure:
            self.ws = torch.empty(snk.snack_prune_regrow_workspace(wt.M, wt.K, wt.nnz,
                                                                   self.n_drop),
                                  dtype=torch.uint8, device="cuda")
        self.step_no = 0

    def products(self, ev=None):
        t = self.topo
        if ev: ev[0].record()
        t.fwd(self.vals, self.X, self.B, self.lay, out=self.Y)
        if ev: ev[1].record()
        t.bwd_input_t(self.vals_t, self.dY, self.B, self.lay, out=self.dX)
        if ev: ev[2].record()
        t.grad_vals(self.dY, self.X, self.B, self.lay, out=self.dV)
        if ev: ev[3].record()

    def bwd_fused(self, lr=0.0):
        """dX and dV in one pass (snack_spmm_bwd_fused); with lr != 0 the SGD
        step on both copies of the values."""
        import unstructured_sparse_nn_amd as snk
        snk.snack_spmm_bwd_fused(self.topo.plan, self.vals, self.X, self.dY, self.lay, self.B,
                                 self.dX, self.dV, lr, vals_t=self.vals_t)

    def restructure(self, ev=None, fused=True):
        import unstructured_sparse_nn_amd as snk
        self.step_no += 1
        if fused:  # prune/regrow and re-prepare in one call
            snk.snack_prune_regrow_prepared(self.topo.plan, self.row, self.col, self.vals,
                                            self.n_drop, 0, self.step_no, None, None, self.ws,
                                            vals_t=self.vals_t)
            if ev: ev[4].record()
            return
        snk.snack_prune_regrow(self.row, self.col, self.vals, self.M, self.K, self.topo.nnz,
                               self.n_drop, 0, self.step_no, None, None, self.ws)
        if ev: ev[4].record()
        snk.snack_coo_prepare(self.topo.plan, self.row, self.col, self.topo.arena)
        snk.snack_gather_vals_t(self.topo.plan, self.vals, self.vals_t)
        if ev: ev[5].record()


def make_instances(w, X, dY, B, R, layout="node", restructure=False, drop_ppm=0):
    """R product instances of one layer (bf16), the first from the host, the
    rest cloned on the device."""
    first = Instance(w, X, dY, B, True, drop_ppm, layout, restructure)
    out = [first]
    for _ in range(R - 1):
        out.append(Instance(w, X, dY, B, True, drop_ppm, layout, restructure, like=first))
    return out


def op_fn(inst, op):
    """The call of one product op on one instance."""
    t = inst.topo
    if op == "fwd":
        return lambda: t.fwd(inst.vals, inst.X, inst.B, inst.lay, out=inst.Y)
    if op == "bwd_input":
        return lambda: t.bwd_input_t(inst.vals_t, inst.dY, inst.B, inst.lay, out=inst.dX)
    if op == "bwd_input_perm":
        return lambda: t.bwd_input(inst.vals, inst.dY, inst.B, inst.lay, out=inst.dX)
    if op == "sddmm":
        return lambda: t.grad_vals(inst.dY, inst.X, inst.B, inst.lay, out=inst.dV)
    if op == "bwd_fused":
        return lambda: inst.bwd_fused()
    raise KeyError(op)


def graph_us(fns, launches=None, replays=3):
    """Mean duration of one launch, from HIP events around replays of a
    captured graph of back-to-back launches cycling through ``fns`` (so no
    host work sits between the kernels).  With len(fns) instances of ``B``
    bytes each, consecutive uses of one instance are len(fns) - 1 instances'
    data apart."""
    import torch
    n = len(fns)
    launches = launches or max(n, 20)
    for i in range(min(n, 3)):
        fns[i]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fns[i % n]()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (launches * replays)
    del g
    return us


def graph_kernel_us(insts, op, launches=None, replays=3):
    return graph_us([op_fn(i, op) for i in insts], launches, replays)


def src_hash():
    h = hashlib.sha256()
    for f in ("spmm.hip", "wave.hip", "wave.h", "wave_kernels.h", "common.h"):
        h.update(open(os.path.join(ROOT, "unstructured_sparse_nn_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(name, launches_bytes):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_sha") != src_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def dense_baselines(wt, X, batches, sparse_us, read_floor_us=None):
    """Forward time of the in-repo dense and Dense+Mask kernels
    (snack_dense_fwd) on the same layer, graph-timed like the sparse products
    and cold the same way (>= 512 MB of weights, masks and activations between
    two uses of one copy).  sparse_us: the cold sparse forward per batch;
    read_floor_us: a cold streaming read of the dense weight's bytes on this
    box (calibration), the floor the dense kernel's own weight stream meets."""
    import torch
    import unstructured_sparse_nn_amd as snk
    M, K = wt.M, wt.K
    dense = np.zeros(M * K, dtype=np.uint16)
    dense[wt.row.astype(np.int64) * K + wt.col] = wt.vals
    mask = np.zeros(M * K, dtype=np.uint8)
    mask[wt.row.astype(np.int64) * K + wt.col] = 1
    w0 = torch.from_numpy(dense.view(np.int16)).view(torch.bfloat16).cuda()
    m0 = torch.from_numpy(mask).cuda()
    out = {}
    for kind, use_mask in (("dense", False), ("dense_mask", True)):
        per = M * K * 2 + (M * K if use_mask else 0)
        R = rotation_for(per)
        Wd = [w0] + [w0.clone() for _ in range(R - 1)]
        Md = ([m0] + [m0.clone() for _ in range(R - 1)]) if use_mask else [None] * R
        for B in batches:
            xb = torch.from_numpy(X.data[:B * K].view(np.int16)).view(torch.bfloat16).cuda()
            Y = torch.empty(B * M, dtype=torch.bfloat16, device="cuda")
            fns = [(lambda i=i: snk.snack_dense_fwd(Wd[i], Md[i], M, K, xb, B, Y))
                   for i in range(R)]
            us = graph_us(fns)
            nbytes = per + B * (K + M) * 2
            rec = {"us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                   "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4), "rotate": R,
                   "floor_us_at_8TBps": round(nbytes / HBM_PEAK_GBPS / 1e3, 2)}
            if read_floor_us and not use_mask:
                rec["weight_read_floor_us"] = read_floor_us
                rec["over_weight_read_floor"] = round(us / read_floor_us, 2)
            if B in sparse_us:
                rec["sparse_fwd_us"] = sparse_us[B]
                rec["sparse_fwd_speedup"] = round(us / sparse_us[B], 2)
                # against the dense layer's own byte floor: what a perfect dense
                # kernel would give
                rec["sparse_fwd_speedup_vs_floor"] = round(rec["floor_us_at_8TBps"]
                                                           / sparse_us[B], 2)
            out[f"{kind}_B{B}"] = rec
        del Wd, Md
        torch.cuda.empty_cache()
    return out


def calibrate():
    """Machine floors on this machine, same process: an empty kernel (graph-timed
    back-to-back launches), a 1 GiB streaming read and write, and the latency
    of dependent loads over 1 GiB (HBM) and over 2 MiB (L2)."""
    import torch
    import unstructured_sparse_nn_amd as snk
    B_ = snk.binding
    out = {}
    out["empty_kernel_us"] = round(graph_us([lambda: snk.snack_calibrate(B_.CALIB_EMPTY, n=1)],
                                            launches=50, replays=5), 2)
    nbytes = 1 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for name, kind in (("read", B_.CALIB_READ), ("write", B_.CALIB_WRITE)):
        us = graph_us([lambda k=kind: snk.snack_calibrate(k, buf, nbytes, 4096)], launches=4,
                      replays=3)
        out[f"stream_{name}_GBps"] = round(nbytes / us / 1e3, 1)
    # HBM: one pass right after the 1 GiB chain is written (the chain from
    # slot 0 was written first, so it has left the caches); L2: a 2 MiB chain,
    # warmed first
    for name, size, hops, warm in (("hbm", nbytes, 20000, 0), ("l2", 2 << 20, 100000, 1)):
        snk.snack_calibrate(B_.CALIB_CHAIN, buf, size)
        us = time_calls(lambda s=size, h=hops: snk.snack_calibrate(B_.CALIB_CHASE, buf, s, h),
                        reps=1, warm=warm)
        out[f"dependent_load_{name}_ns"] = round(us * 1e3 / hops, 1)
    # reads of 5.6 MB (one 4096^2 product launch's bytes), 1.0 MB (at 99%) and
    # 33.6 MB (the dense bf16 weight of the baselines), each over distinct
    # regions of the buffer (cold): the best a launch that size can do,
    # launch, ramp and drain included
    for tag, small in (("5.6MB", 5_573_888), ("1.0MB", 1_039_616), ("33.6MB", 33_554_432)):
        regions = min(64, nbytes // small)
        base = buf.data_ptr()
        fns = [(lambda a=base + k * small: snk.snack_calibrate(B_.CALIB_READ, a, small, 2048))
               for k in range(regions)]
        out[f"stream_read_{tag}_us"] = round(graph_us(fns, launches=regions, replays=3), 2)
    del buf
    torch.cuda.empty_cache()
    return out


def time_calls(fn, reps=10, warm=3):
    """Mean microseconds of fn() between HIP events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def time_config(w, B, bf16, layout, ops=("fwd", "bwd_input", "sddmm"), cold=True):
    """Per-launch time of each product on one layer configuration, from HIP
    events around graph replays.  cold: rotate over enough device copies of
    the layer (COO, plan, column-ordered values, activations, outputs) that
    >= 512 MB of an op's data lies between two uses of one copy; else one
    instance, caches warm."""
    import torch
    import unstructured_sparse_nn_amd as snk
    dt = torch.bfloat16 if bf16 else torch.float32
    lay = snk.NODE_MAJOR if layout == "node" else snk.BATCH_MAJOR
    s_el = 2 if bf16 else 4
    op_bytes = min(algo_bytes(op, w.M, w.K, w.nnz, B, s_el, s_el) for op in ops)
    R = rotation_for(op_bytes, cap=64) if cold else 1
    g = torch.Generator(device="cuda").manual_seed(0)
    row, col, vals = to_dev(w.row), to_dev(w.col), to_dev(w.vals, bf16)
    X0 = torch.randn(B * w.K, device="cuda", generator=g).to(dt)
    dY0 = torch.randn(B * w.M, device="cuda", generator=g).to(dt)
    insts = []
    for r in range(R):
        rr, cc, vv = (row, col, vals) if r == 0 else (row.clone(), col.clone(), vals.clone())
        topo = snk.Topology(rr, cc, w.M, w.K, B)
        insts.append({"topo": topo, "vals": vv, "vt": topo.gather_vals_t(vv),
                      "X": X0 if r == 0 else X0.clone(), "dY": dY0 if r == 0 else dY0.clone(),
                      "Y": torch.empty(B * w.M, dtype=dt, device="cuda"),
                      "dX": torch.empty(B * w.K, dtype=dt, device="cuda"),
                      "dV": torch.empty(w.nnz, dtype=dt, device="cuda")})

    def fn(d, op):
        t = d["topo"]
        if op == "fwd":
            return lambda: t.fwd(d["vals"], d["X"], B, lay, out=d["Y"])
        if op == "bwd_input":
            return lambda: t.bwd_input_t(d["vt"], d["dY"], B, lay, out=d["dX"])
        if op == "bwd_fused":  # dX and dV in one call, lr = 0 (the values stay)
            return lambda: snk.snack_spmm_bwd_fused(t.plan, d["vals"], d["X"], d["dY"], lay, B,
                                                    d["dX"], d["dV"], 0.0, vals_t=d["vt"])
        return lambda: t.grad_vals(d["dY"], d["X"], B, lay, out=d["dV"])

    plan = insts[0]["topo"].plan
    out = {"split_rows": int(plan.has_split_row), "split_cols": int(plan.has_split_col),
           "rotate": R, "cache": "cold (HBM)" if cold else "warm"}
    for op in ops:
        us = graph_us([fn(d, op) for d in insts], launches=max(R, 10))
        b = algo_bytes(op, w.M, w.K, w.nnz, B, s_el, s_el)
        out[op] = {"us": round(us, 2), "GBps": round(b / (us * 1e3), 1),
                   "frac": round(b / (us * 1e3) / HBM_PEAK_GBPS, 4),
                   "GFLOPs": round(2 * w.nnz * B / (us * 1e3), 1)}
    del insts
    torch.cuda.empty_cache()
    return out


def other_configs():
    """fwd, dX and dV on the other layer configurations: 256^2 at 90% (fp32,
    B=4, warm: it is launch-bound), the GPT-2-small MLP layers at 90% and 99%
    (fp32, 1024 tokens, batch-major), the LLaMA-7B-shaped projections with
    skewed rows (bf16, B = 1, 4, 16, node-major; also the fused backward, the
    layer's training path) and the 200,000-node graph
    (fp32, 128 node-major features; forward and input gradient), all cold
    but the first."""
    import synth
    out = {}
    log("configs: single layer")
    w = synth.single_layer()
    out["single_256_s0.9_B4_f32"] = time_config(w.weights[0], 4, False, "batch", cold=False)
    for sp in (0.9, 0.99):
        log(f"configs: gpt2 mlp {sp}")
        wl = synth.gpt2_mlp(sparsity=sp)
        for name, wt in (("W1_3072x768", wl.weights[0]), ("W2_768x3072", wl.weights[1])):
            out[f"gpt2_{name}_s{sp}_B1024_f32"] = time_config(wt, 1024, False, "batch")
    for which in ("up", "down"):
        log(f"configs: llama {which}")
        wt = synth.llama_proj(which=which, B=1).weights[0]
        for B in (1, 4, 16):
            out[f"llama_{which}_B{B}_bf16"] = time_config(
                wt, B, True, "node", ops=("fwd", "bwd_input", "sddmm", "bwd_fused"))
    log("configs: graph 200k")
    wt = synth.graph_layer().weights[0]
    out["graph_200k_B128_f32"] = time_config(wt, 128, False, "node", ops=("fwd", "bwd_input"))
    return out


def graph_inference(layers=3):
    """Multi-layer graph-style inference, H <- GELU(A H) `layers` times with A a
    synthetic power-law adjacency (random-walk weights) and 128 fp32 node-major
    features: (1) the 200,000-node, 2,400,000-edge graph, activation fused into
    the propagation (snack_graph_propagate) against a separate GELU pass;
    (2) a 16,384-node graph at 99% sparsity against the in-repo Dense+Mask and
    dense kernels on the same graph (snack_dense_fwd + snack_gelu_fwd per
    layer, batch-major)."""
    import torch
    import synth
    import unstructured_sparse_nn_amd as snk
    out = {}
    NM, F32, GELU = snk.NODE_MAJOR, snk.F32, snk.ACT_GELU

    def sparse_setup(wl):
        w, X = wl.weights[0], wl.X[0]
        topo = snk.Topology(to_dev(w.row), to_dev(w.col), w.M, w.K, wl.B,
                            flags=snk.binding.PLAN_NODE_MAJOR_ONLY)
        return w, topo, to_dev(w.vals), to_dev(X.data)

    def layer_bytes(w, Bsz):  # index + value per edge, offsets, H in and out (fp32)
        return w.nnz * 8 + 4 * (w.M + 1) + 2 * w.M * Bsz * 4

    log("graph inference: 200k nodes")
    wl = synth.graph_layer()
    w, topo, vals, X = sparse_setup(wl)
    Y, tmp, Z = torch.empty_like(X), torch.empty_like(X), torch.empty_like(X)

    def fused(act=GELU):
        snk.snack_graph_propagate(topo.plan, vals, X, NM, wl.B, layers, act, Y, tmp)

    def separate():
        src = X
        for l in range(layers):
            dst = Y if (layers - 1 - l) % 2 == 0 else tmp
            snk.snack_spmm_fwd(topo.plan, vals, src, NM, wl.B, Z)
            snk.snack_gelu_fwd(Z, dst)
            src = dst

    uf, us = time_calls(fused), time_calls(separate)
    un = time_calls(lambda: fused(snk.ACT_NONE))
    ur = time_calls(lambda: fused(snk.ACT_RELU))
    lb = layer_bytes(w, wl.B)
    out["graph200k"] = {"nodes": w.M, "edges": w.nnz, "features": wl.B, "layers": layers,
                        "us_gelu": round(uf, 1), "us_relu": round(ur, 1),
                        "us_no_act": round(un, 1), "us_gelu_two_calls": round(us, 1),
                        "GBps_relu": round(layers * lb / (ur * 1e3), 1),
                        "GBps_gelu": round(layers * lb / (uf * 1e3), 1),
                        "note": "snack_graph_propagate: ReLU applied in the product's store, "
                                "GELU as an in-place pass after each product; two_calls = "
                                "snack_spmm_fwd + snack_gelu_fwd per layer"}
    del topo, vals, X, Y, tmp, Z
    torch.cuda.empty_cache()

    log("graph inference: 16k nodes at 99% against Dense+Mask")
    n = 16384
    wl = synth.graph_layer(n=n, nnz=synth.nnz_for(n, n, 0.99), B=128)
    w, topo, vals, X = sparse_setup(wl)
    Y, tmp = torch.empty_like(X), torch.empty_like(X)
    us_sp = time_calls(lambda: snk.snack_graph_propagate(topo.plan, vals, X, NM, wl.B, layers,
                                                          GELU, Y, tmp))
    lin = torch.from_numpy(w.row.astype(np.int64) * n + w.col).cuda()
    Wd = torch.zeros(n * n, dtype=torch.float32, device="cuda")
    Wd[lin] = vals
    mask = torch.zeros(n * n, dtype=torch.uint8, device="cuda")
    mask[lin] = 1
    Xb = X.view(n, wl.B).t().contiguous()  # batch-major B x n
    Zb, Hb, Gb = torch.empty_like(Xb), torch.empty_like(Xb), torch.empty_like(Xb)

    def dense(m):
        src = Xb
        for l in range(layers):
            dst = Hb if (layers - 1 - l) % 2 == 0 else Gb
            snk.snack_dense_fwd(Wd, m, n, n, src, wl.B, Zb)
            snk.snack_gelu_fwd(Zb, dst)
            src = dst

    us_dm = time_calls(lambda: dense(mask), reps=3, warm=1)
    us_d = time_calls(lambda: dense(None), reps=3, warm=1)
    # same results: the last layer of both paths (node-major vs batch-major)
    diff = float((Y.view(n, wl.B).t() - Hb).abs().max())
    out["graph16k_s0.99"] = {"nodes": n, "edges": w.nnz, "features": wl.B, "layers": layers,
                             "act": "gelu", "us_sparse": round(us_sp, 1),
                             "us_dense_mask": round(us_dm, 1), "us_dense": round(us_d, 1),
                             "speedup_vs_dense_mask": round(us_dm / us_sp, 2),
                             "speedup_vs_dense": round(us_d / us_sp, 2),
                             "max_abs_diff_sparse_vs_dense": diff,
                             "dense_fp32_flop_floor_us": round(
                                 layers * 2 * n * n * wl.B / 157.3e12 * 1e6, 1)}
    del topo, vals, X, Y, tmp, Wd, mask, Xb, Zb, Hb, Gb, lin
    torch.cuda.empty_cache()
    return out


def conv1x1_bench(N=8, HW=56 * 56, C=256, sparsity=0.9):
    """A 1x1 convolution C -> C over N images of HW pixels at `sparsity`: the
    kernel generated for the fixed weight (NCHW, one launch), the generic
    products (NCHW: one node-major launch per image; NHWC: one batch-major
    launch), and the in-repo dense kernel on the same weight (NHWC)."""
    import torch
    import synth
    import unstructured_sparse_nn_amd as snk
    out = {}
    for dt in ("bf16", "f32"):
        wl = synth.random_case(23, C, C, synth.nnz_for(C, C, sparsity), 1, dt, "node")
        w = wl.weights[0]
        sd = snk.F32 if dt == "f32" else snk.BF16
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        t0 = time.time()
        f = snk.snack_fixed_build(w.row, w.col, w.vals, C, C, dtype=sd)
        build_s = time.time() - t0
        P = N * HW
        X = torch.randn(P * C, device="cuda").to(tdt)
        Y = torch.empty(P * C, dtype=tdt, device="cuda")
        topo = snk.Topology(to_dev(w.row), to_dev(w.col), C, C, P)
        vals = to_dev(w.vals, dt == "bf16")
        Wd = torch.zeros(C * C, dtype=tdt, device="cuda")
        Wd[torch.from_numpy(w.row.astype(np.int64) * C + w.col).cuda()] = vals
        t = {"fixed_nchw": time_calls(lambda: snk.snack_fixed_fwd(f, X, HW, N, Y)),
             "generic_nchw": time_calls(lambda: snk.snack_conv1x1(topo.plan, vals, X, N, HW,
                                                                  snk.CONV_NCHW, Y)),
             "generic_nhwc": time_calls(lambda: snk.snack_conv1x1(topo.plan, vals, X, N, HW,
                                                                  snk.CONV_NHWC, Y)),
             "dense_nhwc": time_calls(lambda: snk.snack_dense_fwd(Wd, None, C, C, X, P, Y))}
        act_bytes = 2 * P * C * (4 if dt == "f32" else 2)
        out[dt] = {"us": {k: round(v, 2) for k, v in t.items()},
                   "act_GBps_fixed": round(act_bytes / (t["fixed_nchw"] * 1e3), 1),
                   "fixed_vs_dense": round(t["dense_nhwc"] / t["fixed_nchw"], 2),
                   "fixed_vs_generic_nchw": round(t["generic_nchw"] / t["fixed_nchw"], 2),
                   "build_seconds": round(build_s, 2), **f.info()}
        f.free()
        del X, Y, topo, vals, Wd
        torch.cuda.empty_cache()
    return {"shape": f"{N}x{C}x56x56 -> {N}x{C}x56x56, 1x1, {sparsity:.0%} sparse "
                     f"({synth.nnz_for(C, C, sparsity)} nnz)", **out}


def fixed_full_bench():
    """Fixed-pattern kernels generated for full-size fully connected layers
    (node-major, one launch each) against the generic forward on the same
    weight and inputs; the generated code and its compile time grow with nnz
    (about a minute per 200K entries)."""
    import torch
    import synth
    import unstructured_sparse_nn_amd as snk
    out = {}
    for name, M, K, sp, B, dt in (("gpt2_W1_s0.9_B1024_f32", 3072, 768, 0.9, 1024, "f32"),
                                  ("gpt2_W2_s0.9_B1024_f32", 768, 3072, 0.9, 1024, "f32"),
                                  ("square4096_s0.99_B32_bf16", 4096, 4096, 0.99, 32, "bf16"),
                                  ("square4096_s0.99_B1024_bf16", 4096, 4096, 0.99, 1024, "bf16")):
        wl = synth.random_case(29, M, K, synth.nnz_for(M, K, sp), 1, dt, "node")
        w = wl.weights[0]
        sd = snk.F32 if dt == "f32" else snk.BF16
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        log(f"fixed-pattern build {name} ({w.nnz} nnz)")
        t0 = time.time()
        f = snk.snack_fixed_build(w.row, w.col, w.vals, M, K, dtype=sd)
        build_s = time.time() - t0
        X = torch.randn(K * B, device="cuda").to(tdt)
        Y = torch.empty(M * B, dtype=tdt, device="cuda")
        Y2 = torch.empty_like(Y)
        topo = snk.Topology(to_dev(w.row), to_dev(w.col), M, K, B,
                            flags=snk.binding.PLAN_NODE_MAJOR_ONLY)
        vals = to_dev(w.vals, dt == "bf16")
        t = {"fixed": time_calls(lambda: snk.snack_fixed_fwd(f, X, B, 1, Y)),
             "generic": time_calls(lambda: topo.fwd(vals, X, B, snk.NODE_MAJOR, out=Y2))}
        # same products up to the order of the fp32 sums
        err = (Y.float() - Y2.float()).abs().max().item()
        scale = Y2.float().abs().max().item()
        flops = 2 * w.nnz * B
        out[name] = {"nnz": w.nnz, "us": {k: round(v, 2) for k, v in t.items()},
                     "fixed_vs_generic": round(t["generic"] / t["fixed"], 2),
                     "fixed_TFLOPs": round(flops / (t["fixed"] * 1e6), 2),
                     "max_abs_diff_vs_generic": err, "max_abs_generic": scale,
                     "build_seconds": round(build_s, 1), **f.info()}
        f.free()
        del X, Y, Y2, topo, vals
        torch.cuda.empty_cache()
    return out


def snk_drop(nnz, ppm):
    import unstructured_sparse_nn_amd as snk
    return snk.snack_drop_count(nnz, ppm)


def footprint(N, nnz, B, n_drop, layout):
    """Device bytes of the benchmarked layer (sparse, with its plan and
    restructuring workspace) against the same layer dense and Dense+Mask
    (snack_memory_footprint), plus the 90%-sparse fp32 point of the same
    shape without restructuring."""
    import synth
    import unstructured_sparse_nn_amd as snk
    flags = snk.binding.PLAN_NODE_MAJOR_ONLY if layout == "node" else 0
    out = {}
    for key, (nz, dt, b, nd, fl) in {
            "bench_layer": (nnz, snk.BF16, B, n_drop, flags),
            "fp32_90pct_no_restructure": (synth.nnz_for(N, N, 0.9), snk.F32, 1, 0, 0)}.items():
        f = snk.snack_memory_footprint(N, N, nz, b, dt, nd, fl)
        f["sparse_vs_dense"] = round(f["sparse_total"] / f["dense_total"], 4)
        f["sparse_vs_masked"] = round(f["sparse_total"] / f["masked_total"], 4)
        out[key] = f
    return out


def cpu_baseline(w, X, dY, B, drop_ppm, seconds):
    """The fp64 oracle, serial, pinned to one host core (sched_setaffinity),
    running the same step on the same layer: three runs of whole steps
    (~seconds / 3 each), the median step time."""
    import oracle
    import synth
    M, K = w.M, w.K
    x64, g64 = X.f64(), dY.f64()
    n_drop = oracle.drop_count(w.nnz, drop_ppm)
    bytes_step = sum(algo_bytes(op, M, K, w.nnz, B, 2, 2) for op in ("fwd", "bwd_input", "sddmm"))
    T = 512
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    try:
        row, col, vals = w.row.copy(), w.col.copy(), w.vals.copy()
        step_no, runs = 0, []
        for _ in range(3):
            n, t_run = 0, 0.0
            while t_run < seconds / 3 and n < 20:
                v = synth.bf16_bits_to_f32(vals).astype(np.float64)
                t0 = time.perf_counter()
                oracle.spmm_fwd(M, K, row, col, v, B, x64)
                oracle.spmm_bwd_input(M, K, row, col, v, B, g64)
                oracle.sddmm(M, K, row, col, B, g64, x64)
                step_no += 1
                out = oracle.prune_regrow(M, K, row, col, vals, "bf16", n_drop, 0, step_no)
                rp = oracle.row_ptr(M, out["row"])
                cp, _, _ = oracle.csc(K, out["row"], out["col"])
                oracle.partition(rp, T)
                oracle.partition(cp, T)
                t_run += time.perf_counter() - t0
                row, col, vals = out["row"], out["col"], out["vals"]
                n += 1
            runs.append(t_run / n)
    finally:
        os.sched_setaffinity(0, old_aff)
    t_step = float(np.median(runs))
    return {"value": round(bytes_step / t_step / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"median of 3 runs of whole steps (fwd, dX, dV, prune/regrow, row/column "
                      f"views and partitions; {step_no} steps, {sum(runs) / 3 * step_no:.1f} s) "
                      f"of the same {M}x{K} layer, B={B}, fp64 serial C pinned to host core "
                      f"{core} of {os.cpu_count()} ({platform.processor() or platform.machine()}); "
                      f"s/step per run " + ", ".join(f"{r:.3f}" for r in runs)}


def cold_products(w, X, dY, B, ops=("fwd", "bwd_input", "sddmm"), layout="node"):
    """Per-launch time of the products on one bf16 layer, cold: rotate over
    enough device copies that >= 512 MB of each op's data lies between two
    uses of one copy."""
    import torch
    op_bytes = {op: algo_bytes(op.replace("_perm", ""), w.M, w.K, w.nnz, B, 2, 2)
                for op in ops}
    R = rotation_for(min(op_bytes.values()))
    insts = make_instances(w, X, dY, B, R, layout)
    out = {"rotate": R}
    for op in ops:
        us = graph_kernel_us(insts, op)
        b = op_bytes[op]
        out[op] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                   "frac": round(b / us / 1e3 / HBM_PEAK_GBPS, 4)}
    del insts
    torch.cuda.empty_cache()
    return out


def time_ops_grid(sizes, sparsities, batches, tag="sweep"):
    """Cold per-op time (fwd, dX from column-ordered values, dV) of square
    bf16 layers over size x sparsity x batch, node-major."""
    import synth
    out = {}
    for N in sizes:
        for sp in sparsities:
            log(f"{tag} N={N} s={sp}: inputs")
            wl = synth.inference_layer(N=N, sparsity=sp, B=max(batches))
            w = wl.weights[0]
            rng = np.random.default_rng(7)
            for B in batches:
                log(f"{tag} N={N} s={sp} B={B}")
                X = synth.activation(rng, B, N, "bf16")
                dY = synth.activation(rng, B, N, "bf16")
                rec = cold_products(w, X, dY, B)
                rec["algo_bytes"] = algo_bytes("fwd", N, N, w.nnz, B, 2, 2)
                out[f"N{N}_s{sp}_B{B}"] = rec
            del wl, w
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU; --gpus must be 1 "
                          "(the data-parallel split of the batch is described in DESIGN.md)"}))
        sys.exit(2)
    import torch

    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    # all work on one dedicated stream (default priority): the legacy null
    # stream serialises every launch against the whole device
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run_bench(args)


def run_bench(args):
    import torch

    import synth

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n * 4}), flush=True)
        return

    calib = None
    if args.calibrate:
        log("calibration floors")
        calib = calibrate()

    N, B, sp = args.size, args.batch, args.sparsity
    log(f"inputs {N}x{N} s={sp} B={B}")
    w = synth.inference_layer(N=N, sparsity=sp, B=B)
    wt = w.weights[0]
    R = max(1, args.rotate)
    log(f"preparing {R} layer instances")
    insts = [Instance(wt, w.X[0], w.dY[0], B, True, args.drop_ppm, args.layout)
             for _ in range(R)]
    torch.cuda.synchronize()

    fused = args.restructure == "fused"

    def step(i, ev=None):
        inst = insts[i % R]
        inst.products(ev)
        if not args.products_only:
            inst.restructure(ev, fused)

    log("warmup")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K_ = args.steps
    n_ev = 6
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(K_)]
    torch.cuda.synchronize()
    log(f"timing {K_} steps")
    t0 = time.perf_counter()
    for i in range(K_):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) / K_ * 1e3
    # per-op breakdown: the same steps again with events between the calls
    # (kept out of the headline loop, whose host time they would add to)
    log(f"per-op events over {K_} more steps")
    for i in range(K_):
        step(args.warmup + K_ + i, ev[i])
    torch.cuda.synchronize()

    n_ops = 3 if args.products_only else (4 if fused else 5)
    ms = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(n_ops)]
                   for i in range(K_)])
    names = (["fwd", "bwd_input", "sddmm", "restructure"] if fused else
             ["fwd", "bwd_input", "sddmm", "prune_regrow", "prepare"])[:n_ops]
    ops = {}
    prod_bytes = 0
    for j, op in enumerate(names):
        rec = {"us_mean": round(float(ms[:, j].mean()) * 1e3, 2),
               "us_median": round(float(np.median(ms[:, j])) * 1e3, 2)}
        if j < 3:
            b = algo_bytes(op, wt.M, wt.K, wt.nnz, B, 2, 2)
            prod_bytes += b
            rec["algo_bytes"] = b
            rec["GBps"] = round(b / (rec["us_mean"] * 1e3), 1)
        ops[op] = rec
    value = prod_bytes / (ms_per_step * 1e-3) / 1e9
    plan0 = insts[0].topo.plan
    if fused and not args.products_only:
        rb = restructure_bytes(wt.M, wt.K, wt.nnz, 2, plan0.P_row, plan0.P_col)
        us_r = ops["restructure"]["us_median"]
        ops["restructure"].update({
            "algo_bytes": rb, "GBps": round(rb / us_r / 1e3, 1),
            "frac": round(rb / us_r / 1e3 / HBM_PEAK_GBPS, 4),
            "model": "COO read and written back (8 + 2 B per connection each way), plan "
                     "arrays written (offsets, perm, row_t, tiles of both views), "
                     "column-ordered values written; event-timed call, host spin included"})

    # the layer's own training step: forward, fused backward with the SGD
    # update of both copies of the values, restructure (snack_prune_regrow_
    # prepared), over the same rotated instances
    train = None
    if fused and not args.products_only:
        log("training step (fwd, fused backward + SGD, restructure)")

        def tstep(i):
            inst = insts[i % R]
            inst.topo.fwd(inst.vals, inst.X, inst.B, inst.lay, out=inst.Y)
            inst.bwd_fused(lr=1e-3)
            inst.restructure(None, True)

        for i in range(args.warmup):
            tstep(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K_):
            tstep(args.warmup + i)
        torch.cuda.synchronize()
        ms_t = (time.perf_counter() - t0) / K_ * 1e3
        tb = (algo_bytes("fwd", wt.M, wt.K, wt.nnz, B, 2, 2)
              + algo_bytes("bwd_fused", wt.M, wt.K, wt.nnz, B, 2, 2))
        train = {"ms_per_step": round(ms_t, 4), "GBps": round(tb / (ms_t * 1e-3) / 1e9, 2),
                 "algo_bytes": tb,
                 "note": "fwd + snack_spmm_bwd_fused (dX, dV, SGD on vals and vals_t) + "
                         "restructure; bytes of the forward and the fused backward"}
    del insts
    torch.cuda.empty_cache()

    # cold per-launch kernel durations of the products (>= 512 MB rotated),
    # then the same with one instance (warm); the dominant product kernel is
    # the one with the largest cold duration
    log("cold product kernels")
    cold = cold_products(wt, w.X[0], w.dY[0], B,
                         ops=("fwd", "bwd_input", "sddmm", "bwd_input_perm", "bwd_fused"),
                         layout=args.layout)
    for op in ("fwd", "bwd_input", "sddmm"):
        ops[op]["us_kernel"] = cold[op]["us"]
        ops[op]["GBps_kernel"] = cold[op]["GBps"]
        ops[op]["frac_kernel"] = cold[op]["frac"]
    fb = algo_bytes("bwd_fused", wt.M, wt.K, wt.nnz, B, 2, 2)
    ops["bwd_fused"] = {"us_kernel": cold["bwd_fused"]["us"], "algo_bytes": fb,
                        "GBps_kernel": round(fb / (cold["bwd_fused"]["us"] * 1e3), 1),
                        "us_separate": round(cold["bwd_input"]["us"] + cold["sddmm"]["us"], 2),
                        "note": "dX + dV in one call over one index stream (its own minimum "
                                "bytes), column-ordered values; not part of the timed step"}
    ops["bwd_input_perm"] = {"us_kernel": cold["bwd_input_perm"]["us"],
                             "note": "dX reading the values through perm (snack_spmm_bwd_input)"}
    log("warm product kernels")
    warm_inst = make_instances(wt, w.X[0], w.dY[0], B, 1, args.layout)
    ops_warm = {"cache": "warm (one instance repeated)"}
    for op in ("fwd", "bwd_input", "sddmm", "bwd_fused"):
        ops_warm[op] = {"us": round(graph_kernel_us(warm_inst, op), 2)}
    del warm_inst
    torch.cuda.empty_cache()

    dom = max(("fwd", "bwd_input", "sddmm"), key=lambda o: ops[o]["us_kernel"])
    split = plan0.has_split_col if dom == "bwd_input" else plan0.has_split_row
    kname = ({"fwd": "k_wave_spmm (row view)", "bwd_input": "k_wave_spmm (column view, "
              "column-ordered values)", "sddmm": "k_wave_sddmm"} if not split else
             {"fwd": "k_wave_spmm_split (row view)", "bwd_input": "k_wave_spmm_split (column "
              "view)", "sddmm": "k_wave_sddmm_split"})[dom]
    ach = ops[dom]["algo_bytes"] / (ops[dom]["us_kernel"] * 1e-6) / 1e9
    tag = f"{dom}_square{N}_s{sp}_B{B}_bf16"
    traffic = read_traffic(tag, ops[dom]["algo_bytes"])
    roof = {"bound": "hbm", "kernel": kname, "op": dom, "achieved": round(ach, 1),
            "us_per_launch": ops[dom]["us_kernel"],
            "timing": f"HIP events around graph replays, cold ({cold['rotate']} instances "
                      f"rotated, >= 512 MB between reuses)",
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": traffic, "algo_bytes_per_launch": ops[dom]["algo_bytes"]}

    rec = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": K_, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": f"sparse linear {N}x{N}, {sp:.0%} sparse "
                                  f"({wt.nnz} nnz, uniform), bf16 values+activations, fp32 "
                                  f"accumulate, batch {B}; step = fwd+dX+dV"
                      + ("" if args.products_only else
                         f"+prune/regrow {args.drop_ppm / 1e4:g}%+prepare"
                         + (" (one fused call)" if fused else "")),
                      "M": N, "K": N, "nnz": wt.nnz, "batch": B,
                      "layout": "node-major (K x B)" if args.layout == "node" else "batch-major (B x K)",
                      "rotate_instances": R,
                      "cache": "cold (HBM): the step's 20 instances touch ~1.2 GB per rotation"},
           "roofline": roof,
           "ops": ops,
           "ops_warm": ops_warm,
           "products_only_GBps": round(prod_bytes / (sum(ops[o]["us_kernel"] for o in
                                                         ("fwd", "bwd_input", "sddmm"))
                                                     * 1e-6) / 1e9, 1)}
    if train:
        rec["train_step"] = train
    if calib:
        rec["calibration"] = calib
    if args.grid:
        log("grid (cold)")
        grid = time_ops_grid([N], (0.95, 0.99), (1, 8, 32), tag="grid")
        rec["grid"] = grid
        log("dense baselines (cold)")
        sparse_us = {b: grid[f"N{N}_s{sp}_B{b}"]["fwd"]["us"] for b in (1, B)
                     if f"N{N}_s{sp}_B{b}" in grid}
        rec["baselines"] = dense_baselines(wt, w.X[0], (1, B), sparse_us,
                                           (calib or {}).get("stream_read_33.6MB_us"))
    sizes = [int(x) for x in args.sizes.split(",") if x.strip()]
    if sizes:
        rec["sweep"] = time_ops_grid(sizes, (0.95, 0.99), (1, 8, 32))
    if args.graph:
        rec["graph_inference"] = graph_inference()
    if args.configs:
        rec["configs"] = other_configs()
    if args.conv:
        log("1x1 convolution")
        rec["conv1x1"] = conv1x1_bench()
    if args.fixed_full:
        rec["fixed_full"] = fixed_full_bench()
    rec["footprint"] = footprint(N, wt.nnz, B, 0 if args.products_only else
                                 snk_drop(wt.nnz, args.drop_ppm), args.layout)
    if args.cpu_baseline:
        log("cpu baseline (oracle, one pinned core)")
        rec["cpu_baseline"] = cpu_baseline(wt, w.X[0], w.dY[0], B, args.drop_ppm,
                                           args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
