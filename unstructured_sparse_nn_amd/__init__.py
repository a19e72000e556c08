"""Truly sparse linear layer for AMD Instinct MI355X (gfx950).

The weight is kept only as its nonzeros (COO); the forward product, the input
gradient, the value gradient and the prune/regrow step all run in the HIP
library ``libsnack.so`` (C ABI in ``include/snack.h``).  ``binding`` mirrors
that ABI one function per entry point; ``layer`` wraps it as a torch module.
PyTorch only provides device memory and streams.
"""
from .binding import (ACT_GELU, ACT_NONE, ACT_RELU, BATCH_MAJOR, BF16, CONV_NCHW,  # noqa: F401
                      CONV_NHWC, F32, FIXED_COMPILE_ONLY, NODE_MAJOR, SnackError, SnackFixed,
                      SnackPlan, snack_conv1x1, snack_fixed_build, snack_fixed_fwd,
                      snack_coo_prepare, snack_dense_fwd, snack_graph_propagate, snack_drop_count, snack_gelu_bwd,
                      snack_gelu_fwd, snack_memory_footprint, snack_plan_array, snack_plan_init, snack_plan_sizeof,
                      snack_prune_regrow, snack_prune_regrow_prepared, snack_prune_regrow_static,
                      snack_prune_regrow_workspace, snack_sddmm_grad_vals, snack_gather_vals_t,
                      snack_spmm_bwd_input_t,
                      snack_spmm_bwd_fused, snack_spmm_bwd_fused_adam, snack_spmm_bwd_input,
                      snack_spmm_fwd,
                      snack_spmm_fwd_act, snack_version, snack_calibrate,
                      status_str)
from .layer import SparseLinear, Topology  # noqa: F401
