"""Hyper-Connections residual glue for AMD Instinct MI355X (gfx950).

The compute lives in libhc.so (hand-written HIP kernels behind the C ABI of
include/hc.h); ``hc`` is its Python binding and ``synth`` the seeded
synthetic-input generator of the benchmark workloads.
"""
from .hc import (BoundaryCall, HCError, hc_boundary, hc_fn_pack, hc_mixes, hc_post, hc_pre,  # noqa: F401
                 hc_split_sinkhorn, lib)

__all__ = ["BoundaryCall", "HCError", "hc_boundary", "hc_fn_pack", "hc_mixes", "hc_post", "hc_pre",
           "hc_split_sinkhorn", "lib"]
