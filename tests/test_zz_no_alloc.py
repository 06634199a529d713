"""hc_boundary_static (the entry point that allocates nothing: the library's
static device workspace) against hc_boundary with a caller workspace, through
the C ABI: the same kernels in the same order, so every output must match to
the bit.  Three calls in a row on the shared static workspace, each smaller
than the one before and on another schedule: the one-launch given-pre
boundary with the RMSNorm (n = 4096), the two launches with a fresh read
(n = 300), the few-tile exchange (n = 64); then the first call again."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import bf16_dev, f32_dev, host_bits, host_f32, say
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu

KEYS = ("x_out", "y", "pre", "post", "comb", "mixes")


def _dev(n, fresh, norm):
    s = synth.boundary_inputs("prefill", 0, n)
    d = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
             pre_in=None if fresh else f32_dev(s["pre_in"]), fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"])),
             hc_base=f32_dev(s["hc_base"]), hc_scale=f32_dev(s["hc_scale"]),
             gamma=f32_dev(s["gamma"]) if norm else None)
    return bf16_dev(s["x"]), d


def _same(a, b, what):
    for k in KEYS:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            assert np.array_equal(host_bits(x), host_bits(y)), f"{what}: {k}"
        else:
            assert np.array_equal(host_f32(x), host_f32(y)), f"{what}: {k}"


def test_static_workspace_matches_caller_workspace():
    cases = [(4096, False, True), (300, True, True), (64, False, False), (4096, False, True)]
    for n, fresh, norm in cases:
        say(f"[static workspace] n={n} fresh={fresh} norm={norm}")
        x, d = _dev(n, fresh, norm)
        got = H.hc_boundary_static(x, **d, want_mixes=True)
        ref = H.hc_boundary(x, **d, want_mixes=True)
        torch.cuda.synchronize()
        assert "workspace" not in got
        _same(got, ref, f"n={n}")


def test_static_workspace_rejects_shapes_beyond_it():
    say("[static workspace] shapes beyond 16 MiB")
    L = H.lib()
    need = L.hc_workspace_bytes(4096, 8, 5120)
    assert need > 16 << 20
    a = H.BoundaryArgs()
    a.struct_size = ctypes.sizeof(H.BoundaryArgs)
    a.hc, a.d, a.iters, a.n = 8, 5120, 20, 4096
    a.hc_eps = a.norm_eps = a.rms_eps = 1e-6
    P = 0x10000
    a.x, a.y_out, a.fn_packed, a.hc_base, a.hc_scale = P, P + (1 << 30), P + (2 << 30), P + (3 << 30), P + (3 << 30) + 4096
    a.pre_in, a.pre_out, a.post_out, a.comb_out = P + (3 << 30) + 8192, P + (4 << 30), P + (5 << 30), P + (6 << 30)
    assert L.hc_boundary_static(ctypes.byref(a), None) == H.HC_ENOTSUP
    assert b"static workspace" in L.hc_last_error()
