"""GPU parity of the stack's two ends ("Final RMSNorm", the model driver): the
entry, whose embedding is copied into the 4 streams (HC_BOUNDARY_X_EXPANDED:
the calls read the [n, d] row for every stream), and the MTP head's tap, the
mean over the streams of a block's input (x_mean_out of the boundary that
writes those streams).  The exit (final write, read with the last pre,
RMSNorm with eps 1e-20) is covered by the stack tests.  Against the oracle on
the decode and the two-launch paths, and a stack fed through the expanded
entry bit for bit against the same stack on materialised streams."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests import numerics as N
from tests.gpu_util import (assert_bf16_close, assert_bits_equal, assert_coef_close, assert_mixes_close, bf16_dev,
                            f32_dev, host_bits, host_f32, say, write_floor)
from tests.test_gpu_parity import _check_boundary
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu


def _case(n, fresh, norm, with_delta, want_mean, d=5120):
    s = synth.boundary_inputs("prefill", 0, n, d)
    h = s["x"][:, 0]                                     # an embedding row per token
    pre = np.full((n, 4), 0.25, np.float32)
    kw = dict(x=h, x_expanded=True, want_mean=want_mean, pre_in=None if fresh else pre,
              gamma=s["gamma"] if norm else None, hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"])
    if with_delta:
        kw.update(delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"])
    ref = O.boundary(**kw)
    dev = dict(fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"])), hc_base=f32_dev(s["hc_base"]),
               hc_scale=f32_dev(s["hc_scale"]), pre_in=None if fresh else f32_dev(pre),
               gamma=f32_dev(s["gamma"]) if norm else None)
    if with_delta:
        dev.update(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]))
    got = H.hc_boundary(bf16_dev(h), x_expanded=True, want_mean=want_mean, want_mixes=True, **dev)
    return ref, got, dict(s, x=O.expand_streams(h))


@pytest.mark.parametrize("n", [40, 300])                # few-tile exchange (given pre) / two launches (fresh)
@pytest.mark.parametrize("fresh,norm", [(False, False), (False, True), (True, True)])
@pytest.mark.parametrize("with_delta", [False, True])
def test_expanded_streams(n, fresh, norm, with_delta):
    say(f"[expanded x] n={n} fresh={fresh} norm={norm} delta={with_delta}")
    ref, got, s = _case(n, fresh, norm, with_delta, want_mean=True)
    _check_boundary(ref, got, s, fresh, norm)
    # the tap: the mean over the new streams (one fp32 rounding of the 4-term sum at most)
    assert_bf16_close(host_bits(got["x_mean"]), ref["x_mean"], "x_mean")
    if not with_delta:
        assert_bits_equal(host_bits(got["x_mean"]), s["x"][:, 0], "x_mean of the copies is the embedding")


@pytest.mark.parametrize("n", [100, 300])
def test_stream_mean_of_written_streams(n):
    """x_mean_out of an ordinary boundary (decode / two-launch) and of the exit
    call equals the mean over the written streams."""
    s = synth.boundary_inputs("prefill", 0, n)
    X = bf16_dev(s["x"])
    base = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
                pre_in=f32_dev(s["pre_in"]))
    say(f"[x_mean] boundary n={n}")
    got = H.hc_boundary(X, fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"])), hc_base=f32_dev(s["hc_base"]),
                        hc_scale=f32_dev(s["hc_scale"]), want_mean=True, **base)
    assert_bf16_close(host_bits(got["x_mean"]), O.stream_mean(host_bits(got["x_out"])), "x_mean (boundary)")
    say(f"[x_mean] exit n={n}")
    ex = H.hc_boundary(X, gamma=f32_dev(s["gamma"]), rms_eps=1e-20, want_mean=True, **base)
    assert_bf16_close(host_bits(ex["x_mean"]), O.stream_mean(host_bits(ex["x_out"])), "x_mean (exit)")


def test_stack_through_expanded_entry_matches_materialised():
    """Three sublayers of the stand-in stack (n=512): fed through the expanded
    entry and first boundary, every output equals, bit for bit, the same calls
    on the materialised 4 streams."""
    n_sub, n = 3, 512
    st = synth.stack_inputs(n_sub, 0, n)
    h = bf16_dev(st["h"])
    X = h.view(n, 1, -1).expand(n, 4, h.shape[-1]).contiguous()
    packed = [H.hc_fn_pack(f32_dev(p[0])) for p in st["params"]]

    def run(expanded):
        x = h if expanded else X
        pre = torch.full((n, 4), 0.25, dtype=torch.float32, device=h.device)
        delta = post = comb = None
        outs = []
        for dep in range(n_sub):
            fn, b, sc = st["params"][dep]
            kw = dict(pre_in=pre, fn_packed=packed[dep], hc_base=f32_dev(b), hc_scale=f32_dev(sc),
                      gamma=f32_dev(st["gammas"][dep]), want_mixes=True, want_mean=True,
                      x_expanded=expanded and dep <= 1)
            if dep > 0:
                kw.update(delta=delta, post_in=post, comb_in=comb)
            o = H.hc_boundary(x, **kw)
            if dep > 0:
                x = o["x_out"]
            delta, post, comb, pre = o["y"], o["post"], o["comb"], o["pre"]
            outs.append({k: o[k].clone() for k in ("y", "mixes", "pre", "post", "comb", "x_mean")
                         if o.get(k) is not None})
        return outs

    say("[stack ends] expanded vs materialised, 3 sublayers, n=512")
    a, b = run(True), run(False)
    for dep in range(n_sub):
        for k in a[dep]:
            assert torch.equal(a[dep][k], b[dep][k]), f"sublayer {dep}: {k} differs"
