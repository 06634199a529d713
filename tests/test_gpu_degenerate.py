"""GPU parity on the degenerate cases of the method, every stream count and
schedule: all-zero streams (the RMS statistic is then eps-dominated and the
mixes vanish, so pre/post/comb come from the offsets alone), saturated gates
(offsets large enough that the sigmoids sit at 0 or 1 and the softmax rows
are close to one-hot), a single Sinkhorn round, and token independence (a NaN in one
token's streams leaves every other token's outputs bit for bit unchanged)."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests.gpu_util import assert_bits_equal, assert_coef_close, bf16_dev, f32_dev, host_bits, host_f32, say
from tests.test_gpu_parity import _check_boundary
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu

# (hc, n, d): hc = 4 at n = 40 and 300 runs the few-tile exchange with a given
# pre and the two launches otherwise
SHAPES = [(4, 40, 1024), (4, 300, 1024), (2, 40, 1024), (8, 40, 1024)]


def _dev(s, fresh, norm, hc):
    d = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
             fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=hc), hc_base=f32_dev(s["hc_base"]),
             hc_scale=f32_dev(s["hc_scale"]))
    if not fresh:
        d["pre_in"] = f32_dev(s["pre_in"])
    if norm:
        d["gamma"] = f32_dev(s["gamma"])
    return d


def _ref(s, fresh, norm, iters=20):
    return O.boundary(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"],
                      pre_in=None if fresh else s["pre_in"], hc_fn=s["hc_fn"], hc_base=s["hc_base"],
                      hc_scale=s["hc_scale"], gamma=s["gamma"] if norm else None, iters=iters)


@pytest.mark.parametrize("hc,n,d", SHAPES)
@pytest.mark.parametrize("fresh,norm", [(False, False), (True, True)])
def test_zero_streams(hc, n, d, fresh, norm):
    say(f"[degenerate] zero streams hc={hc} n={n} d={d} fresh={fresh} norm={norm}")
    s = synth.boundary_inputs("prefill", 0, n, d, hc=hc)
    s["x"] = np.zeros_like(s["x"])
    s["delta"] = np.zeros_like(s["delta"])
    ref = _ref(s, fresh, norm)
    got = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, **_dev(s, fresh, norm, hc))
    # the mixes are exactly zero on both sides (the floored relative error is 0/0 here)
    assert not ref["mixes"].any() and not host_f32(got["mixes"]).any(), "mixes of zero streams"
    for k in ("pre", "post", "comb"):
        assert_coef_close(host_f32(got[k]), ref[k], k)
    assert_bits_equal(host_bits(got["x_out"]), ref["x_out"], "x_out")
    assert_bits_equal(host_bits(got["y"]), ref["y"], "y")


@pytest.mark.parametrize("hc,n,d", SHAPES)
def test_saturated_gates(hc, n, d):
    """Offsets of +-50 drive the sigmoids into saturation (pre at eps or 1+eps,
    post at 0 or 2 in fp32) and the softmax rows close to one-hot, without
    amplifying the mixes' rounding (the scales stay as drawn)."""
    say(f"[degenerate] saturated gates hc={hc} n={n} d={d}")
    s = synth.boundary_inputs("prefill", 0, n, d, hc=hc)
    sign = np.where(np.random.default_rng(5).random(s["hc_base"].shape) < 0.5, -1.0, 1.0)
    s["hc_base"] = (50.0 * sign).astype(np.float32)
    for fresh, norm in ((False, False), (True, True)):
        ref = _ref(s, fresh, norm)
        got = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, **_dev(s, fresh, norm, hc))
        _check_boundary(ref, got, s, fresh, norm)
        post = host_f32(got["post"])
        assert ((post == 2.0) | (post < 1e-6)).mean() > 0.95, "post not saturated"


@pytest.mark.parametrize("hc,n,d", SHAPES)
def test_single_sinkhorn_round(hc, n, d):
    """iters = 1: the softmax rows, then one column normalisation."""
    say(f"[degenerate] iters=1 hc={hc} n={n} d={d}")
    s = synth.boundary_inputs("prefill", 0, n, d, hc=hc)
    ref = _ref(s, False, False, iters=1)
    got = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, iters=1, **_dev(s, False, False, hc))
    _check_boundary(ref, got, s, False, False)
    # the last step is a column normalisation: the column sums (S/(S + eps) of the
    # sums S before it) agree with the oracle's to the entries' tolerance
    cs = host_f32(got["comb"]).astype(np.float64).sum(axis=1)
    assert np.abs(cs - ref["comb"].sum(axis=1)).max() < hc * 1e-5


@pytest.mark.parametrize("hc,n,d", SHAPES)
@pytest.mark.parametrize("fresh,norm", [(False, False), (True, True)])
def test_token_independence(hc, n, d, fresh, norm):
    """A NaN in one token's streams stays in that token."""
    say(f"[degenerate] NaN isolation hc={hc} n={n} d={d} fresh={fresh} norm={norm}")
    s = synth.boundary_inputs("prefill", 0, n, d, hc=hc)
    dev = _dev(s, fresh, norm, hc)
    clean = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, **dev)
    torch.cuda.synchronize()
    clean = {k: v.clone() for k, v in clean.items() if isinstance(v, torch.Tensor) and k != "workspace"}
    bad = s["x"].copy()
    bad[3, 0, 17] = 0x7FC0                                       # a quiet NaN
    got = H.hc_boundary(bf16_dev(bad), want_mixes=True, **dev)
    torch.cuda.synchronize()
    keep = np.ones(n, bool)
    keep[3] = False
    for k, v in clean.items():
        g = got[k]
        a = host_bits(g) if g.dtype == torch.bfloat16 else host_f32(g).view(np.uint32)
        b = host_bits(v) if v.dtype == torch.bfloat16 else host_f32(v).view(np.uint32)
        assert_bits_equal(a[keep], b[keep], f"{k} of the other tokens")
    assert np.isnan(host_f32(got["mixes"])[3]).any(), "the NaN token's mixes"
