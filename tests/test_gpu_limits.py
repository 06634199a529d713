"""GPU parity at the library's size limits (hc = 4): the widest rows
(d = 32768, and d = 10240 with the RMSNorm) on every schedule that takes
them, ragged token counts, and the full-size boundary at hc = 8 (the bench's
other-hc configuration) on sampled tokens."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests.gpu_util import assert_bits_equal, bf16_dev, f32_dev, host_bits, say
from tests.test_gpu_parity import _boundary_case, _check_boundary
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [5, 70])
def test_streams_widest_rows(n):
    say(f"[limits] hc_post / hc_pre n={n} d=32768")
    s = synth.boundary_inputs("prefill", 0, n, 32768)
    X = bf16_dev(s["x"])
    xo = H.hc_post(bf16_dev(s["delta"]), X, f32_dev(s["post_in"]), f32_dev(s["comb_in"]))
    assert_bits_equal(host_bits(xo), O.hc_post(s["delta"], s["x"], s["post_in"], s["comb_in"]), "hc_post")
    y = H.hc_pre(X, f32_dev(s["pre_in"]))
    assert_bits_equal(host_bits(y), O.hc_pre(s["x"], s["pre_in"]), "hc_pre")


# (n, d, fresh, norm): d = 32768 on the two launches (the few-tile exchange
# takes d up to 8192, so a given pre falls back to them too); d = 10240 with the
# RMSNorm on the two launches; d = 8192 on the few-tile exchange
CASES = [(20, 32768, True, False), (20, 32768, False, False), (130, 32768, False, False),
         (70, 10240, True, True), (9, 10240, False, True), (20, 8192, False, False)]


@pytest.mark.parametrize("n,d,fresh,norm", CASES)
def test_boundary_widest_rows(n, d, fresh, norm):
    say(f"[limits] boundary n={n} d={d} fresh={fresh} norm={norm}")
    ref, got, s = _boundary_case("prefill", 0, n, fresh, norm, d=d)
    _check_boundary(ref, got, s, fresh, norm)


def test_hc8_full_size_every_token():
    """The boundary at hc = 8 in the bench's configuration (n = 4096, d = 5120,
    write, fresh pre, RMSNorm) against the oracle on every token."""
    say("[limits] hc=8 n=4096: generating inputs")
    s = synth.boundary_inputs("prefill", hc=8)
    dev = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
               fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=8), hc_base=f32_dev(s["hc_base"]),
               hc_scale=f32_dev(s["hc_scale"]), gamma=f32_dev(s["gamma"]))
    say("  launching")
    got = H.hc_boundary(bf16_dev(s["x"]), **dev, want_mixes=True)
    torch.cuda.synchronize()
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else None) for k, v in got.items() if k != "workspace"}
    assert host["y"].shape == (4096, 5120)
    for a in range(0, 4096, 512):
        b = a + 512
        say(f"  oracle tokens {a}..{b}")
        ref = O.boundary(x=s["x"][a:b], delta=s["delta"][a:b], post_in=s["post_in"][a:b],
                         comb_in=s["comb_in"][a:b], hc_fn=s["hc_fn"], hc_base=s["hc_base"],
                         hc_scale=s["hc_scale"], gamma=s["gamma"])
        sub = {k: (v[a:b] if v is not None else None) for k, v in host.items()}
        _check_boundary(ref, sub, {"x": s["x"][a:b], "gamma": s["gamma"]}, True, True)
