"""GPU parity of the address-order sweeps, the stream-only calls ("Write the
streams"; "Source layer, pairs pooled": Block.hc_pre, Block.hc_post; "Final
RMSNorm"), at widths that give every shape of their work split: one partial
512-feature chunk (d = 64, 320), several chunks with a partial last one
(d = 1088), one chunk per wave (d = 5120: ten waves), two chunks for some
waves (d = 7168, 10240), and token counts from 1 up.  hc_post and hc_pre are
bit-exact; the exit (write, read, RMSNorm), the read with the RMSNorm, and
the stream mean (the MTP tap) of the exit are checked against the oracle."""
import pytest

from oracle import hc_oracle as O
from tests.gpu_util import assert_bf16_close, assert_bits_equal, bf16_dev, f32_dev, host_bits, say
from tests.test_gpu_parity import _boundary_case, _check_boundary
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu

WIDTHS = [64, 320, 1088, 5120, 7168, 10240]


@pytest.mark.parametrize("d", WIDTHS)
@pytest.mark.parametrize("n", [1, 37, 300])
def test_post_and_pre(n, d):
    say(f"[sweep] hc_post / hc_pre n={n} d={d}")
    s = synth.boundary_inputs("prefill", 0, n, d)
    got = H.hc_post(bf16_dev(s["delta"]), bf16_dev(s["x"]), f32_dev(s["post_in"]), f32_dev(s["comb_in"]))
    assert_bits_equal(host_bits(got), O.hc_post(s["delta"], s["x"], s["post_in"], s["comb_in"]), "hc_post")
    got = H.hc_pre(bf16_dev(s["x"]), f32_dev(s["pre_in"]))
    assert_bits_equal(host_bits(got), O.hc_pre(s["x"], s["pre_in"]), "hc_pre")


@pytest.mark.parametrize("d", WIDTHS)
@pytest.mark.parametrize("n", [1, 37])
def test_exit(n, d):
    """The exit: the last write, the read with the last pre, its RMSNorm."""
    say(f"[sweep] exit n={n} d={d}")
    ref, got, s = _boundary_case("prefill", 0, n, False, True, exit_=True, d=d)
    _check_boundary(ref, got, s, False, True)


@pytest.mark.parametrize("d", WIDTHS)
def test_read_with_norm(d):
    """A read of given streams with a given pre and the RMSNorm (no write, no mixes)."""
    say(f"[sweep] read with the RMSNorm n=45 d={d}")
    ref, got, s = _boundary_case("stress", 0, 45, False, True, entry=True, exit_=True, d=d)
    _check_boundary(ref, got, s, False, True)


@pytest.mark.parametrize("d", [320, 7168])
def test_exit_stream_mean(d):
    """The exit's stream mean (the MTP tap) equals the mean over the written streams."""
    say(f"[sweep] exit with the tap n=29 d={d}")
    s = synth.boundary_inputs("prefill", 0, 29, d)
    ex = H.hc_boundary(bf16_dev(s["x"]), delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]),
                       comb_in=f32_dev(s["comb_in"]), pre_in=f32_dev(s["pre_in"]), gamma=f32_dev(s["gamma"]),
                       rms_eps=1e-20, want_mean=True)
    assert_bits_equal(host_bits(ex["x_out"]), O.hc_post(s["delta"], s["x"], s["post_in"], s["comb_in"]), "x_out")
    assert_bf16_close(host_bits(ex["x_mean"]), O.stream_mean(host_bits(ex["x_out"])), "x_mean (exit)")
