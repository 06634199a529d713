"""GPU parity of hc_boundary (hc = 4) on seeded random shapes and forms,
against the oracle on every token: token counts from 1 to 9000 and widths
from 64 to 10240, so that every schedule the call can pick (the decode
schedule, the one-launch read-row exchange with either slice width, the two
launches, consecutive 4096-token parts) and every edge of its choice is hit
with ragged tiles; each case also with the block-entry form, the expanded
embedding, the stream mean and the two-launch flag drawn at random."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests.gpu_util import assert_bits_equal, bf16_dev, f32_dev, host_bits, say
from tests.test_gpu_parity import _check_boundary, packed
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu

# token counts around the schedules' edges, then random ones
_EDGE_N = [1, 63, 128, 129, 1215, 1300, 2047, 2049, 4095, 4097, 8193]
_WIDTHS = [64, 320, 1024, 2560, 5120, 7168, 10240]


# fixed cases for the schedule combinations a random draw may miss: the
# expanded entry in one launch (stream-summed weight) and in consecutive parts,
# the exchange with 10-chunk slices at d = 2560 (4 slices), and a given-pre
# decode call with the RMSNorm and the stream mean
_FIXED = [(4096, 5120, False, True, True, True, True, False), (8200, 5120, False, True, True, True, False, False),
          (2000, 2560, False, True, False, False, False, False), (100, 5120, False, True, False, False, True, False)]


def _cases(count=24, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = [(100 + i, *c) for i, c in enumerate(_FIXED)]
    for i in range(count):
        n = int(_EDGE_N[i]) if i < len(_EDGE_N) else int(rng.integers(1, 9001))
        d = int(rng.choice(_WIDTHS)) if n <= 4096 else 5120
        fresh = bool(rng.integers(2))
        norm = bool(rng.integers(4) > 0)
        entry = bool(rng.integers(4) == 0)
        expanded = entry and bool(rng.integers(2))
        mean = bool(rng.integers(3) == 0)
        two = bool(rng.integers(5) == 0)
        cases.append((i, n, d, fresh, norm, entry, expanded, mean, two))
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "c%d-n%d-d%d" % c[:3])
def test_random_boundary(case):
    i, n, d, fresh, norm, entry, expanded, mean, two = case
    say(f"[random {i}] n={n} d={d} fresh={fresh} norm={norm} entry={entry} expanded={expanded} mean={mean} "
        f"two={two}")
    s = synth.boundary_inputs("stress" if i % 3 == 0 else "prefill", 0, n, d)
    x = s["x"][:, 0] if expanded else s["x"]
    kw = dict(x=x, pre_in=None if fresh else s["pre_in"], gamma=s["gamma"] if norm else None, hc_fn=s["hc_fn"],
              hc_base=s["hc_base"], hc_scale=s["hc_scale"])
    if not entry:
        kw.update(delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"])
    dev = {k: (bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)) for k, v in kw.items()
           if v is not None and k != "hc_fn"}
    dev["fn_packed"] = packed(kw["hc_fn"])
    X = dev.pop("x")
    got = H.hc_boundary(X, **dev, want_mixes=True, want_mean=mean, two_launch=two, x_expanded=expanded)
    torch.cuda.synchronize()
    ref = O.boundary(**kw, x_expanded=expanded, want_mean=mean)
    streams = O.expand_streams(x) if expanded else s["x"]
    _check_boundary(ref, got, {"x": streams, "gamma": s["gamma"]}, fresh, norm)
    if mean:
        assert_bits_equal(host_bits(got["x_mean"]), ref["x_mean"], "stream mean")


def _entry_cases(count=20, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        hc = int(rng.choice([2, 4, 8]))
        n = int(rng.integers(1, 5001))
        d = int(rng.choice([64, 320, 1024, 5120] if hc != 8 else [64, 320, 1024, 2048]))
        out.append((i, hc, n, d, str(rng.choice(["mixes", "pre", "post", "boundary", "static"]))))
    return out


@pytest.mark.parametrize("case", _entry_cases(), ids=lambda c: "e%d-hc%d-n%d-d%d-%s" % c)
def test_random_entry_points(case):
    """The standalone entry points, the boundary at hc = 2 and 8, and the
    boundary on the library's static workspace, on seeded random shapes."""
    i, hc, n, d, what = case
    say(f"[random entry {i}] hc={hc} n={n} d={d} {what}")
    from tests.gpu_util import assert_coef_close, assert_mixes_close, host_f32
    s = synth.boundary_inputs("prefill", 0, n, d, hc=hc)
    X = bf16_dev(s["x"])
    if what == "mixes":
        fn = H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=hc)
        pre, post, comb, mixes = H.hc_mixes(X, fn, f32_dev(s["hc_scale"]), f32_dev(s["hc_base"]), return_mixes=True)
        rm = O.hc_mixes(s["x"], s["hc_fn"], 1e-6)
        assert_mixes_close(host_f32(mixes), rm)
        rp, rq, rc = O.hc_split_sinkhorn(rm, s["hc_scale"], s["hc_base"], hc)
        assert_coef_close(host_f32(pre), rp, "pre")
        assert_coef_close(host_f32(post), rq, "post")
        assert_coef_close(host_f32(comb), rc, "comb")
    elif what == "pre":
        assert_bits_equal(host_bits(H.hc_pre(X, f32_dev(s["pre_in"]))), O.hc_pre(s["x"], s["pre_in"]), "hc_pre")
    elif what == "post":
        got = H.hc_post(bf16_dev(s["delta"]), X, f32_dev(s["post_in"]), f32_dev(s["comb_in"]))
        assert_bits_equal(host_bits(got), O.hc_post(s["delta"], s["x"], s["post_in"], s["comb_in"]), "hc_post")
    else:
        kw = dict(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"], pre_in=s["pre_in"],
                  hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"], gamma=s["gamma"])
        dev = {k: (bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)) for k, v in kw.items() if k not in ("x",
                                                                                                         "hc_fn")}
        dev["fn_packed"] = H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=hc)
        if what == "static" and hc == 4 and H.lib().hc_boundary_workspace_bytes(n, hc, d) <= 16 << 20:
            got = H.hc_boundary_static(X, **dev, want_mixes=True)
        else:
            got = H.hc_boundary(X, **dev, want_mixes=True)
        torch.cuda.synchronize()
        ref = O.boundary(**kw, hc=hc)
        _check_boundary(ref, got, {"x": s["x"], "gamma": s["gamma"]}, False, True)
