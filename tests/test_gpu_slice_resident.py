"""GPU parity of the slice-resident boundary schedule (HC_BOUNDARY_SLICE_RESIDENT:
one launch, one workgroup per compute unit, each keeping a 160-feature slice
of the packed weights in LDS, the new streams of its last tiles in registers,
and the per-token sums exchanged between the 32 slices of a tile through the
workspace).  Every output against the CPU oracle at the standard bars; token
counts that leave ragged tiles and XCDs with one tile more than others; calls
repeated on one workspace (the exchange tags advance per call); the full
prefill size on sampled tokens."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests.gpu_util import assert_workspace_clean, bf16_dev, f32_dev, host_bits, host_f32, say
from tests.test_gpu_parity import SAMPLE_RANGES, _check_boundary, packed
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(t0, t1, workload="prefill"):
    s = synth.boundary_inputs(workload, t0, t1)
    dev = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
               fn_packed=packed(s["hc_fn"]), hc_base=f32_dev(s["hc_base"]), hc_scale=f32_dev(s["hc_scale"]))
    return s, bf16_dev(s["x"]), dev


def _oracle(s, a, b, norm):
    return O.boundary(x=s["x"][a:b], delta=s["delta"][a:b], post_in=s["post_in"][a:b], comb_in=s["comb_in"][a:b],
                      pre_in=None, hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"],
                      gamma=s["gamma"] if norm else None)


# n = 1: one tile on one XCD; 40: three tiles; 300: 19 tiles (XCDs with 2 and 3,
# the last ragged); 1000: 63 tiles, 7 or 8 per XCD (past the 6-interval unroll)
@pytest.mark.parametrize("n", [1, 40, 300, 1000])
@pytest.mark.parametrize("norm", [True, False])
def test_slice_resident_vs_oracle(n, norm):
    say(f"[slice-resident] n={n} norm={norm}")
    s, X, dev = _inputs(0, n)
    got = H.hc_boundary(X, **dev, gamma=f32_dev(s["gamma"]) if norm else None, want_mixes=True,
                        slice_resident=True)
    torch.cuda.synchronize()
    assert_workspace_clean(got)
    ref = _oracle(s, 0, n, norm)
    _check_boundary(ref, got, {"x": s["x"], "gamma": s["gamma"]}, True, norm)


def test_slice_resident_repeated_calls_and_default_schedule():
    """Five calls on one workspace give the same bits each time with no wait
    timed out; X' is bit-identical to the default schedule's, the rest within
    the parity bars (the projection is summed over other feature slices)."""
    n = 500
    say(f"[slice-resident] 5 calls on one workspace, n={n}")
    s, X, dev = _inputs(0, n)
    dev["gamma"] = f32_dev(s["gamma"])
    base = H.hc_boundary(X, **dev, want_mixes=True)
    ws = torch.zeros(H.lib().hc_workspace_bytes(n, 4, 5120), dtype=torch.uint8, device=X.device)
    first = None
    for rep in range(5):
        got = H.hc_boundary(X, **dev, want_mixes=True, slice_resident=True, out={"workspace": ws})
        torch.cuda.synchronize()
        assert_workspace_clean(got)
        cur = {k: host_bits(got[k]) if got[k].dtype == torch.bfloat16 else host_f32(got[k])
               for k in ("x_out", "y", "pre", "post", "comb", "mixes")}
        if first is None:
            first = cur
        else:
            for k in cur:
                assert np.array_equal(cur[k], first[k]), f"call {rep}: {k} differs from call 0"
    assert np.array_equal(first["x_out"], host_bits(base["x_out"]))
    for k in ("pre", "post", "comb"):
        assert np.abs(first[k].astype(np.float64) - host_f32(base[k])).max() <= 2e-5, k


def test_slice_resident_between_other_schedules():
    """The slice-resident ring has its own place in the workspace: calls of the
    default and single-launch schedules in between leave it working."""
    n = 200
    say(f"[slice-resident] interleaved with the other schedules, n={n}")
    s, X, dev = _inputs(0, n)
    dev["gamma"] = f32_dev(s["gamma"])
    ws = torch.zeros(H.lib().hc_workspace_bytes(n, 4, 5120), dtype=torch.uint8, device=X.device)
    ref = _oracle(s, 0, n, True)
    for sched in ("slice", "default", "single", "slice", "slice"):
        kw = {"slice_resident": sched == "slice", "single_launch": sched == "single"}
        got = H.hc_boundary(X, **dev, want_mixes=True, out={"workspace": ws}, **kw)
        torch.cuda.synchronize()
        assert_workspace_clean(got)
        if sched == "slice":
            _check_boundary(ref, got, {"x": s["x"], "gamma": s["gamma"]}, True, True)


def test_slice_resident_prefill_full_size_sampled():
    say("[slice-resident n=4096] generating inputs")
    s, X, dev = _inputs(0, 4096)
    dev["gamma"] = f32_dev(s["gamma"])
    say("  launching")
    got = H.hc_boundary(X, **dev, want_mixes=True, slice_resident=True)
    torch.cuda.synchronize()
    assert_workspace_clean(got)
    for a, b in SAMPLE_RANGES + [(1000, 1003), (3071, 3073)]:
        say(f"  oracle tokens {a}..{b}")
        sub = {k: (v[a:b] if v is not None else None) for k, v in got.items() if k != "workspace"}
        _check_boundary(_oracle(s, a, b, True), sub, {"x": s["x"][a:b], "gamma": s["gamma"]}, True, True)
