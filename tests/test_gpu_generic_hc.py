"""GPU parity for hc = 2 and hc = 8 streams (the pages fix hc = 4; the
Block code is written for any hc, and the projection, split and Sinkhorn
definitions carry over unchanged).  Every entry point, through the C ABI,
against the oracle on the same seeded inputs: hc_pre / hc_post bit for bit;
mixes floored relative error <= 1e-4; pre/post/comb absolute error <= 1e-5;
the boundary in all its forms (entry, write, fresh or given pre, RMSNorm,
stream mean, expanded entry, exit, the two halves)."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests import numerics as N
from tests.gpu_util import (assert_bf16_close, assert_bits_equal, assert_coef_close, assert_mixes_close, bf16_dev,
                            f32_dev, host_bits, host_f32, say)
from tests.test_gpu_parity import _check_boundary
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu

HCS = [2, 8]


def _inputs(hc, n, d, t0=0):
    return synth.boundary_inputs("prefill", t0, t0 + n, d, hc=hc)


def _dev_params(s):
    return dict(fn_packed=H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=s["x"].shape[1]), hc_base=f32_dev(s["hc_base"]),
                hc_scale=f32_dev(s["hc_scale"]))


@pytest.mark.parametrize("hc", HCS)
def test_packed_weight_terms(hc):
    """Packed column q = 16*tile + lane%16 of a 32-feature step holds term
    q // mixp (hi, mid, lo) of row q % mixp at features 8*(lane//16)..+7:
    hi is the nearest bf16 of the weight, hi + mid + lo the weight itself
    (normal values), and the padding rows are zero."""
    say(f"[hc={hc}] pack d=1024")
    d = 1024
    s = _inputs(hc, 1, d)
    mix, K = (2 + hc) * hc, hc * d
    rt = (mix + 15) // 16
    p = H.hc_fn_pack(f32_dev(s["hc_fn"]), hc=hc).cpu().numpy().view(np.uint16)
    v = N.bits_to_f64(p.reshape(K // 32, 3 * rt, 4, 16, 8))         # [step][tile][lane//16][lane%16][8]
    cols = v.transpose(1, 3, 0, 2, 4).reshape(3 * rt * 16, K)         # [packed column][feature]
    terms = cols.reshape(3, rt * 16, K)
    assert not terms[:, mix:].any()
    hi, mid, lo = terms[:, :mix]
    w = s["hc_fn"].astype(np.float64)
    assert np.array_equal(hi, torch.from_numpy(s["hc_fn"]).to(torch.bfloat16).double().numpy())
    assert np.array_equal((hi + mid) + lo, w)


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("n,d", [(1, 64), (37, 1088), (300, 5120), (2100, 1024)])
def test_pre_post_bit_exact(hc, n, d):
    say(f"[hc={hc}] pre/post n={n} d={d}")
    s = _inputs(hc, n, d)
    X = bf16_dev(s["x"])
    y = H.hc_pre(X, f32_dev(s["pre_in"]))
    assert_bits_equal(host_bits(y), O.hc_pre(s["x"], s["pre_in"]), "hc_pre")
    xo = H.hc_post(bf16_dev(s["delta"]), X, f32_dev(s["post_in"]), f32_dev(s["comb_in"]))
    assert_bits_equal(host_bits(xo), O.hc_post(s["delta"], s["x"], s["post_in"], s["comb_in"]), "hc_post")


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("n", [1, 255, 300])
def test_split_sinkhorn(hc, n):
    say(f"[hc={hc}] split n={n}")
    s = _inputs(hc, n, 256)
    m = O.hc_mixes(s["x"], s["hc_fn"], 1e-6).astype(np.float32)
    pre, post, comb = H.hc_split_sinkhorn(f32_dev(m), f32_dev(s["hc_scale"]), f32_dev(s["hc_base"]), hc_mult=hc)
    rp, rq, rc = O.hc_split_sinkhorn(m, s["hc_scale"], s["hc_base"], hc)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")
    # every comb column and row of the last round sums to about one
    c = host_f32(comb).astype(np.float64)
    assert np.abs(c.sum(axis=1) - 1).max() < 1e-4


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("n,d", [(1, 64), (13, 1024), (300, 5120), (4096, 1024)])
def test_mixes(hc, n, d):
    say(f"[hc={hc}] mixes n={n} d={d}")
    s = _inputs(hc, n, d)
    X = bf16_dev(s["x"])
    p = _dev_params(s)
    ref = O.hc_mixes(s["x"], s["hc_fn"], 1e-6)
    rp, rq, rc = O.hc_split_sinkhorn(ref, s["hc_scale"], s["hc_base"], hc)
    pre, post, comb, mixes = H.hc_mixes(X, p["fn_packed"], p["hc_scale"], p["hc_base"], return_mixes=True)
    assert_mixes_close(host_f32(mixes), ref)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")
    # without a mixes output: the same coefficients
    pre2, post2, comb2 = H.hc_mixes(X, p["fn_packed"], p["hc_scale"], p["hc_base"])
    assert_bits_equal(host_f32(pre2).view(np.uint32), host_f32(pre).view(np.uint32), "pre (workspace mixes)")
    assert_bits_equal(host_f32(comb2).view(np.uint32), host_f32(comb).view(np.uint32), "comb (workspace mixes)")
    # mixes only
    m2 = H.hc_mixes(X, p["fn_packed"])
    assert_bits_equal(host_f32(m2).view(np.uint32), host_f32(mixes).view(np.uint32), "mixes alone")


def _boundary(hc, n, d, fresh, norm, with_delta, want_mean=True, t0=0):
    s = _inputs(hc, n, d, t0)
    kw = dict(x=s["x"], pre_in=None if fresh else s["pre_in"], gamma=s["gamma"] if norm else None,
              hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"], want_mean=want_mean)
    dev = dict(_dev_params(s), pre_in=None if fresh else f32_dev(s["pre_in"]),
               gamma=f32_dev(s["gamma"]) if norm else None, want_mean=want_mean)
    if with_delta:
        kw.update(delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"])
        dev.update(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]))
    return s, kw, dev


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("n,d", [(40, 1024), (300, 5120)])
@pytest.mark.parametrize("fresh,norm", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("with_delta", [False, True])
def test_boundary(hc, n, d, fresh, norm, with_delta):
    say(f"[hc={hc}] boundary n={n} d={d} fresh={fresh} norm={norm} delta={with_delta}")
    s, kw, dev = _boundary(hc, n, d, fresh, norm, with_delta)
    ref = O.boundary(**kw)
    got = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, **dev)
    _check_boundary(ref, got, s, fresh, norm)
    # the tap: the mean over the new streams (one fp32 rounding of the hc-term sum at most)
    assert_bf16_close(host_bits(got["x_mean"]), ref["x_mean"], "x_mean")


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("fresh", [False, True])
def test_boundary_halves_and_workspace_mixes(hc, fresh):
    """begin + end equals the whole call bit for bit, with or without a mixes
    output."""
    say(f"[hc={hc}] boundary halves fresh={fresh}")
    s, _, dev = _boundary(hc, 130, 2048, fresh, True, True)
    X = bf16_dev(s["x"])
    whole = H.hc_boundary(X, want_mixes=True, **dev)
    a, o = H._prepare_boundary(X, **dev)           # no mixes output: workspace
    assert o.get("mixes") is None
    import ctypes
    st = torch.cuda.current_stream().cuda_stream
    assert H.lib().hc_boundary_begin(ctypes.byref(a), ctypes.c_void_p(st)) == 0
    assert H.lib().hc_boundary_end(ctypes.byref(a), ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    for k in ("x_out", "y", "x_mean"):
        assert_bits_equal(host_bits(o[k]), host_bits(whole[k]), k)
    for k in ("pre", "post", "comb"):
        assert_bits_equal(host_f32(o[k]).view(np.uint32), host_f32(whole[k]).view(np.uint32), k)


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("with_delta", [False, True])
def test_expanded_entry(hc, with_delta):
    say(f"[hc={hc}] expanded entry delta={with_delta}")
    s = _inputs(hc, 100, 1024)
    h = s["x"][:, 0]
    kw = dict(x=h, x_expanded=True, hc=hc, want_mean=True, gamma=s["gamma"], hc_fn=s["hc_fn"],
              hc_base=s["hc_base"], hc_scale=s["hc_scale"])
    dev = dict(_dev_params(s), gamma=f32_dev(s["gamma"]))
    if with_delta:
        kw.update(delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"])
        dev.update(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]))
    ref = O.boundary(**kw)
    got = H.hc_boundary(bf16_dev(h), x_expanded=True, hc_mult=hc, want_mean=True, want_mixes=True, **dev)
    _check_boundary(ref, got, dict(s, x=O.expand_streams(h, hc)), True, True)
    assert_bf16_close(host_bits(got["x_mean"]), ref["x_mean"], "x_mean")
    if not with_delta:
        assert_bits_equal(host_bits(got["x_mean"]), h, "x_mean of the copies is the embedding")


@pytest.mark.parametrize("hc", HCS)
def test_stack_exit(hc):
    """Last write, read with the last pre, RMSNorm (eps 1e-20); no mixes."""
    say(f"[hc={hc}] exit")
    s = _inputs(hc, 77, 5120)
    ref = O.boundary(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"], pre_in=s["pre_in"],
                     gamma=s["gamma"], rms_eps=1e-20)
    got = H.hc_boundary(bf16_dev(s["x"]), delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]),
                        comb_in=f32_dev(s["comb_in"]), pre_in=f32_dev(s["pre_in"]), gamma=f32_dev(s["gamma"]),
                        rms_eps=1e-20)
    assert_bits_equal(host_bits(got["x_out"]), ref["x_out"], "x_out")
    assert_bf16_close(host_bits(got["y"]), ref["y"], "z")


def test_hc4_workspace_survives_other_hc_calls():
    """A workspace shared with hc = 8 calls (their per-slice records) keeps the hc = 4 exchange words
    intact: the hc = 4 few-tile boundary before and after gives the same bits."""
    say("[hc=4/8] shared workspace")
    s4 = synth.boundary_inputs("decode", 0, 64, 1024)
    s8 = _inputs(8, 64, 1024)
    ws = torch.zeros(max(H.lib().hc_workspace_bytes(64, 4, 1024), H.lib().hc_workspace_bytes(64, 8, 1024)),
                     dtype=torch.uint8, device="cuda")
    dev4 = dict(delta=bf16_dev(s4["delta"]), post_in=f32_dev(s4["post_in"]), comb_in=f32_dev(s4["comb_in"]),
                pre_in=f32_dev(s4["pre_in"]), fn_packed=H.hc_fn_pack(f32_dev(s4["hc_fn"])),
                hc_base=f32_dev(s4["hc_base"]), hc_scale=f32_dev(s4["hc_scale"]))
    X4 = bf16_dev(s4["x"])
    first = H.hc_boundary(X4, out={"workspace": ws}, **dev4)
    torch.cuda.synchronize()
    first = {k: v.clone() for k, v in first.items() if isinstance(v, torch.Tensor) and k != "workspace"}
    _, _, dev8 = _boundary(8, 64, 1024, True, True, True)
    for _ in range(3):
        H.hc_boundary(bf16_dev(s8["x"]), out={"workspace": ws}, **dev8)
    again = H.hc_boundary(X4, out={"workspace": ws}, **dev4)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(again[k], v), k
    assert int(ws[4160:4164].cpu().numpy().view(np.uint32)[0]) == 0


@pytest.mark.parametrize("hc,n,d,norm", [(8, 40, 10240, True), (8, 19, 32768, False), (2, 3, 32768, True)])
def test_boundary_widest_rows(hc, n, d, norm):
    """The widest rows: d = 10240 with the RMSNorm (its limit) and d = 32768
    (the library's limit; hc = 2 with the RMSNorm is rejected above 10240)."""
    if norm and d > 10240:
        with pytest.raises(H.HCError):
            H.hc_boundary(bf16_dev(np.zeros((n, hc, d), np.uint16)), gamma=f32_dev(np.ones(d, np.float32)),
                          **_dev_params(_inputs(hc, 1, d)))
        return
    say(f"[hc={hc}] widest rows n={n} d={d} norm={norm}")
    s, kw, dev = _boundary(hc, n, d, True, norm, True)
    ref = O.boundary(**kw)
    got = H.hc_boundary(bf16_dev(s["x"]), want_mixes=True, **dev)
    _check_boundary(ref, got, s, True, norm)


@pytest.mark.parametrize("hc", HCS)
def test_graph_replay_and_determinism(hc):
    """The four-launch boundary captured in a graph and replayed on changing
    inputs (eager work and synchronisations between the replays): every replay
    equals the eager call on the same inputs bit for bit, and two eager calls
    agree bit for bit."""
    say(f"[hc={hc}] graph replay")
    s0 = _inputs(hc, 300, 1024)
    s1 = _inputs(hc, 300, 1024, t0=300)
    dev = _dev_params(s0)
    X, D = bf16_dev(s0["x"]), bf16_dev(s0["delta"])
    P, C, G = f32_dev(s0["post_in"]), f32_dev(s0["comb_in"]), f32_dev(s0["gamma"])
    call = H.BoundaryCall(X, delta=D, post_in=P, comb_in=C, gamma=G, want_mixes=True, want_mean=True, **dev)
    o = call.outputs

    def load(s):
        X.copy_(bf16_dev(s["x"]))
        D.copy_(bf16_dev(s["delta"]))
        P.copy_(f32_dev(s["post_in"]))
        C.copy_(f32_dev(s["comb_in"]))

    def snapshot():
        torch.cuda.synchronize()
        return {k: (host_bits(v) if v.dtype == torch.bfloat16 else host_f32(v).view(np.uint32))
                for k, v in o.items() if isinstance(v, torch.Tensor) and k != "workspace"}

    eager = []
    for s in (s0, s1):
        load(s)
        call.run()
        first = snapshot()
        call.run()
        again = snapshot()
        for k in first:
            assert np.array_equal(first[k], again[k]), f"{k}: two eager calls differ"
        eager.append(first)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run()
    for rep, i in enumerate((0, 1, 1, 0)):
        load((s0, s1)[i])
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k in got:
            assert np.array_equal(got[k], eager[i][k]), f"replay {rep}: {k} differs from the eager call"
