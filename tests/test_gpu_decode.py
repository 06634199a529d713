"""GPU parity of the few-tile exchange at decode sizes: hc_boundary with a
given pre (with and without the RMSNorm of the read row), for n <= 128 run
as one launch ("Source layer, pairs pooled": Block.forward at
decode; "Reading weights"; "Final RMSNorm"): 64-token tiles, one 64-feature
chunk per workgroup; the owner slice of a token sums its words over the
slices, derives its coefficients and, with the RMSNorm, publishes the token's
factor r for the other slices.  Checked against the oracle on ragged token
counts and on widths that give a slice 1 to 16 owned tokens; on one workspace
reused across calls of changing n and inputs (the call epoch carried in the
workspace); and captured in a graph with the decode block's other calls and
replayed on new inputs."""
import numpy as np
import pytest
import torch

import transformer_hyper_connection_amd as P
from oracle import hc_oracle as O
from tests import test_gpu_parity as T
from tests.gpu_util import assert_workspace_clean, bf16_dev, f32_dev, host_bits, host_f32, say
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu


# widths from 256 to 8192 run the few-tile exchange (one 64-feature chunk per
# workgroup: S = d / 64 slices, an owner slice per token); 1088 and 1344 (17
# and 21 slices) give a slice up to four owned tokens, 2112 (33) two, 512 (8
# slices) eight and 768 (12) six; n = 65 leaves one valid token in the second
# tile; d = 10240 runs the two launches
@pytest.mark.parametrize("n,d", [(1, 5120), (16, 5120), (17, 5120), (100, 5120), (128, 5120), (129, 5120),
                                 (45, 7168), (70, 10240), (65, 1088), (128, 1344), (100, 2112), (3, 1024),
                                 (20, 512), (128, 768)])
@pytest.mark.parametrize("entry", [False, True])
def test_decode_boundary(n, d, entry):
    say(f"[decode] n={n} d={d} entry={entry}")
    ref, got, s = T._boundary_case("prefill", 0, n, False, False, entry=entry, d=d)
    T._check_boundary(ref, got, s, False, False)


# with the RMSNorm: each token's owner slice publishes its factor r for every
# slice of the tile (d = 8192 at n = 128 is 2 tiles x 128 slices = 256
# workgroups, the most the schedule takes)
@pytest.mark.parametrize("n,d", [(1, 5120), (17, 5120), (128, 5120), (129, 5120), (45, 7168), (128, 8192),
                                 (65, 1088), (128, 1344), (100, 2112), (3, 1024), (20, 512), (128, 768),
                                 (70, 10240)])
@pytest.mark.parametrize("entry", [False, True])
def test_decode_boundary_norm(n, d, entry):
    say(f"[decode norm] n={n} d={d} entry={entry}")
    ref, got, s = T._boundary_case("prefill", 0, n, False, True, entry=entry, d=d)
    T._check_boundary(ref, got, s, False, True)


def test_decode_norm_repeated_and_against_two_launches():
    """The few-tile exchange with the RMSNorm on one workspace, called again on
    new inputs (the call epoch advances) and beside the two launches of the
    same call (bit-equal streams); every call against the oracle."""
    ws = torch.zeros(H.lib().hc_workspace_bytes(128, 4, 5120), dtype=torch.uint8, device="cuda:0")
    for i, (t0, n) in enumerate(((0, 128), (500, 100), (0, 128))):
        say(f"[decode norm repeat] call {i}: tokens {t0}..{t0 + n}")
        s, dev = _inputs(t0, t0 + n)
        dev["gamma"] = f32_dev(s["gamma"])
        fn = H.hc_fn_pack(f32_dev(s["hc_fn"]))
        x = bf16_dev(s["x"])
        one = H.hc_boundary(x, fn_packed=fn, want_mixes=True, out={"workspace": ws}, **dev)
        two = H.hc_boundary(x, fn_packed=fn, want_mixes=True, two_launch=True, **dev)
        torch.cuda.synchronize()
        assert_workspace_clean(ws)
        assert np.array_equal(host_bits(one["x_out"]), host_bits(two["x_out"]))
        ref = O.boundary(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"],
                         pre_in=s["pre_in"], hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"],
                         gamma=s["gamma"])
        T._check_boundary(ref, one, s, False, True)


def _inputs(t0, t1, d=5120):
    s = synth.boundary_inputs("prefill", t0, t1, d)
    return s, dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
                   pre_in=f32_dev(s["pre_in"]), hc_base=f32_dev(s["hc_base"]), hc_scale=f32_dev(s["hc_scale"]))


def test_decode_workspace_reused_across_n():
    """One zeroed workspace for calls of n = 128, 64, 128, 256 (slices of two
    chunks), 17 and d = 7168 on changing inputs: every call matches the
    oracle and no wait times out."""
    ws = torch.zeros(max(H.lib().hc_workspace_bytes(256, 4, 5120), H.lib().hc_workspace_bytes(256, 4, 7168)),
                     dtype=torch.uint8, device="cuda:0")
    fns = {}
    for i, (n, d) in enumerate(((128, 5120), (64, 5120), (128, 5120), (256, 5120), (17, 5120), (60, 7168),
                                (128, 5120))):
        t0 = 300 * i
        say(f"[decode reuse] call {i}: tokens {t0}..{t0 + n}, d={d}")
        s, dev = _inputs(t0, t0 + n, d)
        if d not in fns:
            fns[d] = H.hc_fn_pack(f32_dev(s["hc_fn"]))
        fn = fns[d]
        got = H.hc_boundary(bf16_dev(s["x"]), fn_packed=fn, want_mixes=True, out={"workspace": ws}, **dev)
        ref = O.boundary(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"],
                         pre_in=s["pre_in"], hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"])
        T._check_boundary(ref, got, s, False, False)
        assert_workspace_clean(ws)


def test_decode_block_graph_replay():
    """The decode block's glue (entry, boundary, last write; n = 128) captured
    in one graph and replayed on new inputs: each replay equals the eager calls
    bit for bit, and the first also the oracle."""
    b0 = synth.block_inputs()
    rng = np.random.default_rng(7)                       # a second input set: tokens permuted, deltas swapped
    b1 = dict(b0, x=b0["x"][rng.permutation(b0["x"].shape[0])], delta_attn=b0["delta_ffn"],
              delta_ffn=b0["delta_attn"])
    blk = [b0, b1]
    (fa, ba, sa), (ff, bf_, sf) = blk[0]["attn"], blk[0]["ffn"]
    A = dict(fn_packed=H.hc_fn_pack(f32_dev(fa)), hc_base=f32_dev(ba), hc_scale=f32_dev(sa))
    F = dict(fn_packed=H.hc_fn_pack(f32_dev(ff)), hc_base=f32_dev(bf_), hc_scale=f32_dev(sf))
    X, PRE, DA, DF = (bf16_dev(blk[0]["x"]), f32_dev(blk[0]["pre_in"]), bf16_dev(blk[0]["delta_attn"]),
                      bf16_dev(blk[0]["delta_ffn"]))
    entry = P.BoundaryCall(X, pre_in=PRE, want_mixes=True, **A)
    e = entry.outputs
    bnd = P.BoundaryCall(X, delta=DA, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"], want_mixes=True, **F)
    b = bnd.outputs
    xo = torch.empty_like(X)

    def glue():
        entry.run()
        bnd.run()
        H.hc_post(DF, b["x_out"], b["post"], b["comb"], out=xo)

    def snapshot():
        torch.cuda.synchronize()
        return {k: host_bits(v) if v.dtype == torch.bfloat16 else host_f32(v)
                for k, v in (("x_out", b["x_out"]), ("y", b["y"]), ("pre", b["pre"]), ("comb", b["comb"]),
                             ("entry_pre", e["pre"]), ("out", xo))}

    def load(i):
        X.copy_(bf16_dev(blk[i]["x"]))
        PRE.copy_(f32_dev(blk[i]["pre_in"]))
        DA.copy_(bf16_dev(blk[i]["delta_attn"]))
        DF.copy_(bf16_dev(blk[i]["delta_ffn"]))

    eager = []
    for i in range(2):
        load(i)
        glue()
        eager.append(snapshot())
    ref = O.block(x=blk[0]["x"], pre_in=blk[0]["pre_in"], delta_attn=blk[0]["delta_attn"],
                  delta_ffn=blk[0]["delta_ffn"], attn=blk[0]["attn"], ffn=blk[0]["ffn"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        glue()                                            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        glue()
    for rep, i in enumerate((0, 1, 0, 1, 1)):
        say(f"[decode graph] replay {rep} on input set {i}")
        load(i)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for k in got:
            assert np.array_equal(got[k], eager[i][k]), f"replay {rep}: {k} differs from the eager call"
        assert_workspace_clean(entry.outputs["workspace"])
        assert_workspace_clean(bnd.outputs["workspace"])
        if rep == 0:
            np.testing.assert_allclose(got["entry_pre"], ref["attn"]["pre"], atol=1e-5, rtol=0)
