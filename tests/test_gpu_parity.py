"""GPU parity: every libhc entry point against the CPU oracle on the same
seeded inputs, through the C ABI (via the ctypes binding).

Bars: bf16 stream outputs bit-exact where both sides run the same fp32
operation sequence on the same inputs (hc_post, hc_pre), else within 1 bf16
ulp; mixes floored relative error <= 1e-4; pre/post/comb absolute error <=
1e-5."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests import numerics as N
from tests.gpu_util import (DEV, assert_bf16_close, assert_bits_equal, assert_coef_close, assert_mixes_close,
                            assert_workspace_clean, bf16_dev, f32_dev, host_bits, host_f32, say, write_floor)
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu
rng = np.random.default_rng(777)


def rand_bits(shape, scale=1.0):
    return synth.f64_to_bf16_bits(rng.standard_normal(shape) * scale)


def params(d, seed=3):
    g = np.random.default_rng(seed)
    fn = (g.standard_normal((24, 4 * d)) * 0.02).astype(np.float32)
    base = (g.standard_normal(24) * 0.1).astype(np.float32)
    scale = g.uniform(0.5, 2.0, 3).astype(np.float32)
    return fn, base, scale


def packed(fn):
    return H.hc_fn_pack(f32_dev(fn))


# ------------------------------------------------------------------ packing
@pytest.mark.parametrize("d", [64, 5120])
def test_pack_terms_reconstruct_weight(d):
    """Tiles 0/1/2 hold hi/mid/lo of rows 0..15 (column n = row n); tile 3 holds
    hi of rows 16..23 in columns 0..7 and mid of rows 16..23 in columns 8..15;
    tile 4 holds lo of rows 16..23 in columns 0..7 and zeros."""
    say(f"[pack] d={d}")
    fn, _, _ = params(d)
    p = packed(fn).cpu().numpy().view(np.uint16)
    main = (d // 32) * 4 * 5 * 64 * 8
    assert p.size == main * 5 // 4                       # the four stream blocks, then their sum

    def terms(rec, blocks):
        # tile[st, k, nt, col, feature-in-step]: lane = 16*g + col holds features 8g..8g+7
        tile = rec.reshape(d // 32, blocks, 5, 4, 16, 8).transpose(0, 1, 2, 4, 3, 5).reshape(d // 32, blocks, 5, 16,
                                                                                            32)

        def rows(nt, cols):                             # -> [len(cols), blocks*d] in feature order k*d + f
            t = tile[:, :, nt][:, :, cols]              # [st, k, col, 32]
            return t.transpose(2, 1, 0, 3).reshape(len(cols), blocks * d)
        lo8, hi8 = np.arange(8), np.arange(8, 16)
        assert not rows(4, hi8).any()
        return (np.concatenate([rows(0, np.arange(16)), rows(3, lo8)]),
                np.concatenate([rows(1, np.arange(16)), rows(3, hi8)]),
                np.concatenate([rows(2, np.arange(16)), rows(4, lo8)]))

    hi, mid, lo = terms(N.bits_to_f64(p[:main]), 4)
    thi = torch.from_numpy(fn).to(torch.bfloat16).float().numpy()
    assert np.array_equal(hi, thi)                      # hi = nearest bf16 of w
    err = np.abs(hi + mid + lo - fn.astype(np.float64))
    assert (err <= 2.0 ** -25 * np.abs(fn) + 1e-45).all()
    # the stream-summed block: the same split of the fp32 rounding of the fp64 sum over the four blocks
    ws = fn.astype(np.float64).reshape(24, 4, d).sum(axis=1).astype(np.float32)
    shi, smid, slo = terms(N.bits_to_f64(p[main:]), 1)
    assert np.array_equal(shi, torch.from_numpy(ws).to(torch.bfloat16).float().numpy())
    serr = np.abs(shi + smid + slo - ws.astype(np.float64))
    assert (serr <= 2.0 ** -25 * np.abs(ws) + 1e-45).all()


# ------------------------------------------------------------------ split / Sinkhorn
@pytest.mark.parametrize("iters", [1, 20])
def test_split_sinkhorn_stage(iters):
    say(f"[split] iters={iters}")
    n = 1000
    mixes = (rng.standard_normal((n, 24)) * 2.86).astype(np.float32)
    _, base, scale = params(64, 11)
    pre, post, comb = H.hc_split_sinkhorn(f32_dev(mixes), f32_dev(scale), f32_dev(base), 4, iters, 1e-6)
    rp, rq, rc = O.hc_split_sinkhorn(mixes, scale, base, 4, iters, 1e-6)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")


@pytest.mark.parametrize("n", [1, 17, 8192, 8193])
def test_split_sinkhorn_both_layouts(n):
    """16 lanes per token up to 8192 tokens, a comb row per lane beyond."""
    say(f"[split] n={n}")
    mixes = (np.random.default_rng(n).standard_normal((n, 24)) * 2.86).astype(np.float32)
    _, base, scale = params(64, 11)
    pre, post, comb = H.hc_split_sinkhorn(f32_dev(mixes), f32_dev(scale), f32_dev(base), 4, 20, 1e-6)
    rp, rq, rc = O.hc_split_sinkhorn(mixes, scale, base, 4, 20, 1e-6)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")


# ------------------------------------------------------------------ hc_post / hc_pre
@pytest.mark.parametrize("n,d", [(37, 5120), (16, 64), (1, 128), (300, 320), (17, 7168)])
def test_hc_post_bit_exact(n, d):
    say(f"[hc_post] n={n} d={d}")
    x = rand_bits((n, 4, d)); delta = rand_bits((n, d))
    post = rng.uniform(0, 2, (n, 4)).astype(np.float32)
    comb = rng.dirichlet(np.ones(4), (n, 4)).transpose(0, 2, 1).astype(np.float32)
    got = H.hc_post(bf16_dev(delta), bf16_dev(x), f32_dev(post), f32_dev(comb))
    assert_bits_equal(host_bits(got), O.hc_post(delta, x, post, comb), "x_out")


@pytest.mark.parametrize("n,d", [(37, 5120), (16, 64), (300, 320), (17, 7168)])
def test_hc_pre_bit_exact(n, d):
    say(f"[hc_pre] n={n} d={d}")
    x = rand_bits((n, 4, d))
    pre = rng.uniform(0, 1, (n, 4)).astype(np.float32)
    got = H.hc_pre(bf16_dev(x), f32_dev(pre))
    assert_bits_equal(host_bits(got), O.hc_pre(x, pre), "y")


def test_identities_on_gpu():
    say("[identities]")
    n, d = 20, 512
    x = rand_bits((n, 4, d)); delta = rand_bits((n, d))
    eye = np.broadcast_to(np.eye(4, dtype=np.float32), (n, 4, 4)).copy()
    got = H.hc_post(bf16_dev(delta), bf16_dev(x), f32_dev(np.zeros((n, 4), np.float32)), f32_dev(eye))
    assert_bits_equal(host_bits(got), x, "post=0, comb=I")
    for j in range(4):
        p = np.zeros((n, 4), np.float32); p[:, j] = 1
        assert_bits_equal(host_bits(H.hc_pre(bf16_dev(x), f32_dev(p))), x[:, j], f"one-hot pre {j}")


# ------------------------------------------------------------------ hc_mixes
# n <= 128 (d a multiple of 64 from 256 to 8192) runs the few-tile exchange; otherwise the stream
# kernel (two chunks in flight, loop unrolled by two) with 64-feature chunks
# up to 2048 tokens and from d = 256 the few-tile exchange (one launch; 1 chunk
# per slice at n <= 192 and d = 5120, 2 at (300, 5120), 5 at (1000, 5120), 10
# at (2048, 5120), 2 at (700, 2048), 8 at (1500, 4096)); else the projection
# kernel and the finish (d = 64; 20 chunks per slice at 4096 and 4097, a
# ragged last tile; 4 at (5000, 1024)): every tail of the unrolled loops
@pytest.mark.parametrize("n,d", [(32, 5120), (45, 5120), (16, 64), (3, 1024), (19, 7168), (1000, 5120),
                                 (2048, 5120), (300, 5120), (4096, 5120), (4097, 5120), (5000, 1024),
                                 (129, 1024), (700, 2048), (1500, 4096)])
def test_hc_mixes_end_to_end(n, d):
    say(f"[hc_mixes] n={n} d={d}")
    x = rand_bits((n, 4, d))
    fn, base, scale = params(d)
    pre, post, comb, mixes = H.hc_mixes(bf16_dev(x), packed(fn), f32_dev(scale), f32_dev(base),
                                        return_mixes=True)
    rm = O.hc_mixes(x, fn, 1e-6)
    assert_mixes_close(host_f32(mixes), rm)
    rp, rq, rc = O.hc_split_sinkhorn(rm, scale, base)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")
    only = H.hc_mixes(bf16_dev(x), packed(fn))
    assert torch.equal(only, mixes)


def test_hc_mixes_stress_full_size_every_token():
    """hc_mixes on the channel-outlier stress workload (n = 32768: 512 tiles x
    one slice of 80 chunks, whose per-chunk sums are carried in fp64), every
    token against the oracle, in chunks."""
    say("[hc_mixes stress] n=32768, every token")
    s = synth.boundary_inputs("stress")
    X = bf16_dev(s["x"])
    pre, post, comb, mixes = H.hc_mixes(X, packed(s["hc_fn"]), f32_dev(s["hc_scale"]), f32_dev(s["hc_base"]),
                                        return_mixes=True)
    torch.cuda.synchronize()
    del X
    got = {k: host_f32(v) for k, v in (("pre", pre), ("post", post), ("comb", comb), ("mixes", mixes))}
    for a in range(0, s["x"].shape[0], 4 * FULL_CHUNK):
        b = a + 4 * FULL_CHUNK
        say(f"  oracle tokens {a}..{b}")
        rm = O.hc_mixes(s["x"][a:b], s["hc_fn"], 1e-6)
        assert_mixes_close(got["mixes"][a:b], rm)
        rp, rq, rc = O.hc_split_sinkhorn(rm, s["hc_scale"], s["hc_base"])
        assert_coef_close(got["pre"][a:b], rp, "pre")
        assert_coef_close(got["post"][a:b], rq, "post")
        assert_coef_close(got["comb"][a:b], rc, "comb")


# ------------------------------------------------------------------ one sublayer step (n=32)
def test_step_workload():
    say("[step workload] n=32")
    s = synth.step_inputs()
    x, delta, fn, base, scale, pre_in = (s[k] for k in ("x", "delta", "hc_fn", "hc_base", "hc_scale", "pre_in"))
    X = bf16_dev(x)
    pre, post, comb = H.hc_mixes(X, packed(fn), f32_dev(scale), f32_dev(base))
    y = H.hc_pre(X, f32_dev(pre_in))
    xo = H.hc_post(bf16_dev(delta), X, post, comb)
    rm = O.hc_mixes(x, fn, 1e-6)
    rp, rq, rc = O.hc_split_sinkhorn(rm, scale, base)
    assert_coef_close(host_f32(pre), rp, "pre")
    assert_coef_close(host_f32(post), rq, "post")
    assert_coef_close(host_f32(comb), rc, "comb")
    assert_bits_equal(host_bits(y), O.hc_pre(x, pre_in), "y")
    assert_bf16_close(host_bits(xo), O.hc_post(delta, x, rq, rc), "x_out", floor=write_floor(delta, x))


# ------------------------------------------------------------------ fused boundary
def _boundary_case(workload, t0, t1, fresh, norm, entry=False, exit_=False, d=None, two=False):
    s = synth.boundary_inputs(workload, t0, t1) if d is None else synth.boundary_inputs(workload, t0, t1, d)
    kw = dict(x=s["x"], pre_in=None if fresh else s["pre_in"], gamma=s["gamma"] if norm else None)
    if not entry:
        kw.update(delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"])
    if not exit_:
        kw.update(hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"])
    ref = O.boundary(**kw)
    dev = {k: (bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)) for k, v in kw.items()
           if v is not None and k != "hc_fn"}
    if "hc_fn" in kw:
        dev["fn_packed"] = packed(kw["hc_fn"])
    x = dev.pop("x")
    got = H.hc_boundary(x, **dev, want_mixes=not exit_, two_launch=two)
    return ref, got, s


def _check_boundary(ref, got, s, fresh, norm):
    assert_workspace_clean(got)
    if ref["x_out"] is not None:
        assert_bits_equal(host_bits(got["x_out"]), ref["x_out"], "x_out")
    if ref["mixes"] is not None:
        assert_mixes_close(host_f32(got["mixes"]), ref["mixes"])
        assert_coef_close(host_f32(got["pre"]), ref["pre"], "pre")
        assert_coef_close(host_f32(got["post"]), ref["post"], "post")
        assert_coef_close(host_f32(got["comb"]), ref["comb"], "comb")
    y = host_bits(got["y"])
    if fresh:
        # The read weights of the two sides differ by <= 1e-5, so the unrounded
        # read rows differ by at most floor = 1e-5 * sum_j |X'_j| (the drift
        # carried through the read).  Each side then rounds to bf16, the GPU's
        # value possibly one binade above the oracle's: |y_g - y_r| <= floor +
        # ulp(y_r)/2 + ulp(2 y_r)/2 = floor + 1.5 ulp(y_r).
        xp = ref["x_out"] if ref["x_out"] is not None else s["x"]
        floor = N.COEF_ABS_TOL * np.abs(N.bits_to_f64(xp)).sum(axis=-2)
        yr = N.bits_to_f64(O.hc_pre(xp, ref["pre"]))
        ybound = floor + 1.5 * N.bf16_ulp(yr)
        if norm:
            # z = bf16(gamma * (y * r)) on the rounded y: the y bound scales by
            # |gamma_i| * r; the two sides' r differ by at most 2^-9 relative (the
            # kernels take the mean square of y before its rounding, the oracle of
            # the bf16 y: each square moves by <= 2^-8 relative) plus the drift;
            # and z's own roundings add 1.5 ulp(z_r) as above.
            r = 1.0 / np.sqrt((yr * yr).mean(axis=-1, keepdims=True) + float(np.float32(1e-6)))
            zr = N.bits_to_f64(ref["y"])
            g = np.abs(s["gamma"].astype(np.float64))[None, :]
            zbound = (ybound * r * g + 2.0 ** -9 * np.abs(zr)) * 1.01 + 1.5 * N.bf16_ulp(zr)
            assert_bf16_close(y, ref["y"], "z (fresh)", floor=zbound)
        else:
            assert_bf16_close(y, ref["y"], "y (fresh)", floor=ybound)
    elif norm:
        assert_bf16_close(y, ref["y"], "z")
    else:
        assert_bits_equal(y, ref["y"], "y")


@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("fresh", [False, True])
@pytest.mark.parametrize("norm", [False, True])
def test_boundary_small(fresh, norm, two):
    say(f"[boundary] prefill tokens 0..40 fresh={fresh} norm={norm} two_launch={two}")
    ref, got, s = _boundary_case("prefill", 0, 40, fresh, norm, two=two)
    _check_boundary(ref, got, s, fresh, norm)


@pytest.mark.parametrize("n,d", [(1, 5120), (17, 1024), (23, 7168), (130, 2048)])
@pytest.mark.parametrize("fresh", [False, True])
def test_boundary_shapes(n, d, fresh):
    """Other widths and ragged token counts."""
    say(f"[boundary] n={n} d={d} fresh={fresh}")
    ref, got, s = _boundary_case("prefill", 0, n, fresh, True, d=d)
    _check_boundary(ref, got, s, fresh, True)


@pytest.mark.parametrize("fresh", [False, True])
def test_boundary_entry(fresh):
    say(f"[boundary entry] fresh={fresh}")
    ref, got, s = _boundary_case("prefill", 100, 133, fresh, True, entry=True)
    assert got["x_out"] is None
    _check_boundary(ref, got, s, fresh, True)


# The block entry from the streams as given stores no X': the 128-token
# projection kernel, whose last workgroup's second 64-token record tile lies
# past n when the count of 64-token tiles is odd (n = 191: 3 tiles; 4160: 65,
# where the given pre with the RMSNorm runs as a 4096-token exchange and a
# 64-token decode call instead).  Every token, with the stream mean.
@pytest.mark.parametrize("n", [191, 4160])
@pytest.mark.parametrize("fresh,norm", [(True, True), (True, False), (False, True), (False, False)])
def test_entry_odd_tile_counts(n, fresh, norm):
    say(f"[entry] n={n} fresh={fresh} norm={norm}: every token, with the stream mean")
    s = synth.boundary_inputs("prefill", 0, n)
    kw = dict(x=s["x"], pre_in=None if fresh else s["pre_in"], gamma=s["gamma"] if norm else None,
              hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"])
    ref = O.boundary(**kw, want_mean=True)
    dev = {k: (bf16_dev(v) if v.dtype == np.uint16 else f32_dev(v)) for k, v in kw.items()
           if v is not None and k != "hc_fn"}
    dev["fn_packed"] = packed(s["hc_fn"])
    x = dev.pop("x")
    got = H.hc_boundary(x, **dev, want_mixes=True, want_mean=True)
    torch.cuda.synchronize()
    assert got["x_out"] is None
    _check_boundary(ref, got, s, fresh, norm)
    assert_bits_equal(host_bits(got["x_mean"]), ref["x_mean"], "stream mean")


def test_boundary_exit():
    say("[boundary exit]")
    ref, got, s = _boundary_case("prefill", 7, 30, False, True, exit_=True)
    _check_boundary(ref, got, s, False, True)


def test_boundary_stress_outliers_small():
    say("[boundary] stress tokens 0..24")
    ref, got, s = _boundary_case("stress", 0, 24, False, True)
    _check_boundary(ref, got, s, False, True)


@pytest.mark.parametrize("two", [False, True])
def test_boundary_deterministic_and_guarded(two):
    say(f"[boundary] determinism + guard bands, two_launch={two}")
    s = synth.boundary_inputs("prefill", 0, 33)
    n, d = 33, 5120
    guard = 4096
    dev = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
               pre_in=f32_dev(s["pre_in"]), fn_packed=packed(s["hc_fn"]), hc_base=f32_dev(s["hc_base"]),
               hc_scale=f32_dev(s["hc_scale"]), gamma=f32_dev(s["gamma"]))
    X = bf16_dev(s["x"])
    outs = []
    for rep in range(2):
        bufs = {
            "x_out": torch.full((n * 4 * d + 2 * guard,), 0x7A7A, dtype=torch.int16, device=DEV),
            "y": torch.full((n * d + 2 * guard,), 0x7A7A, dtype=torch.int16, device=DEV),
            "pre": torch.full((n * 4 + 2 * guard,), 7.5, device=DEV),
            "post": torch.full((n * 4 + 2 * guard,), 7.5, device=DEV),
            "comb": torch.full((n * 16 + 2 * guard,), 7.5, device=DEV),
            "mixes": torch.full((n * 24 + 2 * guard,), 7.5, device=DEV),
        }
        shapes = {"x_out": (n, 4, d), "y": (n, d), "pre": (n, 4), "post": (n, 4), "comb": (n, 4, 4),
                  "mixes": (n, 24)}
        views = {}
        for k, b in bufs.items():
            v = b[guard:-guard]
            if b.dtype == torch.int16:
                v = v.view(torch.bfloat16)
            views[k] = v.view(shapes[k])
        H.hc_boundary(X, **dev, out=views, two_launch=two)
        torch.cuda.synchronize()
        for k, b in bufs.items():
            fill = 0x7A7A if b.dtype == torch.int16 else 7.5
            assert bool((b[:guard] == fill).all()) and bool((b[-guard:] == fill).all()), f"guard of {k} touched"
        outs.append({k: v.clone() for k, v in views.items()})
    for k in outs[0]:
        assert torch.equal(outs[0][k].view(torch.int16) if outs[0][k].dtype == torch.bfloat16 else outs[0][k],
                           outs[1][k].view(torch.int16) if outs[1][k].dtype == torch.bfloat16 else outs[1][k]), k


def test_prepared_call_matches_and_repeats():
    """BoundaryCall (checked once, re-enqueued) gives the bits of hc_boundary,
    call after call on the same buffers and workspace."""
    say("[boundary] prepared call, fresh read, n=300")
    s = synth.boundary_inputs("prefill", 0, 300)
    dev = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
               fn_packed=packed(s["hc_fn"]), hc_base=f32_dev(s["hc_base"]), hc_scale=f32_dev(s["hc_scale"]),
               gamma=f32_dev(s["gamma"]))
    X = bf16_dev(s["x"])
    ref = H.hc_boundary(X, **dev, want_mixes=True)
    call = H.BoundaryCall(X, **dev, want_mixes=True)
    for rep in range(3):
        for k in ("x_out", "y", "pre", "post", "comb", "mixes"):
            call.outputs[k].fill_(7)
        call.run()
        torch.cuda.synchronize()
        for k in ("x_out", "y", "pre", "post", "comb", "mixes"):
            a, b = call.outputs[k], ref[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"{k} differs on call {rep}"
    # the two-launch split (hc_boundary_begin + _end, enqueued apart) sums the
    # projection over other feature slices: the same X', the other outputs within
    # the parity bars of the oracle
    for k in ("x_out", "y", "pre", "post", "comb", "mixes"):
        call.outputs[k].fill_(7)
    call.begin()
    call.end()
    torch.cuda.synchronize()
    assert torch.equal(call.outputs["x_out"].view(torch.int16), ref["x_out"].view(torch.int16))
    kw = dict(x=s["x"], delta=s["delta"], post_in=s["post_in"], comb_in=s["comb_in"], pre_in=None,
              hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"], gamma=s["gamma"])
    oref = O.boundary(**kw)
    split = dict(call.outputs)
    split["workspace"] = None
    _check_boundary(oref, split, s, True, True)


# ------------------------------------------------------------------ full size, every token
FULL_CHUNK = 1024      # tokens per oracle call (bounds the oracle's temporaries)


def _host(got):
    return {k: (v.detach().cpu() if isinstance(v, torch.Tensor) else v) for k, v in got.items() if k != "workspace"}


def _compare_every_token(s, got, fresh, tag):
    n = s["x"].shape[0]
    host = _host(got)
    for a in range(0, n, FULL_CHUNK):
        b = min(n, a + FULL_CHUNK)
        say(f"  {tag}: oracle tokens {a}..{b}")
        ref = O.boundary(x=s["x"][a:b], delta=s["delta"][a:b], post_in=s["post_in"][a:b],
                         comb_in=s["comb_in"][a:b], pre_in=None if fresh else s["pre_in"][a:b],
                         hc_fn=s["hc_fn"], hc_base=s["hc_base"], hc_scale=s["hc_scale"], gamma=s["gamma"])
        sub = {k: (v[a:b] if v is not None else None) for k, v in host.items()}
        _check_boundary(ref, sub, {"x": s["x"][a:b], "gamma": s["gamma"]}, fresh, True)


def _full_size(workload, fresh, two):
    s = synth.boundary_inputs(workload)
    X = bf16_dev(s["x"])
    dev = dict(delta=bf16_dev(s["delta"]), post_in=f32_dev(s["post_in"]), comb_in=f32_dev(s["comb_in"]),
               pre_in=None if fresh else f32_dev(s["pre_in"]), fn_packed=packed(s["hc_fn"]),
               hc_base=f32_dev(s["hc_base"]), hc_scale=f32_dev(s["hc_scale"]), gamma=f32_dev(s["gamma"]))
    say("  launching")
    got = H.hc_boundary(X, **dev, want_mixes=True, two_launch=two)
    torch.cuda.synchronize()
    assert_workspace_clean(got)
    del X, dev
    return s, got


@pytest.mark.parametrize("fresh,two", [(True, False), (False, False), (False, True)])
def test_prefill_full_size_every_token(fresh, two):
    """The benchmark's call (B=1, T=4096, d=5120, RMSNorm) compared with the
    oracle on every token: the fresh read (two launches), the given read in one
    launch (the read-row exchange) and the given read in two launches."""
    say(f"[prefill n=4096] fresh={fresh} two_launch={two}: generating inputs")
    s, got = _full_size("prefill", fresh, two)
    assert got["y"].shape == (4096, 5120)
    _compare_every_token(s, got, fresh, "prefill")


@pytest.mark.parametrize("fresh", [True, False])
def test_stress_full_size_every_token(fresh):
    """The bandwidth-stress boundary: B=4 T=8192 (32768 tokens, X = 1.34 GB),
    heavy-tailed streams (1% of features x30), RMSNorm, both reads; every
    token against the oracle."""
    say(f"[stress n=32768] fresh={fresh}: generating inputs")
    s, got = _full_size("stress", fresh, False)
    _compare_every_token(s, got, fresh, "stress")
