"""GPU parity on the multi-call workloads: one decode block's glue (n=128, two
sublayers) and the 80-sublayer HC stack with the stand-in sublayer (n=8192).

Both go through the C ABI (hc_boundary for the entry, the boundaries and the
stack exit; hc_post for the block's last write).  Every step is checked
teacher-forced: the GPU step gets the oracle's inputs and must meet the parity
bars (mixes floored relative error <= 1e-4, pre/post/comb absolute error <= 1e-5,
bf16 streams bit-exact where both sides run the same fp32 sequence, else within
1 ulp).  The free-running chains are compared too, as relative errors of the
streams (the block's output, the stack's streams at every depth): the pages fix
no bound for a chain, so the 1e-2 guard here is this suite's (parity unpinned
for chains)."""
import numpy as np
import pytest
import torch

from oracle import hc_oracle as O
from tests import numerics as N
from tests.gpu_util import (assert_bf16_close, assert_bits_equal, assert_coef_close, assert_mixes_close,
                            bf16_dev, f32_dev, host_bits, host_f32, say, write_floor)
from transformer_hyper_connection_amd import hc as H
from transformer_hyper_connection_amd import synth

pytestmark = pytest.mark.gpu


def _packed(fn):
    return H.hc_fn_pack(f32_dev(fn))


def _check_step(got, ref, what):
    assert_mixes_close(host_f32(got["mixes"]), ref["mixes"], f"{what} mixes")
    for k in ("pre", "post", "comb"):
        assert_coef_close(host_f32(got[k]), ref[k], f"{what} {k}")


# ------------------------------------------------------------------ decode block
def test_decode_block():
    """One block at decode (B=128, T=1): attention reads with the incoming mix,
    the feed-forward with the attention's pre; each step teacher-forced, then the
    chain end to end."""
    say("[decode block] n=128")
    s = synth.block_inputs()
    x, pre0, da, df = s["x"], s["pre_in"], s["delta_attn"], s["delta_ffn"]
    (fa, ba, sa), (ff, bf_, sf) = s["attn"], s["ffn"]
    ref = O.block(x=x, pre_in=pre0, delta_attn=da, delta_ffn=df, attn=s["attn"], ffn=s["ffn"])
    A = dict(fn_packed=_packed(fa), hc_base=f32_dev(ba), hc_scale=f32_dev(sa))
    Fp = dict(fn_packed=_packed(ff), hc_base=f32_dev(bf_), hc_scale=f32_dev(sf))
    X = bf16_dev(x)

    # entry: read with the incoming mix (no write), derive the attention's coefficients
    e = H.hc_boundary(X, pre_in=f32_dev(pre0), want_mixes=True, **A)
    _check_step(e, ref["attn"], "attn")
    assert_bits_equal(host_bits(e["y"]), ref["attn"]["y"], "attn read row")

    # boundary, teacher-forced: the oracle's attention coefficients in
    ra = ref["attn"]
    b = H.hc_boundary(X, delta=bf16_dev(da), post_in=f32_dev(ra["post"]), comb_in=f32_dev(ra["comb"]),
                      pre_in=f32_dev(ra["pre"]), want_mixes=True, **Fp)
    rf = ref["ffn"]
    assert_bits_equal(host_bits(b["x_out"]), rf["x_out"], "ffn streams (teacher-forced)")
    assert_bits_equal(host_bits(b["y"]), rf["y"], "ffn read row (teacher-forced)")
    _check_step(b, rf, "ffn (teacher-forced)")
    # last write, teacher-forced
    xo = H.hc_post(bf16_dev(df), bf16_dev(rf["x_out"]), f32_dev(rf["post"]), f32_dev(rf["comb"]))
    assert_bits_equal(host_bits(xo), ref["x_out"], "block output streams (teacher-forced)")

    # the chain end to end: the GPU's own coefficients carried from step to step.
    # The feed-forward step then starts from streams that differ from the
    # oracle's by up to an ulp, so its mixes and coefficients are those of a
    # perturbed input and the per-stage bars do not apply; the chain is held to
    # the suite's relative-error guard (the pages fix no bound for it).
    b2 = H.hc_boundary(X, delta=bf16_dev(da), post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"],
                       want_mixes=True, **Fp)
    xo2 = H.hc_post(bf16_dev(df), b2["x_out"], b2["post"], b2["comb"])
    assert_bf16_close(host_bits(b2["x_out"]), rf["x_out"], "ffn streams", floor=write_floor(da, x))
    drift = max(float(np.abs(host_f32(b2[k]).astype(np.float64) - rf[k]).max()) for k in ("pre", "post", "comb"))
    mix = float(N.floored_rel_err(host_f32(b2["mixes"]), rf["mixes"]).max())
    g, r = N.bits_to_f64(host_bits(xo2)), N.bits_to_f64(ref["x_out"])
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    say(f"  chained: ffn mixes floored rel {mix:.1e}, coefficient drift {drift:.1e}, block output rel {rel:.1e}")
    assert rel <= 1e-2


# ------------------------------------------------------------------ 80-sublayer stack
N_SUB = 80
SAMPLE = np.r_[0:256, 8192 - 256:8192]               # tokens checked against the oracle (both batch rows)


@pytest.fixture(scope="module")
def stack_case():
    say("[stack] generating the 8192-token, 80-sublayer inputs")
    s = synth.stack_inputs(N_SUB)
    say("  oracle, free-running on the sampled tokens")
    rec = []
    ref = O.stack(h=s["h"][SAMPLE], params=s["params"], gammas=s["gammas"], gamma_final=s["gamma_final"],
                  record=rec)
    return s, ref, rec


def test_stack_teacher_forced_every_depth(stack_case):
    """Each of the 80 sublayer boundaries and the stack exit, on the sampled
    tokens, with the oracle's state at that depth as input."""
    s, ref, rec = stack_case
    n, hc = len(SAMPLE), 4
    h = s["h"][SAMPLE]
    x = np.repeat(h[:, None, :], hc, axis=1)
    pre_in = np.full((n, hc), 0.25, dtype=np.float32)
    delta = post = comb = None
    worst = {"mixes": 0.0, "coef": 0.0}
    for d in range(N_SUB):
        fn, base, scale = s["params"][d]
        kw = dict(pre_in=f32_dev(pre_in), fn_packed=_packed(fn), hc_base=f32_dev(base), hc_scale=f32_dev(scale),
                  gamma=f32_dev(s["gammas"][d]), want_mixes=True)
        if d > 0:
            kw.update(delta=bf16_dev(delta), post_in=f32_dev(post), comb_in=f32_dev(comb))
        got = H.hc_boundary(bf16_dev(x), **kw)
        o = O.stack_step(s=d, x=x, delta=delta, post_in=post, comb_in=comb, pre_in=pre_in, params=s["params"],
                         gammas=s["gammas"])
        if d > 0:
            assert_bits_equal(host_bits(got["x_out"]), o["x_out"], f"depth {d} streams")
        assert_bf16_close(host_bits(got["y"]), o["y"], f"depth {d} stand-in sublayer output")
        _check_step(got, o, f"depth {d}")
        worst["mixes"] = max(worst["mixes"], float(N.floored_rel_err(host_f32(got["mixes"]), o["mixes"]).max()))
        worst["coef"] = max(worst["coef"], max(float(np.abs(host_f32(got[k]).astype(np.float64) - o[k]).max())
                                               for k in ("pre", "post", "comb")))
        # the oracle's state moves on (teacher forcing)
        xs, y, pre, post, comb = rec[d]
        x, delta, pre_in = xs, y, pre
    # exit: final write, final read with the last pre, final RMSNorm (eps 1e-20)
    got = H.hc_boundary(bf16_dev(x), delta=bf16_dev(delta), post_in=f32_dev(post), comb_in=f32_dev(comb),
                        pre_in=f32_dev(pre_in), gamma=f32_dev(s["gamma_final"]), rms_eps=1e-20)
    assert_bits_equal(host_bits(got["x_out"]), ref["x_out"], "exit streams")
    assert_bf16_close(host_bits(got["y"]), ref["z"], "exit read row")
    say(f"  worst over depth: mixes floored rel {worst['mixes']:.2e}, coefficients abs {worst['coef']:.2e}")


def test_stack_free_running_error_growth(stack_case):
    """The whole stack on the GPU at n=8192, its own outputs carried through all
    80 sublayers; the relative error of the streams against the free-running
    oracle, per depth, on the sampled tokens."""
    s, ref, rec = stack_case
    n, hc, d = 8192, 4, 5120
    say("  packing 80 weights, uploading the embedding")
    packed = [_packed(p[0]) for p in s["params"]]
    x = bf16_dev(s["h"]).view(n, 1, d).expand(n, hc, d).contiguous()
    pre = torch.full((n, hc), 0.25, dtype=torch.float32, device=x.device)
    delta = post = comb = None
    idx = torch.as_tensor(SAMPLE, device=x.device)
    curve = []
    for dep in range(N_SUB):
        fn, base, scale = s["params"][dep]
        kw = dict(pre_in=pre, fn_packed=packed[dep], hc_base=f32_dev(base), hc_scale=f32_dev(scale),
                  gamma=f32_dev(s["gammas"][dep]))
        if dep > 0:
            kw.update(delta=delta, post_in=post, comb_in=comb)
        o = H.hc_boundary(x, **kw)
        if dep > 0:
            x = o["x_out"]
        delta, post, comb, pre = o["y"], o["post"], o["comb"], o["pre"]
        g = N.bits_to_f64(host_bits(x.index_select(0, idx)))
        r = N.bits_to_f64(rec[dep][0])
        curve.append(float(np.linalg.norm(g - r) / np.linalg.norm(r)))
    o = H.hc_boundary(x, delta=delta, post_in=post, comb_in=comb, pre_in=pre, gamma=f32_dev(s["gamma_final"]),
                      rms_eps=1e-20)
    g = N.bits_to_f64(host_bits(o["y"].index_select(0, idx)))
    r = N.bits_to_f64(ref["z"])
    final = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    say("  relative error of the streams by depth: " +
        " ".join(f"{dep}:{e:.1e}" for dep, e in enumerate(curve) if dep % 10 == 0 or dep == N_SUB - 1) +
        f"; final read row {final:.1e}")
    assert curve[0] == 0.0                               # the entry does not write: the streams are the embedding
    assert max(curve) <= 1e-2 and final <= 1e-2
