"""CPU oracle for the Hyper-Connections (HC) residual glue.

TEST INFRASTRUCTURE.  This module is a plain, slow, deliberately unoptimised
NumPy statement of what the HC glue computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and this module imports
nothing from the product path.

Sources.  Every function cites the page of the model atlas it follows, by the
page title and the part of that page (code panel, equation, table):

* "Source layer, pairs pooled" -- the code panel with the ``Block`` class:
  its constructor (parameter shapes), ``forward`` (data flow and the lag of the
  reading mix), ``hc_mixes``, ``hc_pre`` and ``hc_post``; the parameter table.
* "Reading weights" -- the reading-weight equation and the code panel with the
  split/Sinkhorn kernel and its host wrapper.
* "Final RMSNorm" -- the RMSNorm equation, the ``RMSNorm`` class and the
  model driver ``Transformer.forward``.
* "Write the streams" -- the stream-update equation for ``hc_post``.

Precision.  The pages fix the arithmetic of ``hc_post`` and ``hc_pre``: both
are elementwise fp32 tensor expressions on bf16 streams (the coefficients are
fp32 parameters or fp32 kernel outputs), each product and each sum a separate
fp32 rounding, then a cast to bf16.  The oracle therefore evaluates those two
steps in IEEE fp32 (NumPy float32 elementwise arithmetic is correctly rounded),
in the one order the expressions name: for the sum over source streams, j
ascending.  Everything whose order the pages leave open -- the 20480-long
sums of squares, the projection, the RMSNorm mean, and the split/Sinkhorn
arithmetic -- is evaluated in float64 and rounded only where the reference
stores a narrower dtype (fp32 for mixes/pre/post/comb, bf16 for streams).

Layouts (row-major, n = batch*positions flattened):
  x      [n, hc, d]  bf16 bits (uint16)     residual streams
  delta  [n, d]      bf16 bits              sublayer output
  hc_fn  [(2+hc)*hc, hc*d] float32          projection weight (out x in)
  hc_base[(2+hc)*hc] float32, hc_scale [3] float32
  mixes  [n, (2+hc)*hc] float32: pre | post | comb (row-major j*hc+k)
  pre, post [n, hc] float32; comb [n, hc, hc] float32 with comb[t, j, k]:
  j = source stream (row), k = destination stream (column).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

# Tokens per block in the float64 steps, to bound temporaries.
_CHUNK = 256


# --------------------------------------------------------------------------
# dtype helpers (the oracle's own; nothing here is shared with the kernels)
# --------------------------------------------------------------------------
def f32(a) -> np.ndarray:
    """Round to nearest-even float32."""
    return np.asarray(a, dtype=F64).astype(F32)


def f32_to_bf16(a32) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN."""
    u = np.ascontiguousarray(np.asarray(a32, dtype=F32)).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if is_nan.any():
        r = np.where(is_nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), r)
    return r


def bf16_to_f32(b) -> np.ndarray:
    """bf16 bits -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def to_bf16(a64) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE): the value a fp32 computation
    would hold, cast to the stream dtype."""
    return f32_to_bf16(f32(a64))


def _eps32(eps: float) -> float:
    """An epsilon as the kernels and the reference hold it: an fp32 scalar."""
    return float(F32(eps))


# --------------------------------------------------------------------------
# hc_post -- "Write the streams" (stream-update equation) and
#            "Source layer, pairs pooled" (code panel, Block.hc_post)
# --------------------------------------------------------------------------
def hc_post(delta: np.ndarray, x: np.ndarray, post: np.ndarray, comb: np.ndarray) -> np.ndarray:
    """X'[t,k,i] = post[t,k] * delta[t,i] + sum_j comb[t,j,k] * X[t,j,i], cast to bf16.

    Argument order follows the pages: the sublayer output first, the residual
    streams second.  Output stream k reads column k of comb.  Arithmetic: the
    post product, each comb product, the running sum over j = 0..hc-1 and the
    final add are each one fp32 rounding; the result is cast to bf16.
    """
    x = np.asarray(x, dtype=np.uint16)
    n, hc, d = x.shape
    assert delta.shape == (n, d) and post.shape == (n, hc) and comb.shape == (n, hc, hc)
    X = bf16_to_f32(x)
    D = bf16_to_f32(delta)
    post = np.asarray(post, dtype=F32)
    comb = np.asarray(comb, dtype=F32)
    out = np.empty((n, hc, d), dtype=np.uint16)
    for k in range(hc):
        a = post[:, k, None] * D                       # fp32 product
        s = comb[:, 0, k, None] * X[:, 0]              # fp32 product
        for j in range(1, hc):
            s = s + comb[:, j, k, None] * X[:, j]      # fp32 product, fp32 sum
        out[:, k] = f32_to_bf16(a + s)                 # fp32 sum, cast
    return out


# --------------------------------------------------------------------------
# hc_pre -- "Source layer, pairs pooled" (code panel, Block.hc_pre)
# --------------------------------------------------------------------------
def hc_pre(x: np.ndarray, pre_mix: np.ndarray) -> np.ndarray:
    """y[t,i] = sum_j pre_mix[t,j] * X[t,j,i], cast to bf16.

    Each product and the running sum over j = 0..hc-1 are fp32 roundings.
    """
    x = np.asarray(x, dtype=np.uint16)
    n, hc, d = x.shape
    assert pre_mix.shape == (n, hc)
    X = bf16_to_f32(x)
    p = np.asarray(pre_mix, dtype=F32)
    s = p[:, 0, None] * X[:, 0]
    for j in range(1, hc):
        s = s + p[:, j, None] * X[:, j]
    return f32_to_bf16(s)


# --------------------------------------------------------------------------
# hc_mixes -- "Source layer, pairs pooled" (code panel, Block.hc_mixes)
# --------------------------------------------------------------------------
def rms_statistic(x: np.ndarray, norm_eps: float) -> np.ndarray:
    """r[t] = 1 / sqrt(mean_c x[t,c]^2 + norm_eps) over the flattened hc*d row
    (flattening index j*d + i).  float64."""
    x = np.asarray(x, dtype=np.uint16)
    n, hc, d = x.shape
    eps = _eps32(norm_eps)
    r = np.empty(n, dtype=F64)
    for t0 in range(0, n, _CHUNK):
        v = bf16_to_f32(x[t0:t0 + _CHUNK]).reshape(-1, hc * d).astype(F64)
        r[t0:t0 + _CHUNK] = 1.0 / np.sqrt((v * v).sum(axis=1) / (hc * d) + eps)
    return r


def hc_mixes(x: np.ndarray, hc_fn: np.ndarray, norm_eps: float) -> np.ndarray:
    """mixes[t,q] = r[t] * sum_c hc_fn[q,c] * x[t,c], stored as fp32.

    The projection is the plain matrix product of the flattened fp64 row with
    the fp64 weight (``F.linear`` layout: weight is out x in).
    """
    x = np.asarray(x, dtype=np.uint16)
    n, hc, d = x.shape
    W = np.asarray(hc_fn, dtype=F32).astype(F64)
    assert W.shape[1] == hc * d
    r = rms_statistic(x, norm_eps)
    out = np.empty((n, W.shape[0]), dtype=F32)
    for t0 in range(0, n, _CHUNK):
        v = bf16_to_f32(x[t0:t0 + _CHUNK]).reshape(-1, hc * d).astype(F64)
        out[t0:t0 + _CHUNK] = f32((v @ W.T) * r[t0:t0 + _CHUNK, None])
    return out


# --------------------------------------------------------------------------
# split + Sinkhorn -- "Reading weights" (reading-weight equation; code panel
#                     with the split/Sinkhorn kernel and its wrapper)
# --------------------------------------------------------------------------
def sigmoid(u: np.ndarray) -> np.ndarray:
    """Logistic function 1/(1+e^-u), evaluated without overflow."""
    u = np.asarray(u, dtype=F64)
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def split_pre_post(mixes: np.ndarray, hc_scale: np.ndarray, hc_base: np.ndarray,
                   hc: int = 4, eps: float = 1e-6):
    """pre[t,j]  = sigmoid(scale[0] * m[t,j] + base[j]) + eps,
    post[t,j] = 2 * sigmoid(scale[1] * m[t,hc+j] + base[hc+j]).   float64."""
    m = np.asarray(mixes, dtype=F32).astype(F64)
    s = np.asarray(hc_scale, dtype=F32).astype(F64)
    b = np.asarray(hc_base, dtype=F32).astype(F64)
    pre = sigmoid(m[:, :hc] * s[0] + b[:hc]) + _eps32(eps)
    post = 2.0 * sigmoid(m[:, hc:2 * hc] * s[1] + b[hc:2 * hc])
    return pre, post


def comb_logits(mixes: np.ndarray, hc_scale: np.ndarray, hc_base: np.ndarray, hc: int = 4) -> np.ndarray:
    """L[t,j,k] = scale[2] * m[t, 2hc + j*hc + k] + base[2hc + j*hc + k].  float64."""
    m = np.asarray(mixes, dtype=F32).astype(F64)
    s = np.asarray(hc_scale, dtype=F32).astype(F64)
    b = np.asarray(hc_base, dtype=F32).astype(F64)
    n = m.shape[0]
    return (m[:, 2 * hc:] * s[2] + b[2 * hc:]).reshape(n, hc, hc)


def sinkhorn(L: np.ndarray, iters: int = 20, eps: float = 1e-6) -> np.ndarray:
    """The comb matrix from its logits, float64.

    Steps, in the kernel's order: softmax along each row (over k) plus eps;
    divide each column by (its sum + eps); then iters-1 rounds of: divide each
    row by (its sum + eps), divide each column by (its sum + eps).  The loop
    runs a fixed count; it is not iterated to convergence.
    """
    if iters < 1:
        raise ValueError("sinkhorn needs iters >= 1")
    e = _eps32(eps)
    A = np.exp(L - L.max(axis=-1, keepdims=True))
    A = A / A.sum(axis=-1, keepdims=True) + e
    A = A / (A.sum(axis=-2, keepdims=True) + e)
    for _ in range(iters - 1):
        A = A / (A.sum(axis=-1, keepdims=True) + e)
        A = A / (A.sum(axis=-2, keepdims=True) + e)
    return A


def hc_split_sinkhorn(mixes: np.ndarray, hc_scale: np.ndarray, hc_base: np.ndarray,
                      hc: int = 4, iters: int = 20, eps: float = 1e-6):
    """(pre [n,hc], post [n,hc], comb [n,hc,hc]) as fp32, computed in float64
    from the fp32 mixes."""
    pre, post = split_pre_post(mixes, hc_scale, hc_base, hc, eps)
    comb = sinkhorn(comb_logits(mixes, hc_scale, hc_base, hc), iters, eps)
    return f32(pre), f32(post), f32(comb)


# --------------------------------------------------------------------------
# RMSNorm -- "Final RMSNorm" (equation and the RMSNorm class)
# --------------------------------------------------------------------------
def rms_norm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """z[t,i] = gamma[i] * y[t,i] / sqrt(mean_i y[t,i]^2 + eps), cast to bf16.
    float64 arithmetic on the bf16 input."""
    y = np.asarray(y, dtype=np.uint16)
    v = bf16_to_f32(y).astype(F64)
    g = np.asarray(gamma, dtype=F32).astype(F64)
    r = 1.0 / np.sqrt((v * v).mean(axis=-1, keepdims=True) + _eps32(eps))
    return to_bf16(g * (v * r))


# --------------------------------------------------------------------------
# Stack entry and the MTP tap -- "Final RMSNorm" (the model driver,
# Transformer.forward)
# --------------------------------------------------------------------------
def expand_streams(h: np.ndarray, hc: int = 4) -> np.ndarray:
    """The driver's entry: the embedding h [n, d] (bf16 bits) copied into hc
    identical streams, [n, hc, d]."""
    h = np.asarray(h, dtype=np.uint16)
    return np.repeat(h[:, None, :], hc, axis=1)


def stream_mean(x: np.ndarray) -> np.ndarray:
    """The MTP head's tap at its target layers: the mean over the hc streams of
    a block's input, [n, d], a bf16 tensor mean.  Reading: the exact mean
    (the sum of hc bf16 values and the division by hc are exact in float64),
    rounded once to bf16."""
    v = bf16_to_f32(x).astype(F64)
    return to_bf16(v.mean(axis=1))


# --------------------------------------------------------------------------
# Compositions -- "Source layer, pairs pooled" (Block.forward) and
#                 "Final RMSNorm" (the model driver)
# --------------------------------------------------------------------------
def boundary(*, x, delta=None, post_in=None, comb_in=None, pre_in=None,
             hc_fn=None, hc_base=None, hc_scale=None, gamma=None,
             iters=20, hc_eps=1e-6, norm_eps=1e-6, rms_eps=1e-6, hc=None,
             x_expanded=False, want_mean=False):
    """One sublayer boundary: write the streams with the previous sublayer's
    (post, comb) and output delta, derive this boundary's (pre, post, comb)
    from the new streams, read the new streams into the next sublayer input.

    * delta None   -> block entry: no write, the new streams are x itself.
    * hc_fn None   -> stack exit: no mixes are derived.
    * pre_in given -> the streams are read with pre_in (the reading mix the
                      previous boundary produced: the lag ``Block.forward``
                      shows); pre_in None -> read with the pre just derived.
    * gamma given  -> the read row is RMS-normalised (rms_eps) before return.
    * x_expanded   -> x is [n, d]: the streams are hc copies of it (the
                      driver's entry expansion; hc defaults to 4).  Otherwise
                      hc is the stream count of x.
    * want_mean    -> also the MTP tap of the new streams (stream_mean).

    Returns a dict with x_out (bf16 bits, None on entry), y (bf16 bits:
    normalised if gamma was given), mixes/pre/post/comb (None on exit), and
    x_mean (or None).
    """
    x = np.asarray(x, dtype=np.uint16)
    if x_expanded:
        x = expand_streams(x, 4 if hc is None else hc)
    hc = x.shape[1]
    xp = x if delta is None else hc_post(delta, x, post_in, comb_in)
    out = {"x_out": None if delta is None else xp,
           "mixes": None, "pre": None, "post": None, "comb": None}
    if hc_fn is not None:
        m = hc_mixes(xp, hc_fn, norm_eps)
        pre, post, comb = hc_split_sinkhorn(m, hc_scale, hc_base, hc, iters, hc_eps)
        out.update(mixes=m, pre=pre, post=post, comb=comb)
    p = pre_in if pre_in is not None else out["pre"]
    if p is None:
        raise ValueError("no reading mix: give pre_in or hc_fn")
    y = hc_pre(xp, p)
    out["y"] = rms_norm(y, gamma, rms_eps) if gamma is not None else y
    out["x_mean"] = stream_mean(xp) if want_mean else None
    return out


def block(*, x, pre_in, delta_attn, delta_ffn, attn, ffn, iters=20, hc_eps=1e-6,
          norm_eps=1e-6):
    """One block's glue with given sublayer outputs ("Source layer, pairs
    pooled", Block.forward): attention reads with the incoming mix and writes
    with its own (post, comb); the feed-forward reads with the attention's pre
    and writes with its own; the block hands on the feed-forward's pre.
    ``attn``/``ffn`` are (hc_fn, hc_base, hc_scale) triples.  No norms."""
    e = boundary(x=x, pre_in=pre_in, hc_fn=attn[0], hc_base=attn[1], hc_scale=attn[2],
                 iters=iters, hc_eps=hc_eps, norm_eps=norm_eps)
    b = boundary(x=x, delta=delta_attn, post_in=e["post"], comb_in=e["comb"], pre_in=e["pre"],
                 hc_fn=ffn[0], hc_base=ffn[1], hc_scale=ffn[2],
                 iters=iters, hc_eps=hc_eps, norm_eps=norm_eps)
    x_final = hc_post(delta_ffn, b["x_out"], b["post"], b["comb"])
    return {"attn": e, "ffn": b, "x_out": x_final, "pre_out": b["pre"]}


def stack_step(*, s, x, delta, post_in, comb_in, pre_in, params, gammas,
               iters=20, hc_eps=1e-6, norm_eps=1e-6, rms_eps=1e-6):
    """Sublayer s of the HC stack with the stand-in sublayer (its output is
    the RMS-normalised read row).  s == 0 is the entry (no write)."""
    fn, base, scale = params[s]
    return boundary(x=x, delta=None if s == 0 else delta, post_in=post_in, comb_in=comb_in,
                    pre_in=pre_in, hc_fn=fn, hc_base=base, hc_scale=scale, gamma=gammas[s],
                    iters=iters, hc_eps=hc_eps, norm_eps=norm_eps, rms_eps=rms_eps)


def stack(*, h, params, gammas, gamma_final, pre0=0.25, iters=20, hc_eps=1e-6,
          norm_eps=1e-6, rms_eps=1e-6, final_eps=1e-20, record=None):
    """The HC stack of the model driver ("Final RMSNorm", Transformer.forward)
    with every sublayer replaced by the stand-in delta = RMSNorm_gamma(read row).

    h [n, d] bf16 bits is copied to hc streams; the first reading mix is pre0
    per stream; len(params) sublayers follow; the stack ends with a final write,
    a final read with the last sublayer's pre and a final RMSNorm (final_eps).
    ``record``, if a list, receives (x, delta, pre, post, comb) per sublayer.
    """
    hc = 4
    h = np.asarray(h, dtype=np.uint16)
    n, d = h.shape
    x = np.repeat(h[:, None, :], hc, axis=1)
    pre_in = np.full((n, hc), pre0, dtype=F32)
    delta = post = comb = None
    for s in range(len(params)):
        o = stack_step(s=s, x=x, delta=delta, post_in=post, comb_in=comb, pre_in=pre_in,
                       params=params, gammas=gammas, iters=iters, hc_eps=hc_eps,
                       norm_eps=norm_eps, rms_eps=rms_eps)
        if s > 0:
            x = o["x_out"]
        if record is not None:
            record.append((x, o["y"], o["pre"], o["post"], o["comb"]))
        delta, post, comb, pre_in = o["y"], o["post"], o["comb"], o["pre"]
    x = hc_post(delta, x, post, comb)
    y = hc_pre(x, pre_in)
    return {"x_out": x, "z": rms_norm(y, gamma_final, final_eps)}
