"""Seeded synthetic inputs for the HC glue workloads.

This module only draws random numbers and converts them to storage dtypes; it
holds none of the glue's arithmetic.  Both the test suite (which feeds the same
bytes to the GPU library and to the CPU oracle) and the benchmark use it.

Every tensor comes from its own PCG64 stream, seeded by
``SeedSequence([BASE_SEED, workload, tensor_id, block])``.  Token-major tensors
are drawn in blocks of ``BLOCK`` tokens, each block from its own stream, so any
token range can be regenerated without drawing the rest.  Draws are float64,
rounded to float32 (nearest-even) and, for bf16 tensors, to bf16
(nearest-even); bf16 tensors are returned as uint16 bit patterns.

Workloads (n = tokens, hc = 4 streams, d = 5120, 24 mix numbers; boundary_inputs
also draws the same distributions at hc = 2 or 8):
  "step"    n=32     one sublayer step (mixes, read, write)
  "decode"  n=128    one block's glue at decode, two parameter sets
  "prefill" n=4096   fused sublayer boundary
  "stress"  n=32768  fused boundary, channel-outlier streams
  "stack"   n=8192   80-sublayer stack with the stand-in sublayer
Distributions: streams and sublayer outputs N(0,1); projection weight
N(0, 0.02^2); offsets N(0, 0.1^2); scales U(0.5, 2); reading mix U(0,1);
given writing weights U(0,2); given comb columns Dirichlet(1,1,1,1) (each
column non-negative, summing to one); RMSNorm gains 1 + N(0, 0.1^2).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261202
BLOCK = 256
HC = 4
D = 5120
MIX = (2 + HC) * HC

WORKLOAD_IDS = {"step": 0, "decode": 1, "prefill": 2, "stress": 3, "stack": 4}
WORKLOAD_TOKENS = {"step": 32, "decode": 128, "prefill": 4096, "stress": 32768, "stack": 8192}


def _rng(workload: str, tensor: int, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([BASE_SEED, WORKLOAD_IDS[workload], tensor, block])
    return np.random.Generator(np.random.PCG64(ss))


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 bit pattern, both steps nearest-even."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32)).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _token_blocks(t0: int, t1: int):
    b = t0 // BLOCK
    while b * BLOCK < t1:
        yield b, max(t0, b * BLOCK), min(t1, (b + 1) * BLOCK)
        b += 1


def token_normal(workload: str, tensor: int, shape_per_token: tuple, t0: int, t1: int,
                 col_scale: np.ndarray | None = None) -> np.ndarray:
    """N(0,1) bf16 bits for tokens [t0, t1), shape [t1-t0, *shape_per_token].
    ``col_scale`` (float32, broadcast over the last axis) multiplies the fp32
    draw before the bf16 rounding."""
    per = int(np.prod(shape_per_token))
    out = np.empty((t1 - t0, per), dtype=np.uint16)
    for b, a, e in _token_blocks(t0, t1):
        g = _rng(workload, tensor, b)
        full = g.standard_normal((BLOCK, per))          # the whole block, always
        v = full[a - b * BLOCK:e - b * BLOCK]
        if col_scale is not None:
            v = (v.astype(np.float32).reshape(e - a, *shape_per_token) * col_scale).reshape(e - a, per)
        out[a - t0:e - t0] = f64_to_bf16_bits(v)
    return out.reshape(t1 - t0, *shape_per_token)


def token_uniform(workload: str, tensor: int, per_token: int, lo: float, hi: float,
                  t0: int, t1: int) -> np.ndarray:
    out = np.empty((t1 - t0, per_token), dtype=np.float32)
    for b, a, e in _token_blocks(t0, t1):
        full = _rng(workload, tensor, b).uniform(lo, hi, (BLOCK, per_token))
        out[a - t0:e - t0] = full[a - b * BLOCK:e - b * BLOCK].astype(np.float32)
    return out


def token_dirichlet_columns(workload: str, tensor: int, hc: int, t0: int, t1: int) -> np.ndarray:
    """[t1-t0, hc, hc] float32: every column (fixed k, over j) ~ Dirichlet(1,...,1)."""
    out = np.empty((t1 - t0, hc, hc), dtype=np.float32)
    for b, a, e in _token_blocks(t0, t1):
        full = _rng(workload, tensor, b).dirichlet(np.ones(hc), size=(BLOCK, hc))  # [t, k, j]
        out[a - t0:e - t0] = np.swapaxes(full[a - b * BLOCK:e - b * BLOCK], 1, 2).astype(np.float32)
    return out


def hc_params(workload: str, tensor: int, hc: int = HC, d: int = D):
    """(hc_fn [mix, hc*d], hc_base [mix], hc_scale [3]) float32."""
    mix = (2 + hc) * hc
    fn = (_rng(workload, tensor, 0).standard_normal((mix, hc * d)) * 0.02).astype(np.float32)
    base = (_rng(workload, tensor, 1).standard_normal(mix) * 0.1).astype(np.float32)
    scale = _rng(workload, tensor, 2).uniform(0.5, 2.0, 3).astype(np.float32)
    return fn, base, scale


def gamma(workload: str, tensor: int, d: int = D) -> np.ndarray:
    return (1.0 + _rng(workload, tensor, 0).standard_normal(d) * 0.1).astype(np.float32)


def outlier_columns(workload: str, tensor: int, d: int = D, frac: float = 0.01,
                    factor: float = 30.0) -> np.ndarray:
    """float32 [d] column multipliers: floor(frac*d) seeded columns get ``factor``."""
    cols = _rng(workload, tensor, 0).permutation(d)[: int(np.floor(frac * d))]
    s = np.ones(d, dtype=np.float32)
    s[cols] = factor
    return s


# Tensor ids per workload (stable: changing one changes every stored fixture).
T_X, T_DELTA, T_FN, T_PRE_IN, T_POST_IN, T_COMB_IN, T_GAMMA, T_OUTLIER, T_DELTA2, T_FN2 = range(10)


def boundary_inputs(workload: str, t0: int = 0, t1: int | None = None, d: int = D, hc: int = HC):
    """Inputs of one fused boundary call for tokens [t0, t1).

    Returns a dict: x [t,hc,d] u16, delta [t,d] u16, pre_in [t,hc], post_in
    [t,hc], comb_in [t,hc,hc], hc_fn/hc_base/hc_scale, gamma [d] (float32
    unless noted).  "stress" scales 1% of the feature columns of x by 30 (all
    streams).  hc other than 4 draws the same distributions at that width.
    """
    n = WORKLOAD_TOKENS[workload]
    t1 = n if t1 is None else t1
    col = outlier_columns(workload, T_OUTLIER, d) if workload == "stress" else None
    fn, base, scale = hc_params(workload, T_FN, hc, d)
    return {
        "x": token_normal(workload, T_X, (hc, d), t0, t1, col_scale=col),
        "delta": token_normal(workload, T_DELTA, (d,), t0, t1),
        "pre_in": token_uniform(workload, T_PRE_IN, hc, 0.0, 1.0, t0, t1),
        "post_in": token_uniform(workload, T_POST_IN, hc, 0.0, 2.0, t0, t1),
        "comb_in": token_dirichlet_columns(workload, T_COMB_IN, hc, t0, t1),
        "hc_fn": fn, "hc_base": base, "hc_scale": scale,
        "gamma": gamma(workload, T_GAMMA, d),
    }


def block_inputs(t0: int = 0, t1: int | None = None, d: int = D):
    """Decode block glue ("decode"): streams, incoming reading mix, the two
    given sublayer outputs and the attention / feed-forward parameter sets."""
    w = "decode"
    n = WORKLOAD_TOKENS[w]
    t1 = n if t1 is None else t1
    return {
        "x": token_normal(w, T_X, (HC, d), t0, t1),
        "pre_in": token_uniform(w, T_PRE_IN, HC, 0.0, 1.0, t0, t1),
        "delta_attn": token_normal(w, T_DELTA, (d,), t0, t1),
        "delta_ffn": token_normal(w, T_DELTA2, (d,), t0, t1),
        "attn": hc_params(w, T_FN, HC, d),
        "ffn": hc_params(w, T_FN2, HC, d),
    }


def step_inputs(d: int = D):
    """One sublayer step ("step", n=32): streams, sublayer output, one
    parameter set and the incoming reading mix."""
    w = "step"
    n = WORKLOAD_TOKENS[w]
    fn, base, scale = hc_params(w, T_FN, HC, d)
    return {
        "x": token_normal(w, T_X, (HC, d), 0, n),
        "delta": token_normal(w, T_DELTA, (d,), 0, n),
        "pre_in": token_uniform(w, T_PRE_IN, HC, 0.0, 1.0, 0, n),
        "hc_fn": fn, "hc_base": base, "hc_scale": scale,
    }


def stack_inputs(n_sublayers: int = 80, t0: int = 0, t1: int | None = None, d: int = D):
    """HC stack ("stack"): token embedding [t, d] u16, per-sublayer parameter
    sets and gains, and the final gain."""
    w = "stack"
    n = WORKLOAD_TOKENS[w]
    t1 = n if t1 is None else t1
    params = [hc_params(w, 100 + s, HC, d) for s in range(n_sublayers)]
    gammas = [gamma(w, 1000 + s, d) for s in range(n_sublayers)]
    return {
        "h": token_normal(w, T_X, (d,), t0, t1),
        "params": params, "gammas": gammas, "gamma_final": gamma(w, 999, d),
    }
