"""Test-side helpers: numpy <-> GPU tensors and the parity assertions.

Inputs come from transformer_hyper_connection_amd.synth (seeded); expected
values come from the CPU oracle; nothing here computes either side."""
from __future__ import annotations

import numpy as np
import torch

from tests import numerics as N

DEV = "cuda:0"


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def say(msg: str) -> None:
    print(msg, flush=True)


def assert_bits_equal(got, ref, what):
    got = np.asarray(got); ref = np.asarray(ref)
    bad = got != ref
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} bf16 values differ, first at "
                             f"{idx.tolist()}: got {got[tuple(idx[0])]:#06x} ref {ref[tuple(idx[0])]:#06x}")


def assert_bf16_close(got, ref, what, ulps=1, floor=None):
    ok = N.bf16_within_ulps(got, ref, ulps, floor)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        g = N.bits_to_f64(got)[tuple(idx[0])]; r = N.bits_to_f64(ref)[tuple(idx[0])]
        raise AssertionError(f"{what}: {(~ok).sum()} of {ok.size} beyond {ulps} ulp, first at "
                             f"{idx.tolist()}: got {g!r} ref {r!r}")


def assert_mixes_close(got, ref, what="mixes"):
    e = N.floored_rel_err(got, ref)
    assert e.max() <= N.MIXES_REL_TOL, f"{what}: floored relative error {e.max():.3e} > {N.MIXES_REL_TOL}"


def assert_coef_close(got, ref, what):
    e = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert e.max() <= N.COEF_ABS_TOL, f"{what}: absolute error {e.max():.3e} > {N.COEF_ABS_TOL}"


def write_floor(delta_bits, x_bits, tol=N.COEF_ABS_TOL):
    """Per-element allowance for X' when the write coefficients of the two
    sides differ by up to ``tol``: tol * (|delta| + sum_j |X_j|)."""
    D = np.abs(N.bits_to_f64(delta_bits))
    X = np.abs(N.bits_to_f64(x_bits)).sum(axis=-2)
    return (tol * (D + X))[:, None, :] * 1.0001


def assert_workspace_clean(got):
    """The error mask of the call's workspace (hc_workspace_status) is zero: no
    wait for another workgroup's words ran into its bound."""
    from transformer_hyper_connection_amd import hc as H
    ws = got.get("workspace") if isinstance(got, dict) else got
    if ws is None:
        return
    mask = H.workspace_status(ws)
    assert mask == 0, f"workspace error mask {mask:#x}"
