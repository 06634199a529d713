"""C-ABI contract of libhc on the CPU: the library loads, exports every symbol
include/hc.h declares, the ctypes mirror of hc_boundary_args matches the C
layout, and argument validation returns its status codes before any HIP call
(fake, never-dereferenced pointers are used; nothing is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

from transformer_hyper_connection_amd import hc as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")

P = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004        # misaligned fake address
S = None             # null stream


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(hc_[a-z_0-9]+)\s*\(", src)) - {"hc_boundary_args"}


@pytest.fixture(scope="module")
def L():
    return H.lib()


def test_library_exports_every_header_symbol(L):
    funcs = header_functions()
    assert funcs == set(H.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", H.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (hc_\w+)", out))
    assert funcs <= exported, funcs - exported
    for f in funcs:
        assert hasattr(L, f)


def test_boundary_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in H.BoundaryArgs._fields_]
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "hc.h"\nint main(void){\n'
        'printf("%zu\\n", sizeof(hc_boundary_args));\n'
        + "".join(f'printf("%zu\\n", offsetof(hc_boundary_args, {f}));\n' for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(H.BoundaryArgs)
    for f, off in zip(fields, vals[1:]):
        assert getattr(H.BoundaryArgs, f).offset == off, f


def test_header_compiles_as_cxx(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text('#include "hc.h"\nint main(){ return hc_version() > 0 ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.dirname(HEADER), str(src)],
                   check=True)


def test_strerror_and_version(L):
    assert L.hc_version() >= 100
    for code in (0, -1, -2, -3, -4, 7):
        assert L.hc_strerror(code)


def test_packed_and_workspace_bytes(L):
    # 72 split rows + 8 zero rows, bf16, for the four stream blocks and their sum
    assert L.hc_fn_packed_bytes(4, 5120) == 80 * 5 * 5120 * 2
    assert L.hc_fn_packed_bytes(3, 5120) == 0
    assert L.hc_fn_packed_bytes(4, 100) == 0
    assert L.hc_fn_packed_bytes(4, 5184) == 80 * 5 * 5184 * 2
    assert L.hc_fn_packed_bytes(4, 32832) == 0
    assert L.hc_workspace_bytes(0, 4, 5120) == 0
    assert L.hc_workspace_bytes(4096, 3, 5120) == 0
    w = L.hc_workspace_bytes(4096, 4, 5120)
    # 8 KB control block; exchange words: 256 groups x 64 tokens x 26 tagged 8-byte words; then the
    # per-slice records: 64 tiles of 64 tokens x 36 floats x the larger slice count of the two first
    # kernels (the stream kernel's 64 tiles take 4 slices, the projection kernel's 32 workgroups of
    # 128 tokens 8)
    fixed = 8192 + 256 * 64 * 26 * 8
    assert w == fixed + 64 * 8 * 64 * 36 * 4
    # n = 128: 2 tiles x 40 slices
    assert L.hc_workspace_bytes(128, 4, 5120) == fixed + 2 * 40 * 64 * 36 * 4
    assert L.hc_boundary_workspace_bytes(4096, 4, 5120) == w
    assert L.hc_workspace_bytes(4097, 4, 5120) > w
    assert L.hc_workspace_bytes(64, 4, 320) == fixed + 1 * 5 * 64 * 36 * 4


def _layout(L, n, hc, d):
    r = (ctypes.c_size_t * 6)()
    assert L.hc_workspace_layout(n, hc, d, r) == H.HC_OK
    return list(r)


def test_workspace_layout_regions_never_overlap(L):
    """Every shape's workspace: the control block and the exchange words sit
    at one place and size whatever (n, hc, d), so no call's per-slice sums (or
    any other region) can lie on another call's persistent words; the regions
    are disjoint and end at hc_workspace_bytes."""
    base = _layout(L, 1, 4, 64)[:4]
    assert base[0] == 0 and base[1] == 8192
    # the exchange words: 256 groups x 64 tokens x 26 words
    assert base[3] >= 256 * 64 * 26 * 8
    ns = (1, 17, 128, 129, 2048, 3000, 4096, 4097, 32768)
    for hc in (2, 4, 8):
        for d in range(64, 32768 + 1, 64):
            for n in ns if d % 1024 == 0 else (1, 4096):
                r = _layout(L, n, hc, d)
                assert r[:4] == base, (n, hc, d)
                spans = sorted((r[i], r[i] + r[i + 1]) for i in range(0, 6, 2))
                for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
                    assert a1 <= b0, (n, hc, d, spans)
                assert r[4] + r[5] == L.hc_workspace_bytes(n, hc, d), (n, hc, d)
    bad = (ctypes.c_size_t * 6)()
    assert L.hc_workspace_layout(16, 3, 5120, bad) == H.HC_ENOTSUP
    assert L.hc_workspace_layout(-1, 4, 5120, bad) == H.HC_EINVAL
    assert L.hc_workspace_layout(16, 4, 5120, None) == H.HC_EINVAL


def test_workspace_status_validates(L):
    mask = ctypes.c_uint32(7)
    assert L.hc_workspace_status(None, 1 << 20, 0, ctypes.byref(mask), S) == H.HC_EINVAL
    assert L.hc_workspace_status(MIS, 1 << 20, 0, ctypes.byref(mask), S) == H.HC_EINVAL
    assert L.hc_workspace_status(P, 4096, 0, ctypes.byref(mask), S) == H.HC_EINVAL      # smaller than the control block
    assert L.hc_workspace_status(P, 1 << 20, 0, None, S) == H.HC_EINVAL


def test_packed_and_workspace_bytes_other_hc(L):
    # hc = 2 and 8: per 32-feature step, 3 terms x ceil(mix/16) tiles of 1 KB (mix = 8 -> 3, 80 -> 15)
    assert L.hc_fn_packed_bytes(2, 5120) == (2 * 5120 // 32) * 3 * 1024
    assert L.hc_fn_packed_bytes(8, 4096) == (8 * 4096 // 32) * 15 * 1024
    assert L.hc_fn_packed_bytes(8, 100) == 0
    assert L.hc_fn_packed_bytes(16, 4096) == 0
    # records [S][n][recw] after the fixed regions; S is the largest divisor of hc*d/64 with at most
    # ~512 workgroups of 128 tokens, 64 at most; recw = mix + 1 rounded up to 4 floats (12 at hc = 2,
    # 84 at hc = 8)
    fixed = 8192 + 256 * 64 * 26 * 8
    assert L.hc_workspace_bytes(4096, 8, 5120) == fixed + 16 * 4096 * 84 * 4

def test_null_misaligned_negative(L):
    assert L.hc_pre(None, P, 16, 4, 64, P, S) == H.HC_EINVAL
    assert b"x" in L.hc_last_error()
    assert L.hc_pre(MIS, P, 16, 4, 64, P, S) == H.HC_EINVAL
    assert b"aligned" in L.hc_last_error()
    assert L.hc_pre(P, P, -1, 4, 64, P, S) == H.HC_EINVAL
    assert L.hc_post(P, P, P, P, 16, 4, 64, P, S) == H.HC_EINVAL           # x_out aliases x
    W = (P, 1 << 30)
    assert L.hc_mixes(P, P, 16, 4, 64, 1e-6, None, None, None, 20, 1e-6, None, None, None, *W, S) == H.HC_EINVAL
    assert L.hc_mixes(P, P, 16, 4, 64, 1e-6, None, P, P, 0, 1e-6, P, P, P, *W, S) == H.HC_EINVAL  # iters 0
    assert L.hc_mixes(P, P, 16, 4, 64, 1e-6, None, P, P, 20, 1e-6, P, None, P, *W, S) == H.HC_EINVAL  # partial split
    assert L.hc_split_sinkhorn(P, P, P, 16, 4, 0, 1e-6, P, P, P, S) == H.HC_EINVAL
    assert L.hc_split_sinkhorn(P, P, P, 16, 3, 20, 1e-6, P, P, P, S) == H.HC_ENOTSUP
    # hc = 8 keeps per-slice records in the workspace: it must hold them
    assert L.hc_mixes(P, P, 16, 8, 64, 1e-6, P, None, None, 20, 1e-6, None, None, None, P, 4096, S) == H.HC_EINVAL
    assert b"workspace" in L.hc_last_error()
    assert L.hc_mixes(P, P, 16, 8, 64, 1e-6, None, P, P, 20, 1e-6, P, P, P, MIS, 1 << 30, S) == H.HC_EINVAL
    assert L.hc_split_sinkhorn(P, P, None, 16, 4, 20, 1e-6, P, P, P, S) == H.HC_EINVAL


def test_zero_tokens_is_a_no_op(L):
    assert L.hc_pre(P, P, 0, 4, 64, P, S) == H.HC_OK
    assert L.hc_post(P, P + 16, P, P, 0, 4, 64, P + 32, S) == H.HC_OK
    assert L.hc_mixes(P, P, 0, 4, 64, 1e-6, P, None, None, 20, 1e-6, None, None, None, None, 0, S) == H.HC_OK
    assert L.hc_split_sinkhorn(P, P, P, 0, 4, 20, 1e-6, P, P, P, S) == H.HC_OK


def _args(**kw):
    a = H.BoundaryArgs()
    a.struct_size = ctypes.sizeof(H.BoundaryArgs)
    a.hc, a.d, a.iters, a.n = 4, 64, 20, 16
    a.hc_eps = a.norm_eps = a.rms_eps = 1e-6
    # the streams far apart (no overlap at the test shapes), the small tensors after them
    a.x, a.y_out = P, P + 0x400000
    a.delta, a.x_out = P + 0x800000, P + 0xC00000
    a.post_in, a.comb_in = P + 0x1000000, P + 0x1001000
    a.pre_in = P + 0x1002000
    a.fn_packed, a.hc_base, a.hc_scale = P + 0x1003000, P + 0x1004000, P + 0x1005000
    a.pre_out, a.post_out, a.comb_out = P + 0x1006000, P + 0x1007000, P + 0x1008000
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_boundary_validation(L):
    call = lambda a: L.hc_boundary(ctypes.byref(a), S)  # noqa: E731
    assert L.hc_boundary(None, S) == H.HC_EINVAL
    assert call(_args(struct_size=8)) == H.HC_EINVAL
    assert call(_args(hc=3)) == H.HC_ENOTSUP
    assert call(_args(x=None)) == H.HC_EINVAL
    assert call(_args(y_out=None)) == H.HC_EINVAL
    assert call(_args(post_in=None)) == H.HC_EINVAL           # delta given, post_in missing
    assert call(_args(x_out=P)) == H.HC_EINVAL                # x_out aliases x
    assert call(_args(pre_out=None)) == H.HC_EINVAL           # mixes derived, outputs missing
    assert call(_args(fn_packed=None, pre_in=None)) == H.HC_EINVAL   # nothing to read with
    assert call(_args(iters=0)) == H.HC_EINVAL
    assert call(_args(gamma=MIS)) == H.HC_EINVAL
    assert call(_args(n=0)) == H.HC_OK
    assert call(_args(n=0, delta=None, post_in=None, comb_in=None, x_out=None)) == H.HC_OK
    assert call(_args(d=10304, gamma=P + 0xD00)) == H.HC_ENOTSUP   # RMSNorm row too long
    # flags: the expanded-x bit and the two-launch bit; every other bit is rejected, the
    # bits of the schedules this library no longer has included
    XE, TL = H.HC_BOUNDARY_X_EXPANDED, H.HC_BOUNDARY_TWO_LAUNCH
    for bad in (1, 2, 8, 32, 1 << 31):
        assert call(_args(flags=bad)) == H.HC_EINVAL
    assert call(_args(flags=XE | TL, n=0)) == H.HC_OK
    assert call(_args(x_mean_out=MIS)) == H.HC_EINVAL                    # misaligned stream-mean output
    # outputs overlapping the streams they are formed from, or each other, by any range
    n, d = 16, 64
    xb, rb = n * 4 * d * 2, n * d * 2                                   # x / x_out bytes, delta / y bytes
    X0, XO, Y0, D0 = P, P + 0x100000, P + 0x200000, P + 0x300000
    ok = dict(x=X0, x_out=XO, y_out=Y0, delta=D0)
    assert call(_args(**ok, n=0)) == H.HC_OK
    assert call(_args(**{**ok, "x_out": X0 + xb - 16})) == H.HC_EINVAL   # x_out's head on x's tail
    assert call(_args(**{**ok, "x_out": X0 - xb + 16})) == H.HC_EINVAL   # x_out's tail on x's head
    assert call(_args(**{**ok, "x_out": D0 + 16})) == H.HC_EINVAL        # x_out on delta
    assert call(_args(**{**ok, "y_out": X0 + 32})) == H.HC_EINVAL        # y_out inside x
    assert call(_args(**{**ok, "y_out": XO + xb - 16})) == H.HC_EINVAL   # y_out on x_out's tail
    assert call(_args(**{**ok, "y_out": D0 + rb - 16})) == H.HC_EINVAL   # y_out on delta
    assert call(_args(**{**ok, "x_mean_out": Y0 + 16})) == H.HC_EINVAL   # the stream mean on y_out
    assert call(_args(**{**ok, "x_out": X0 + xb})) in (H.HC_ENODEV, H.HC_OK)      # adjacent is fine
    assert call(_args(**{**ok, "y_out": XO + xb})) in (H.HC_ENODEV, H.HC_OK)
    # expanded x is [n, d]: an x_out right after it does not overlap
    assert call(_args(**{**ok, "x_out": X0 + rb}, flags=XE)) in (H.HC_ENODEV, H.HC_OK)
    assert call(_args(**{**ok, "x_out": X0 + rb - 16}, flags=XE)) == H.HC_EINVAL
    # a caller of the struct without the trailing flags field (shorter struct_size) gets flags 0
    short = H.BoundaryArgs.flags.offset
    assert call(_args(struct_size=short, flags=1)) in (H.HC_ENODEV, H.HC_OK)
    # ... and without the trailing x_mean_out field, no stream mean
    assert call(_args(struct_size=H.BoundaryArgs.x_mean_out.offset, x_mean_out=MIS)) in (H.HC_ENODEV, H.HC_OK)
    assert call(_args(struct_size=short - 8)) == H.HC_EINVAL
    for half in (L.hc_boundary_begin, L.hc_boundary_end):          # the halves validate alike
        assert half(None, S) == H.HC_EINVAL
        assert half(ctypes.byref(_args(iters=0)), S) == H.HC_EINVAL
        assert half(ctypes.byref(_args(hc=3)), S) == H.HC_ENOTSUP
        assert half(ctypes.byref(_args(n=0)), S) == H.HC_OK


def test_no_device_reported_without_gpu(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert L.hc_pre(P, P + 0x400000, 16, 4, 64, P + 0x800000, S) == H.HC_ENODEV


def test_workspace_covers_the_parts_of_a_long_call(L):
    """A call beyond 4096 tokens may run as 4096-token parts and a rest: the
    workspace asked for its n covers the parts and any rest (whose slices can
    be more than the whole call's)."""
    for d in (1024, 2560, 5120, 10240):
        for n in list(range(4097, 4096 + 4097, 61)) + [8712, 32768 + 520]:
            w = L.hc_workspace_bytes(n, 4, d)
            assert w >= L.hc_workspace_bytes(4096, 4, d), (n, d)
            r = n % 4096
            if r:
                assert w >= L.hc_workspace_bytes(r, 4, d), (n, d, r)
