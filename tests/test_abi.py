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
    assert L.hc_fn_packed_bytes(4, 5120) == 80 * 4 * 5120 * 2  # 72 split rows + 8 zero rows, bf16
    assert L.hc_fn_packed_bytes(3, 5120) == 0
    assert L.hc_fn_packed_bytes(4, 100) == 0
    assert L.hc_fn_packed_bytes(4, 5184) == 80 * 4 * 5184 * 2
    assert L.hc_fn_packed_bytes(4, 32832) == 0
    assert L.hc_workspace_bytes(0, 4, 5120) == 0
    assert L.hc_workspace_bytes(4096, 3, 5120) == 0
    w = L.hc_workspace_bytes(4096, 4, 5120)
    # 8 KB control block; decode region (fixed for d): 256 B of arrival words + 8 tiles x 20 slices
    # x 16 tokens x 25 tagged 8-byte words; slice-resident ring (d = 5120 only): 8 XCDs x 16 slots
    # x 32 slices x 16 tokens x 48 tagged record words (36 used), and 8 XCDs x 16 slots x 16 tokens x 8
    # read-coefficient words; single-launch records: 256 tiles of
    # 16 tokens x 10 slices x 34 tagged words; two-launch records: 64 tiles of 64 tokens x 4 slices
    # x 36 floats
    decode = 256 + 8 * 20 * 16 * 25 * 8
    ring = 8 * 16 * 32 * 16 * 48 * 8 + 8 * 16 * 16 * 8 * 8
    assert w == 8192 + decode + ring + 256 * 10 * 16 * 34 * 8 + 64 * 4 * 64 * 36 * 4
    # n = 128: 8 single-launch tiles; two-launch: 2 tiles x 40 slices
    assert L.hc_workspace_bytes(128, 4, 5120) == 8192 + decode + ring + 8 * 10 * 16 * 34 * 8 + 2 * 40 * 64 * 36 * 4
    assert L.hc_boundary_workspace_bytes(4096, 4, 5120) == w
    assert L.hc_workspace_bytes(4097, 4, 5120) > w
    # widths the single launch does not take (d % 512 != 0): control block + two-launch records only
    assert L.hc_workspace_bytes(64, 4, 320) == 8192 + 1 * 5 * 64 * 36 * 4


def test_packed_and_workspace_bytes_other_hc(L):
    # hc = 2 and 8: per 32-feature step, 3 terms x ceil(mix/16) tiles of 1 KB (mix = 8 -> 3, 80 -> 15)
    assert L.hc_fn_packed_bytes(2, 5120) == (2 * 5120 // 32) * 3 * 1024
    assert L.hc_fn_packed_bytes(8, 4096) == (8 * 4096 // 32) * 15 * 1024
    assert L.hc_fn_packed_bytes(8, 100) == 0
    assert L.hc_fn_packed_bytes(16, 4096) == 0
    # records [S][n][recw] after the hc = 4 control block and decode region of the same d; S is the
    # largest divisor of hc*d/64 with at most ~512 workgroups of 128 tokens, 64 at most; recw = mix + 1
    # rounded up to 4 floats (12 at hc = 2, 84 at hc = 8)
    decode = 256 + 8 * 20 * 16 * 25 * 8
    ring = 8 * 16 * 32 * 16 * 48 * 8 + 8 * 16 * 16 * 8 * 8   # slice-resident ring at d = 5120
    assert L.hc_workspace_bytes(4096, 8, 5120) == 8192 + decode + ring + 16 * 4096 * 84 * 4
    assert L.hc_workspace_bytes(100, 2, 320) == 8192 + 10 * 100 * 12 * 4     # 10 chunks of 64: S = 10
    assert L.hc_workspace_bytes(40, 8, 1024) == 8192 + (256 + 8 * 4 * 16 * 25 * 8) + 64 * 40 * 84 * 4
    assert L.hc_workspace_bytes(0, 8, 5120) == 0
    assert L.hc_boundary_workspace_bytes(7, 2, 1024) == L.hc_workspace_bytes(7, 2, 1024)


@pytest.mark.parametrize("hc,d,code", [(3, 5120, H.HC_ENOTSUP), (16, 5120, H.HC_ENOTSUP), (1, 64, H.HC_ENOTSUP),
                                       (4, 100, H.HC_ENOTSUP), (2, 100, H.HC_ENOTSUP), (8, 0, H.HC_ENOTSUP),
                                       (4, 0, H.HC_ENOTSUP), (4, 5152, H.HC_ENOTSUP),
                                       (4, 32832, H.HC_ENOTSUP)])
def test_unsupported_shapes(L, hc, d, code):
    assert L.hc_pre(P, P, 16, hc, d, P, S) == code
    assert L.hc_post(P, P, P, P, 16, hc, d, P, S) == code
    assert L.hc_mixes(P, P, 16, hc, d, 1e-6, P, None, None, 20, 1e-6, None, None, None, P, 1 << 30, S) == code
    assert L.hc_fn_pack(P, hc, d, P, S) == code
    assert L.hc_last_error()


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
    a.x, a.y_out = P, P + 0x100
    a.delta, a.post_in, a.comb_in, a.x_out = P + 0x200, P + 0x300, P + 0x400, P + 0x500
    a.pre_in = P + 0x600
    a.fn_packed, a.hc_base, a.hc_scale = P + 0x700, P + 0x800, P + 0x900
    a.pre_out, a.post_out, a.comb_out = P + 0xA00, P + 0xB00, P + 0xC00
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
    # the single-launch schedule flag: unknown bits, shapes it does not take, no halves
    SL, XE = H.HC_BOUNDARY_SINGLE_LAUNCH, H.HC_BOUNDARY_X_EXPANDED
    assert call(_args(flags=16)) == H.HC_EINVAL
    assert call(_args(flags=SL | XE, d=1024)) == H.HC_ENOTSUP            # no expanded x in the single launch
    assert call(_args(flags=SL, d=1024, x_mean_out=P + 0xE00)) == H.HC_ENOTSUP   # nor the stream mean
    assert call(_args(x_mean_out=MIS)) == H.HC_EINVAL                    # misaligned stream-mean output
    assert call(_args(flags=SL)) == H.HC_ENOTSUP                  # d=64: not a multiple of 512
    assert call(_args(flags=SL, d=512)) == H.HC_ENOTSUP           # at least 1024
    assert call(_args(flags=SL, d=1024, fn_packed=None, pre_in=P + 0x600)) == H.HC_EINVAL   # needs the mixes
    assert call(_args(flags=SL, d=1024, hc=8)) == H.HC_ENOTSUP    # hc = 4 only
    assert L.hc_boundary_begin(ctypes.byref(_args(flags=SL, d=1024)), S) == H.HC_EINVAL
    # the slice-resident schedule: hc = 4, d = 5120, a write, the mixes, the fresh pre; one launch
    SR = H.HC_BOUNDARY_SLICE_RESIDENT
    assert call(_args(flags=SR | SL, d=5120, pre_in=None)) == H.HC_EINVAL        # one schedule at a time
    assert call(_args(flags=SR, d=1024, pre_in=None)) == H.HC_ENOTSUP            # d = 5120 only
    assert call(_args(flags=SR, d=5120, hc=8, pre_in=None)) == H.HC_ENOTSUP      # hc = 4 only
    assert call(_args(flags=SR, d=5120)) == H.HC_ENOTSUP                         # a given pre
    assert call(_args(flags=SR, d=5120, pre_in=None, delta=None, post_in=None, comb_in=None,
                      x_out=None)) == H.HC_ENOTSUP                               # a block entry
    assert call(_args(flags=SR, d=5120, pre_in=None, x_mean_out=P + 0xE00)) == H.HC_ENOTSUP
    assert call(_args(flags=SR | XE, d=5120, pre_in=None)) == H.HC_ENOTSUP
    assert L.hc_boundary_begin(ctypes.byref(_args(flags=SR, d=5120, pre_in=None)), S) == H.HC_EINVAL
    assert call(_args(flags=SR, d=5120, pre_in=None, n=0)) == H.HC_OK
    # a caller of the struct without the trailing flags field (shorter struct_size) gets flags 0
    short = H.BoundaryArgs.flags.offset
    assert call(_args(struct_size=short, flags=16)) in (H.HC_ENODEV, H.HC_OK)
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
    assert L.hc_pre(P, P, 16, 4, 64, P + 0x100, S) == H.HC_ENODEV
