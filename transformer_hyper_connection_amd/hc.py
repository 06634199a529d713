"""Python binding of libhc (the HIP library), argument marshalling only.

Every function checks dtypes, devices, shapes and contiguity, allocates its
outputs with torch (unless given), and calls the C entry point of the same
name on the current HIP stream.  All arithmetic runs in libhc's kernels; if
libhc.so is missing the first call raises -- there is no fallback.

Names and argument orders follow the model-atlas pages ("Source layer, pairs
pooled": Block.hc_mixes / hc_pre / hc_post; "Reading weights": the
hc_split_sinkhorn wrapper).  Streams are [..., hc, d] bf16, coefficients fp32.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhc.so")

HC_OK, HC_EINVAL, HC_ENOTSUP, HC_EHIP, HC_ENODEV = 0, -1, -2, -3, -4
HC_BOUNDARY_X_EXPANDED = 4
HC_BOUNDARY_TWO_LAUNCH = 16


class HCError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class BoundaryArgs(ctypes.Structure):
    """Mirror of ``hc_boundary_args`` in include/hc.h."""
    _fields_ = [
        ("struct_size", c_uint32), ("hc", c_int32), ("d", c_int32), ("iters", c_int32),
        ("n", c_int64), ("hc_eps", c_float), ("norm_eps", c_float), ("rms_eps", c_float),
        ("delta", c_void_p), ("x", c_void_p), ("post_in", c_void_p), ("comb_in", c_void_p),
        ("pre_in", c_void_p), ("fn_packed", c_void_p), ("hc_base", c_void_p),
        ("hc_scale", c_void_p), ("gamma", c_void_p), ("x_out", c_void_p), ("y_out", c_void_p),
        ("mixes_out", c_void_p), ("pre_out", c_void_p), ("post_out", c_void_p),
        ("comb_out", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("flags", c_uint32), ("x_mean_out", c_void_p),
    ]


# name -> (restype, argtypes); every symbol include/hc.h declares
SIGNATURES = {
    "hc_version": (c_int, []),
    "hc_strerror": (ctypes.c_char_p, [c_int]),
    "hc_last_error": (ctypes.c_char_p, []),
    "hc_fn_packed_bytes": (c_size_t, [c_int, c_int]),
    "hc_fn_pack": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "hc_mixes": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_int, c_float, c_void_p, c_void_p,
                         c_void_p, c_int, c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                         c_void_p]),
    "hc_workspace_bytes": (c_size_t, [c_int64, c_int, c_int]),
    "hc_split_sinkhorn": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int, c_float,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
    "hc_pre": (c_int, [c_void_p, c_void_p, c_int64, c_int, c_int, c_void_p, c_void_p]),
    "hc_post": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int, c_void_p,
                        c_void_p]),
    "hc_boundary": (c_int, [ctypes.POINTER(BoundaryArgs), c_void_p]),
    "hc_boundary_static": (c_int, [ctypes.POINTER(BoundaryArgs), c_void_p]),
    "hc_boundary_begin": (c_int, [ctypes.POINTER(BoundaryArgs), c_void_p]),
    "hc_boundary_end": (c_int, [ctypes.POINTER(BoundaryArgs), c_void_p]),
    "hc_boundary_workspace_bytes": (c_size_t, [c_int64, c_int, c_int]),
    "hc_workspace_status": (c_int, [c_void_p, c_size_t, c_int, ctypes.POINTER(c_uint32), c_void_p]),
    "hc_workspace_layout": (c_int, [c_int64, c_int, c_int, ctypes.POINTER(c_size_t)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libhc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m transformer_hyper_connection_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != HC_OK:
        L = lib()
        detail = L.hc_last_error().decode()
        raise HCError(rc, f"{what}: {L.hc_strerror(rc).decode()} ({detail})")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


_workspaces: dict = {}


def workspace(n: int, hc: int, d: int, device) -> torch.Tensor | None:
    """A device workspace of at least hc_workspace_bytes(n, hc, d) bytes,
    zero-filled when allocated (the library keeps it valid from call to call),
    cached per (device, stream): calls on one stream may share it."""
    nbytes = lib().hc_workspace_bytes(n, hc, d)
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def workspace_status(ws: torch.Tensor, clear: bool = False) -> int:
    """The sticky error mask of a workspace (hc_workspace_status): bit 0 set if
    a call on it waited for another workgroup's words until its bound.
    Synchronises the current stream; with clear, resets the mask."""
    mask = c_uint32(0)
    _check(lib().hc_workspace_status(ws.data_ptr(), ws.numel(), 1 if clear else 0, ctypes.byref(mask),
                                     _stream(ws.device)), "hc_workspace_status")
    return int(mask.value)


def _need(t, name, dtype, device=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _streams_shape(x):
    if x.dim() < 2:
        raise ValueError("streams must be [..., hc, d]")
    lead = tuple(x.shape[:-2])
    n = 1
    for s in lead:
        n *= s
    return lead, n, x.shape[-2], x.shape[-1]


# ------------------------------------------------------------------ packing
def hc_fn_pack(hc_fn: torch.Tensor, hc: int = 4) -> torch.Tensor:
    """Pack an fp32 projection weight [(2+hc)*hc, hc*d] for the kernels."""
    _need(hc_fn, "hc_fn", torch.float32)
    mix, hd = hc_fn.shape
    d = hd // hc
    nbytes = lib().hc_fn_packed_bytes(hc, d)
    if nbytes == 0 or mix != (2 + hc) * hc or hd != hc * d:
        raise HCError(HC_ENOTSUP, f"hc_fn shape {tuple(hc_fn.shape)} not supported")
    out = torch.empty(nbytes, dtype=torch.uint8, device=hc_fn.device)
    _check(lib().hc_fn_pack(hc_fn.data_ptr(), hc, d, out.data_ptr(), _stream(hc_fn.device)), "hc_fn_pack")
    return out


# ------------------------------------------------------------------ entry points
def hc_split_sinkhorn(mixes, hc_scale, hc_base, hc_mult: int = 4, sinkhorn_iters: int = 20,
                      eps: float = 1e-6):
    """mixes [..., (2+hc)*hc] -> (pre [..., hc], post [..., hc], comb [..., hc, hc])."""
    dev = mixes.device
    _need(mixes, "mixes", torch.float32)
    _need(hc_scale, "hc_scale", torch.float32, dev, (3,))
    _need(hc_base, "hc_base", torch.float32, dev, ((2 + hc_mult) * hc_mult,))
    if mixes.dim() < 1 or mixes.shape[-1] != (2 + hc_mult) * hc_mult:
        raise ValueError(f"mixes: last dimension {tuple(mixes.shape)[-1:]} is not (2+hc)*hc for hc={hc_mult}")
    lead = tuple(mixes.shape[:-1])
    n = mixes.numel() // mixes.shape[-1]
    pre = torch.empty(*lead, hc_mult, dtype=torch.float32, device=dev)
    post = torch.empty_like(pre)
    comb = torch.empty(*lead, hc_mult, hc_mult, dtype=torch.float32, device=dev)
    _check(lib().hc_split_sinkhorn(mixes.data_ptr(), hc_scale.data_ptr(), hc_base.data_ptr(), n, hc_mult,
                                   sinkhorn_iters, eps, pre.data_ptr(), post.data_ptr(), comb.data_ptr(),
                                   _stream(dev)), "hc_split_sinkhorn")
    return pre, post, comb


def hc_mixes(x, fn_packed, hc_scale=None, hc_base=None, *, norm_eps: float = 1e-6,
             sinkhorn_iters: int = 20, hc_eps: float = 1e-6, return_mixes: bool = False):
    """Block.hc_mixes.  With hc_scale/hc_base: (pre, post, comb) [+ mixes if
    return_mixes]; without: mixes [..., (2+hc)*hc]."""
    dev = x.device
    _need(x, "x", torch.bfloat16)
    _need(fn_packed, "fn_packed", torch.uint8, dev)
    lead, n, hc, d = _streams_shape(x)
    mix = (2 + hc) * hc
    split = hc_scale is not None or hc_base is not None
    mixes = torch.empty(*lead, mix, dtype=torch.float32, device=dev) if (return_mixes or not split) else None
    pre = post = comb = None
    if split:
        _need(hc_scale, "hc_scale", torch.float32, dev)
        _need(hc_base, "hc_base", torch.float32, dev)
        pre = torch.empty(*lead, hc, dtype=torch.float32, device=dev)
        post = torch.empty_like(pre)
        comb = torch.empty(*lead, hc, hc, dtype=torch.float32, device=dev)
    ws = workspace(n, hc, d, dev)
    _check(lib().hc_mixes(x.data_ptr(), fn_packed.data_ptr(), n, hc, d, norm_eps, _ptr(mixes),
                          _ptr(hc_scale), _ptr(hc_base), sinkhorn_iters, hc_eps, _ptr(pre), _ptr(post),
                          _ptr(comb), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)), "hc_mixes")
    if not split:
        return mixes
    return (pre, post, comb, mixes) if return_mixes else (pre, post, comb)


def hc_pre(x, pre_mix):
    """Block.hc_pre: [..., hc, d] x [..., hc] -> [..., d] bf16."""
    dev = x.device
    _need(x, "x", torch.bfloat16)
    lead, n, hc, d = _streams_shape(x)
    _need(pre_mix, "pre_mix", torch.float32, dev, (*lead, hc))
    y = torch.empty(*lead, d, dtype=torch.bfloat16, device=dev)
    _check(lib().hc_pre(x.data_ptr(), pre_mix.data_ptr(), n, hc, d, y.data_ptr(), _stream(dev)), "hc_pre")
    return y


def hc_post(x, residual, post, comb, out=None):
    """Block.hc_post (argument order as the pages: sublayer output x first,
    residual streams second) -> [..., hc, d] bf16, into ``out`` if given."""
    dev = residual.device
    _need(residual, "residual", torch.bfloat16)
    lead, n, hc, d = _streams_shape(residual)
    _need(x, "x", torch.bfloat16, dev, (*lead, d))
    _need(post, "post", torch.float32, dev, (*lead, hc))
    _need(comb, "comb", torch.float32, dev, (*lead, hc, hc))
    if out is None:
        out = torch.empty_like(residual)
    else:
        _need(out, "out", torch.bfloat16, dev, tuple(residual.shape))
    _check(lib().hc_post(x.data_ptr(), residual.data_ptr(), post.data_ptr(), comb.data_ptr(), n, hc, d,
                         out.data_ptr(), _stream(dev)), "hc_post")
    return out


def _prepare_boundary(x, *, delta=None, post_in=None, comb_in=None, pre_in=None, fn_packed=None,
                      hc_base=None, hc_scale=None, gamma=None, iters: int = 20, hc_eps: float = 1e-6,
                      norm_eps: float = 1e-6, rms_eps: float = 1e-6, out: dict | None = None,
                      want_mixes: bool = False, x_expanded: bool = False, want_mean: bool = False,
                      hc_mult: int = 4, two_launch: bool = False, own_workspace: bool = True):
    """Checks the arguments of one boundary call, allocates missing outputs and
    fills the C argument struct.  Returns (struct, outputs).  hc_mult is the
    number of streams of an expanded x (otherwise x's shape gives it)."""
    dev = x.device
    _need(x, "x", torch.bfloat16)
    if x_expanded:                   # x [..., d]: every stream is that row
        if x.dim() < 1:
            raise ValueError("an expanded x must be [..., d]")
        lead, d, hc = tuple(x.shape[:-1]), x.shape[-1], hc_mult
        n = 1
        for v in lead:
            n *= v
    else:
        lead, n, hc, d = _streams_shape(x)
    mix = (2 + hc) * hc
    o = dict(out or {})

    def alloc(key, shape, dtype):
        if o.get(key) is None:
            o[key] = torch.empty(*shape, dtype=dtype, device=dev)
        return _need(o[key], key, dtype, dev, shape)

    if delta is not None:
        _need(delta, "delta", torch.bfloat16, dev, (*lead, d))
        _need(post_in, "post_in", torch.float32, dev, (*lead, hc))
        _need(comb_in, "comb_in", torch.float32, dev, (*lead, hc, hc))
        alloc("x_out", (*lead, hc, d), torch.bfloat16)
    else:
        o["x_out"] = None
    if pre_in is not None:
        _need(pre_in, "pre_in", torch.float32, dev, (*lead, hc))
    if gamma is not None:
        _need(gamma, "gamma", torch.float32, dev, (d,))
    alloc("y", (*lead, d), torch.bfloat16)
    if want_mean or o.get("x_mean") is not None:
        alloc("x_mean", (*lead, d), torch.bfloat16)
    if fn_packed is not None:
        _need(fn_packed, "fn_packed", torch.uint8, dev)
        _need(hc_base, "hc_base", torch.float32, dev, (mix,))
        _need(hc_scale, "hc_scale", torch.float32, dev, (3,))
        alloc("pre", (*lead, hc), torch.float32)
        alloc("post", (*lead, hc), torch.float32)
        alloc("comb", (*lead, hc, hc), torch.float32)
        if want_mixes or o.get("mixes") is not None:
            alloc("mixes", (*lead, mix), torch.float32)
    a = BoundaryArgs()
    a.struct_size = ctypes.sizeof(BoundaryArgs)
    a.hc, a.d, a.iters, a.n = hc, d, iters, n
    a.hc_eps, a.norm_eps, a.rms_eps = hc_eps, norm_eps, rms_eps
    a.delta, a.x, a.post_in, a.comb_in = _ptr(delta), x.data_ptr(), _ptr(post_in), _ptr(comb_in)
    a.pre_in, a.fn_packed, a.hc_base, a.hc_scale = _ptr(pre_in), _ptr(fn_packed), _ptr(hc_base), _ptr(hc_scale)
    a.gamma, a.x_out, a.y_out = _ptr(gamma), _ptr(o.get("x_out")), o["y"].data_ptr()
    a.mixes_out, a.pre_out = _ptr(o.get("mixes")), _ptr(o.get("pre"))
    a.post_out, a.comb_out = _ptr(o.get("post")), _ptr(o.get("comb"))
    a.flags = (HC_BOUNDARY_X_EXPANDED if x_expanded else 0) | (HC_BOUNDARY_TWO_LAUNCH if two_launch else 0)
    a.x_mean_out = _ptr(o.get("x_mean"))
    if fn_packed is not None and own_workspace:
        ws = o.get("workspace")
        if ws is None:
            ws = workspace(n, hc, d, dev)
        if ws is not None:
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
            o["workspace"] = ws
    return a, o


def hc_boundary(x, **kw):
    """One fused sublayer boundary (see include/hc.h).  Keyword arguments:
    delta, post_in, comb_in, pre_in, fn_packed, hc_base, hc_scale, gamma, iters,
    hc_eps, norm_eps, rms_eps, out, want_mixes, two_launch (the
    HC_BOUNDARY_TWO_LAUNCH schedule), x_expanded (x is [..., d], every stream
    that row: HC_BOUNDARY_X_EXPANDED; hc_mult then gives the number of
    streams), want_mean (the mean over the streams, "x_mean").  Returns a dict with x_out (None at a block entry), y,
    and pre/post/comb (+ mixes) unless fn_packed is None.
    ``out`` may hold preallocated outputs under the same keys (and a
    "workspace"); they are used as given."""
    a, o = _prepare_boundary(x, **kw)
    _check(lib().hc_boundary(ctypes.byref(a), _stream(x.device)), "hc_boundary")
    return o


def hc_boundary_static(x, **kw):
    """hc_boundary on the library's static device workspace (include/hc.h,
    hc_boundary_static): the same keyword arguments, no workspace allocated
    or passed.  Returns the output dict of hc_boundary (without a workspace)."""
    a, o = _prepare_boundary(x, **kw, own_workspace=False)
    _check(lib().hc_boundary_static(ctypes.byref(a), _stream(x.device)), "hc_boundary_static")
    return o


class BoundaryCall:
    """One hc_boundary call on fixed buffers, checked once: run() enqueues it
    again on the current stream with no per-call checking or allocation (for a
    loop over the same buffers, such as a serving step).  The tensors given
    and the outputs in ``outputs`` must stay alive and in place meanwhile."""

    def __init__(self, x, **kw):
        self._a, self.outputs = _prepare_boundary(x, **kw)
        self._keep = (x, kw)
        self._dev = x.device
        L = lib()
        self._fn, self._begin, self._end = L.hc_boundary, L.hc_boundary_begin, L.hc_boundary_end
        self._ref = ctypes.byref(self._a)

    def _go(self, fn, stream, what):
        rc = fn(self._ref, _stream(self._dev) if stream is None else stream)
        if rc != HC_OK:
            _check(rc, what)

    def run(self, stream: int | None = None) -> None:
        """The whole boundary (hc_boundary)."""
        self._go(self._fn, stream, "hc_boundary")

    def begin(self, stream: int | None = None) -> None:
        """The streaming half (hc_boundary_begin)."""
        self._go(self._begin, stream, "hc_boundary_begin")

    def end(self, stream: int | None = None) -> None:
        """The finishing half (hc_boundary_end); after begin() on the same stream."""
        self._go(self._end, stream, "hc_boundary_end")
