"""Python binding of libss.so: marshals PyTorch tensors into the C ABI.

Every function here only checks that the tensors can be handed over
(contiguous, on the GPU, of a dtype the ABI knows), allocates outputs with
PyTorch, and calls the library on the current HIP stream.  All arithmetic
runs in the library's kernels; there is no other code path.  If libss.so is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libss.so")
# SS_ABI_VERSION of include/ss.h that these signatures follow
ABI_VERSION = 12
_lock = threading.Lock()
_lib = None

SS_F32, SS_BF16 = 0, 1
SS_OK, SS_EINVAL, SS_EUNSUPPORTED, SS_EDEVICE = 0, 1, 2, 3
SS_SCAN_AUTO, SS_SCAN_SEQUENTIAL, SS_SCAN_SEGMENTED = 0, 1, 2


class SSError(RuntimeError):
    """A libss call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libss status {status}: {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libss.so (built by ``python -m selective_state_space_scan_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with "
                    "`python -m selective_state_space_scan_amd.build`")
            lib = ctypes.CDLL(_LIB_PATH)
            i64, vp, c_int, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            lib.ss_abi_version.restype = c_int
            lib.ss_abi_version.argtypes = []
            if lib.ss_abi_version() != ABI_VERSION:
                raise RuntimeError(
                    f"{_LIB_PATH} implements ABI {lib.ss_abi_version()}, this binding "
                    f"ABI {ABI_VERSION}: rebuild it with `python -m selective_state_space_scan_amd.build`")
            lib.ss_last_error.restype = ctypes.c_char_p
            lib.ss_last_error.argtypes = []
            lib.ss_fwd.restype = c_int
            lib.ss_fwd.argtypes = ([i64] * 4 + [c_int] + [vp] * 8 + [c_int] + [vp] * 5
                                   + [sz, vp])
            lib.ss_fwd_conv.restype = c_int
            lib.ss_fwd_conv.argtypes = ([i64] * 4 + [c_int] + [vp] * 2 + [i64] + [vp] + [c_int]
                                        + [vp] * 8 + [c_int] + [vp] * 6 + [sz, vp])
            lib.ss_bwd_conv.restype = c_int
            lib.ss_bwd_conv.argtypes = ([i64] * 4 + [c_int] + [vp] * 2 + [i64] + [vp] + [c_int]
                                        + [vp] * 8 + [c_int] + [vp] * 17 + [sz, vp])
            lib.ss_fwd_workspace_size.restype = sz
            lib.ss_fwd_workspace_size.argtypes = [i64] * 4
            lib.ss_ckpt_size.restype = sz
            lib.ss_ckpt_size.argtypes = [i64] * 4
            lib.ss_bwd_workspace_size.restype = sz
            lib.ss_bwd_workspace_size.argtypes = [i64] * 4 + [c_int]
            lib.ss_bwd.restype = c_int
            lib.ss_bwd.argtypes = ([i64] * 4 + [c_int] + [vp] * 8 + [c_int] + [vp] * 14
                                   + [sz, vp])
            lib.ss_bwd_noalloc.restype = c_int
            lib.ss_bwd_noalloc.argtypes = ([i64] * 4 + [c_int] + [vp] * 8 + [c_int] + [vp] * 13
                                           + [vp])
            lib.ss_bwd_noalloc_max_scratch.restype = sz
            lib.ss_bwd_noalloc_max_scratch.argtypes = []
            lib.ss_state_update.restype = c_int
            lib.ss_state_update.argtypes = ([i64] * 3 + [c_int] + [vp] * 9 + [c_int]
                                            + [vp] * 2)
            lib.ss_ssd_fwd.restype = c_int
            lib.ss_ssd_fwd.argtypes = [i64] * 6 + [c_int] + [vp] * 7 + [c_int] + [vp] * 5
            lib.ss_ssd_ckpt_size.restype = sz
            lib.ss_ssd_ckpt_size.argtypes = [i64] * 5
            lib.ss_ssd_bwd_workspace_size.restype = sz
            lib.ss_ssd_bwd_workspace_size.argtypes = [i64] * 6
            lib.ss_ssd_bwd.restype = c_int
            lib.ss_ssd_bwd.argtypes = ([i64] * 6 + [c_int] + [vp] * 7 + [c_int] + [vp] * 13
                                       + [sz, vp])
            lib.ss_conv1d_fwd.restype = c_int
            lib.ss_conv1d_fwd.argtypes = [i64] * 4 + [c_int] + [vp] * 3 + [c_int] + [vp] * 4
            lib.ss_conv1d_bwd.restype = c_int
            lib.ss_conv1d_bwd.argtypes = [i64] * 4 + [c_int] + [vp] * 3 + [c_int] + [vp] * 7
            lib.ss_conv1d_update.restype = c_int
            lib.ss_conv1d_update.argtypes = [i64] * 3 + [c_int] + [vp] * 4 + [c_int] + [vp] * 2
            lib.ss_set_scan_regime.restype = c_int
            lib.ss_set_scan_regime.argtypes = [c_int]
            lib.ss_scan_regime.restype = c_int
            lib.ss_scan_regime.argtypes = []
            _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != SS_OK:
        raise SSError(status, load().ss_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _ptr(t)


def _io_dtype(t) -> int:
    if t.dtype == torch.float32:
        return SS_F32
    if t.dtype == torch.bfloat16:
        return SS_BF16
    raise TypeError(f"unsupported io dtype {t.dtype} (float32 or bfloat16)")


def _same_io(io, *ts):
    for t in ts:
        if t is not None and _io_dtype(t) != io:
            raise TypeError("u, delta, B, C, z (and dout) must share one dtype")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def abi_version() -> int:
    return load().ss_abi_version()


def set_scan_regime(regime: int) -> None:
    """Scan regime of the calling thread (SS_SCAN_AUTO, SS_SCAN_SEQUENTIAL or
    SS_SCAN_SEGMENTED) for every later scan call and workspace query on it."""
    _check(load().ss_set_scan_regime(int(regime)))


def scan_regime() -> int:
    """The calling thread's scan regime."""
    return int(load().ss_scan_regime())


def ss_ckpt_size(batch, dim, dstate, seqlen) -> int:
    """Bytes of the chunk checkpoints ss_fwd can save for ss_bwd."""
    return int(load().ss_ckpt_size(batch, dim, dstate, seqlen))


def ss_ckpt_empty(u, dstate=16):
    """Allocate a checkpoint buffer for inputs shaped like ``u``."""
    batch, dim, seqlen = u.shape
    n = ss_ckpt_size(batch, dim, dstate, seqlen) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=u.device)


def ss_fwd_workspace_size(batch, dim, dstate, seqlen) -> int:
    return int(load().ss_fwd_workspace_size(batch, dim, dstate, seqlen))


def ss_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
           h0=None, out=None, last_state=None, return_last_state=False, ckpt=None,
           workspace=None):
    """Forward scan; returns ``out`` or ``(out, last_state)``.

    u, delta, z: (batch, dim, L); B, C: (batch, dstate, L) in float32 or bfloat16;
    A: (dim, dstate), D, delta_bias: (dim,), h0: (batch, dim, dstate) float32.
    ckpt: optional float32 buffer (see ss_ckpt_empty) that receives the chunk
    checkpoints for a later ss_bwd.  workspace: device buffer of at least
    ss_fwd_workspace_size() bytes (allocated here when None and needed, i.e.
    dstate > 16).
    """
    lib = load()
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    io = _io_dtype(u)
    _same_io(io, delta, B, C, z)
    if out is None:
        out = torch.empty_like(u)
    if return_last_state and last_state is None:
        last_state = torch.empty(batch, dim, dstate, dtype=torch.float32, device=u.device)
    need = ss_fwd_workspace_size(batch, dim, dstate, seqlen)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
    _check(lib.ss_fwd(batch, dim, dstate, seqlen, io, _ptr(u), _ptr(delta), _f32(A, "A"),
                      _ptr(B), _ptr(C), _f32(D, "D"), _ptr(z), _f32(delta_bias, "delta_bias"),
                      int(bool(delta_softplus)), _f32(h0, "h0"), _ptr(out),
                      _f32(last_state, "last_state"), _f32(ckpt, "ckpt"), _ptr(workspace),
                      0 if workspace is None else workspace.numel() * workspace.element_size(),
                      _stream()))
    return (out, last_state) if (return_last_state or last_state is not None) else out


def ss_fwd_conv(x, conv_weight, delta, A, B, C, D=None, z=None, delta_bias=None,
                delta_softplus=False, conv_bias=None, conv_silu=True, conv_init=None,
                h0=None, out=None, last_state=None, conv_final=None, ckpt=None,
                workspace=None):
    """The causal convolution fused in front of the scan: ss_fwd with
    ``u = ss_conv1d_fwd(x, conv_weight, conv_bias, conv_silu, conv_init)``
    computed inside the scan.  Returns ``out``; last_state and conv_final,
    when given, are filled in place.  dstate up to 64."""
    lib = load()
    batch, dim, seqlen = x.shape
    dstate = A.shape[1]
    width = conv_weight.shape[1]
    io = _io_dtype(x)
    _same_io(io, delta, B, C, z)
    if out is None:
        out = torch.empty_like(x)
    need = ss_fwd_workspace_size(batch, dim, dstate, seqlen)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib.ss_fwd_conv(batch, dim, dstate, seqlen, io, _ptr(x),
                           _f32(conv_weight, "conv_weight"), width,
                           _f32(conv_bias, "conv_bias"), int(bool(conv_silu)),
                           _f32(conv_init, "conv_init"), _ptr(delta), _f32(A, "A"), _ptr(B),
                           _ptr(C), _f32(D, "D"), _ptr(z), _f32(delta_bias, "delta_bias"),
                           int(bool(delta_softplus)), _f32(h0, "h0"), _ptr(out),
                           _f32(last_state, "last_state"), _f32(conv_final, "conv_final"),
                           _f32(ckpt, "ckpt"), _ptr(workspace),
                           0 if workspace is None else workspace.numel() * workspace.element_size(),
                           _stream()))
    return out


def ss_bwd_conv(x, conv_weight, delta, A, B, C, D=None, z=None, delta_bias=None,
                delta_softplus=False, dout=None, conv_bias=None, conv_silu=True,
                conv_init=None, h0=None, dlast=None, want_dh0=False, want_dconv_init=False,
                workspace=None, ckpt=None):
    """Backward of ss_fwd_conv (the convolution's backward fused into the
    scan's reverse pass).  Returns a dict with dx, dconv_weight, ddelta, dA,
    dB, dC and, for the optional inputs given, dconv_bias, dconv_init, dD,
    dz, ddelta_bias, dh0.  dstate up to 16."""
    lib = load()
    batch, dim, seqlen = x.shape
    dstate = A.shape[1]
    width = conv_weight.shape[1]
    io = _io_dtype(x)
    _same_io(io, delta, B, C, z, dout)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty_like(x), dconv_weight=torch.empty(dim, width, **f32),
             ddelta=torch.empty_like(delta), dA=torch.empty(dim, dstate, **f32),
             dB=torch.empty_like(B), dC=torch.empty_like(C))
    if conv_bias is not None:
        g["dconv_bias"] = torch.empty(dim, **f32)
    if conv_init is not None or want_dconv_init:
        g["dconv_init"] = torch.empty(batch, dim, width - 1, **f32)
    if D is not None:
        g["dD"] = torch.empty(dim, **f32)
    if z is not None:
        g["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(dim, **f32)
    if h0 is not None or want_dh0:
        g["dh0"] = torch.empty(batch, dim, dstate, **f32)
    if workspace is None:
        need = ss_bwd_workspace_size(batch, dim, dstate, seqlen, io)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.ss_bwd_conv(batch, dim, dstate, seqlen, io, _ptr(x),
                           _f32(conv_weight, "conv_weight"), width,
                           _f32(conv_bias, "conv_bias"), int(bool(conv_silu)),
                           _f32(conv_init, "conv_init"), _ptr(delta), _f32(A, "A"), _ptr(B),
                           _ptr(C), _f32(D, "D"), _ptr(z), _f32(delta_bias, "delta_bias"),
                           int(bool(delta_softplus)), _f32(h0, "h0"), _ptr(dout),
                           _f32(dlast, "dlast"), _ptr(g["dx"]), _ptr(g["dconv_weight"]),
                           _ptr(g.get("dconv_bias")), _ptr(g.get("dconv_init")),
                           _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                           _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                           _ptr(g.get("dh0")), _f32(ckpt, "ckpt"), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream()))
    return g


def ss_bwd_workspace_size(batch, dim, dstate, seqlen, io_dtype=SS_F32) -> int:
    return int(load().ss_bwd_workspace_size(batch, dim, dstate, seqlen, io_dtype))


def ss_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
           dout=None, h0=None, dlast=None, want_dh0=False, workspace=None, ckpt=None):
    """Backward of ``sum(dout * out) + sum(dlast * last_state)``.

    Returns a dict with du, ddelta, dA, dB, dC and, for the optional inputs
    given, dD, dz, ddelta_bias, plus dh0 when ``want_dh0`` or h0 is given.
    ckpt: checkpoints saved by ss_fwd for the same inputs (skips recomputing them).
    """
    lib = load()
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    io = _io_dtype(u)
    _same_io(io, delta, B, C, z, dout)
    dev = u.device
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(delta),
             dA=torch.empty(dim, dstate, dtype=torch.float32, device=dev),
             dB=torch.empty_like(B), dC=torch.empty_like(C))
    if D is not None:
        g["dD"] = torch.empty(dim, dtype=torch.float32, device=dev)
    if z is not None:
        g["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty(dim, dtype=torch.float32, device=dev)
    if want_dh0 or h0 is not None:
        g["dh0"] = torch.empty(batch, dim, dstate, dtype=torch.float32, device=dev)
    need = ss_bwd_workspace_size(batch, dim, dstate, seqlen, io)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.ss_bwd(batch, dim, dstate, seqlen, io, _ptr(u), _ptr(delta), _f32(A, "A"),
                      _ptr(B), _ptr(C), _f32(D, "D"), _ptr(z), _f32(delta_bias, "delta_bias"),
                      int(bool(delta_softplus)), _f32(h0, "h0"), _ptr(dout), _f32(dlast, "dlast"),
                      _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                      _ptr(g["dC"]), _ptr(g.get("dD")), _ptr(g.get("dz")),
                      _ptr(g.get("ddelta_bias")), _ptr(g.get("dh0")), _f32(ckpt, "ckpt"),
                      _ptr(workspace),
                      workspace.numel(), _stream()))
    return g


def ss_bwd_noalloc_max_scratch() -> int:
    return int(load().ss_bwd_noalloc_max_scratch())


def ss_bwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   dout=None, h0=None, dlast=None, want_dh0=False, ckpt=None, grads=None):
    """ss_bwd through the allocation-free entry point (its workspace is the
    library's device-resident scratch array).  ``grads``: preallocated
    gradient tensors, as the dict ss_bwd returns; allocated here when None.
    """
    lib = load()
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    io = _io_dtype(u)
    _same_io(io, delta, B, C, z, dout)
    dev = u.device
    g = grads
    if g is None:
        g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(delta),
                 dA=torch.empty(dim, dstate, dtype=torch.float32, device=dev),
                 dB=torch.empty_like(B), dC=torch.empty_like(C))
        if D is not None:
            g["dD"] = torch.empty(dim, dtype=torch.float32, device=dev)
        if z is not None:
            g["dz"] = torch.empty_like(z)
        if delta_bias is not None:
            g["ddelta_bias"] = torch.empty(dim, dtype=torch.float32, device=dev)
        if want_dh0 or h0 is not None:
            g["dh0"] = torch.empty(batch, dim, dstate, dtype=torch.float32, device=dev)
    _check(lib.ss_bwd_noalloc(batch, dim, dstate, seqlen, io, _ptr(u), _ptr(delta), _f32(A, "A"),
                              _ptr(B), _ptr(C), _f32(D, "D"), _ptr(z),
                              _f32(delta_bias, "delta_bias"), int(bool(delta_softplus)),
                              _f32(h0, "h0"), _ptr(dout), _f32(dlast, "dlast"), _ptr(g["du"]),
                              _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
                              _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("ddelta_bias")),
                              _ptr(g.get("dh0")), _f32(ckpt, "ckpt"), _stream()))
    return g


def ss_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                    delta_softplus=False, out=None):
    """One-token update of ``state`` (batch, dim, dstate) float32 in place.

    u, delta, z: (batch, dim); B, C: (batch, dstate).  Returns the output (batch, dim).
    """
    lib = load()
    batch, dim = u.shape
    dstate = A.shape[1]
    io = _io_dtype(u)
    _same_io(io, delta, B, C, z)
    if out is None:
        out = torch.empty_like(u)
    _check(lib.ss_state_update(batch, dim, dstate, io, _f32(state, "state"), _ptr(u),
                               _ptr(delta), _f32(A, "A"), _ptr(B), _ptr(C), _f32(D, "D"),
                               _ptr(z), _f32(delta_bias, "delta_bias"), int(bool(delta_softplus)),
                               _ptr(out), _stream()))
    return out


def ss_conv1d_fwd(x, weight, bias=None, silu=True, init_state=None, out=None,
                  final_state=None, return_final_state=False):
    """Causal depthwise convolution (+ SiLU); returns ``out`` or ``(out, final_state)``.

    x: (batch, dim, L) float32 or bfloat16; weight: (dim, width), bias: (dim,),
    init_state / final_state: (batch, dim, width - 1), all float32.
    """
    lib = load()
    batch, dim, seqlen = x.shape
    width = weight.shape[1]
    io = _io_dtype(x)
    if out is None:
        out = torch.empty_like(x)
    if return_final_state and final_state is None:
        final_state = torch.empty(batch, dim, width - 1, dtype=torch.float32, device=x.device)
    _check(lib.ss_conv1d_fwd(batch, dim, seqlen, width, io, _ptr(x), _f32(weight, "weight"),
                             _f32(bias, "bias"), int(bool(silu)), _f32(init_state, "init_state"),
                             _ptr(out), _f32(final_state, "final_state"), _stream()))
    return (out, final_state) if (return_final_state or final_state is not None) else out


def ss_conv1d_bwd(x, weight, bias=None, silu=True, init_state=None, dout=None,
                  want_dinit_state=False):
    """Backward of ``sum(dout * ss_conv1d_fwd(...))``.

    Returns a dict with dx, dweight, and dbias when bias is given, dinit_state
    when init_state is given or ``want_dinit_state``.
    """
    lib = load()
    batch, dim, seqlen = x.shape
    width = weight.shape[1]
    io = _io_dtype(x)
    _same_io(io, dout)
    dev = x.device
    g = dict(dx=torch.empty_like(x),
             dweight=torch.empty(dim, width, dtype=torch.float32, device=dev))
    if bias is not None:
        g["dbias"] = torch.empty(dim, dtype=torch.float32, device=dev)
    if want_dinit_state or init_state is not None:
        g["dinit_state"] = torch.empty(batch, dim, width - 1, dtype=torch.float32, device=dev)
    _check(lib.ss_conv1d_bwd(batch, dim, seqlen, width, io, _ptr(x), _f32(weight, "weight"),
                             _f32(bias, "bias"), int(bool(silu)), _f32(init_state, "init_state"),
                             _ptr(dout), _ptr(g["dx"]), _ptr(g["dweight"]), _ptr(g.get("dbias")),
                             _ptr(g.get("dinit_state")), _stream()))
    return g


def ss_conv1d_update(state, x, weight, bias=None, silu=True, out=None):
    """Decode step of the convolution; ``state`` (batch, dim, width - 1) float32
    is shifted in place.  x: (batch, dim).  Returns the output (batch, dim)."""
    lib = load()
    batch, dim = x.shape
    width = weight.shape[1]
    io = _io_dtype(x)
    if out is None:
        out = torch.empty_like(x)
    _check(lib.ss_conv1d_update(batch, dim, width, io, _f32(state, "state"), _ptr(x),
                                _f32(weight, "weight"), _f32(bias, "bias"), int(bool(silu)),
                                _ptr(out), _stream()))
    return out


def ss_ssd_ckpt_size(batch, seqlen, nheads, headdim, dstate) -> int:
    """Bytes of the chunk states ss_ssd_fwd can save for ss_ssd_bwd."""
    return int(load().ss_ssd_ckpt_size(batch, seqlen, nheads, headdim, dstate))


def ss_ssd_ckpt_empty(x, dstate):
    """A float32 device buffer for ss_ssd_fwd's ckpt (x: the forward's input)."""
    batch, seqlen, nheads, headdim = x.shape
    n = ss_ssd_ckpt_size(batch, seqlen, nheads, headdim, dstate) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=x.device)


def ss_ssd_fwd(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, h0=None, out=None,
               last_state=None, return_last_state=False, ckpt=None):
    """Mamba-2 SSD forward; returns ``out`` or ``(out, last_state)``.

    x: (batch, L, nheads, headdim), dt: (batch, L, nheads), B, C: (batch, L,
    ngroups, dstate), all bfloat16; A, D, dt_bias: (nheads,) float32;
    h0 / last_state: (batch, nheads, headdim, dstate) float32.
    ckpt: optional float32 buffer (see ss_ssd_ckpt_empty) that receives the
    state entering every chunk of 64 steps, for ss_ssd_bwd.
    """
    lib = load()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    io = _io_dtype(x)
    _same_io(io, dt, B, C)
    if out is None:
        out = torch.empty_like(x)
    if return_last_state and last_state is None:
        last_state = torch.empty(batch, nheads, headdim, dstate, dtype=torch.float32,
                                 device=x.device)
    _check(lib.ss_ssd_fwd(batch, seqlen, nheads, headdim, ngroups, dstate, io, _ptr(x), _ptr(dt),
                          _f32(A, "A"), _ptr(B), _ptr(C), _f32(D, "D"), _f32(dt_bias, "dt_bias"),
                          int(bool(dt_softplus)), _f32(h0, "h0"), _ptr(out),
                          _f32(last_state, "last_state"), _f32(ckpt, "ckpt"), _stream()))
    return (out, last_state) if (return_last_state or last_state is not None) else out


def ss_ssd_bwd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate) -> int:
    return int(load().ss_ssd_bwd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate))


def ss_ssd_bwd(x, dt, A, B, C, D=None, dt_bias=None, dt_softplus=True, h0=None, dout=None,
               dlast=None, want_dh0=False, workspace=None, ckpt=None):
    """Backward of ``sum(dout * y) + sum(dlast * last_state)`` for ss_ssd_fwd.

    Returns a dict with dx, ddt, dA, dB, dC and, for the optional inputs
    given, dD, ddt_bias, plus dh0 when ``want_dh0`` or h0 is given.
    ckpt: chunk states saved by ss_ssd_fwd for the same inputs (skips the
    states pass).
    """
    lib = load()
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    io = _io_dtype(x)
    _same_io(io, dt, B, C, dout)
    dev = x.device
    g = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt),
             dA=torch.empty(nheads, dtype=torch.float32, device=dev),
             dB=torch.empty_like(B), dC=torch.empty_like(C))
    if D is not None:
        g["dD"] = torch.empty(nheads, dtype=torch.float32, device=dev)
    if dt_bias is not None:
        g["ddt_bias"] = torch.empty(nheads, dtype=torch.float32, device=dev)
    if want_dh0 or h0 is not None:
        g["dh0"] = torch.empty(batch, nheads, headdim, dstate, dtype=torch.float32, device=dev)
    need = ss_ssd_bwd_workspace_size(batch, seqlen, nheads, headdim, ngroups, dstate)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.ss_ssd_bwd(batch, seqlen, nheads, headdim, ngroups, dstate, io, _ptr(x), _ptr(dt),
                          _f32(A, "A"), _ptr(B), _ptr(C), _f32(D, "D"), _f32(dt_bias, "dt_bias"),
                          int(bool(dt_softplus)), _f32(h0, "h0"), _ptr(dout),
                          _f32(dlast, "dlast"), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]),
                          _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dD")),
                          _ptr(g.get("ddt_bias")), _ptr(g.get("dh0")), _f32(ckpt, "ckpt"),
                          _ptr(workspace), workspace.numel(), _stream()))
    return g
