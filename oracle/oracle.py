"""Python access to the double-precision oracle in ``ss_oracle.c``.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It never touches the
GPU library and shares no code with it.

Every input is widened exactly to float64 (float32 and bfloat16 values are
representable in double), passed to the C routines, and the results come
back as float64 numpy arrays.  The arithmetic itself lives entirely in
``ss_oracle.c``; this file only marshals arrays and, when asked for more
than one thread, splits independent rows (forward, state update) or batch
entries (backward) across threads and folds the per-thread parameter
gradients in ascending batch order.  The causal convolution routines
(``conv_fwd``, ``conv_bwd``, ``conv_update``) and the Mamba-2 SSD forward
(``ssd_fwd``) follow the same pattern.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ss_oracle.c")
_LIB = os.path.join(_HERE, "libss_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``ss_oracle.c`` with gcc (-O2, IEEE semantics, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=_HERE)
    os.close(fd)
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.chmod(tmp, 0o755)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # The mutation test points this at a deliberately broken copy of
            # the oracle to show that the pins catch each planted mistake.
            path = os.environ.get("SS_ORACLE_LIB_OVERRIDE") or build()
            lib = ctypes.CDLL(path)
            i64, dp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            lib.sso_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 8 + [c_int] + [dp] * 3 + [i64, i64]
            lib.sso_fwd.restype = None
            lib.sso_bwd.argtypes = ([i64, i64, i64, i64] + [dp] * 8 + [c_int] + [dp] * 12
                                    + [i64, i64])
            lib.sso_bwd.restype = c_int
            lib.sso_state_update.argtypes = ([i64, i64, i64] + [dp] * 9 + [c_int] + [dp]
                                             + [i64, i64])
            lib.sso_state_update.restype = None
            lib.sso_conv_fwd.argtypes = [i64] * 4 + [dp] * 3 + [c_int] + [dp] * 3 + [i64, i64]
            lib.sso_conv_fwd.restype = None
            lib.sso_conv_bwd.argtypes = [i64] * 4 + [dp] * 3 + [c_int] + [dp] * 6 + [i64, i64]
            lib.sso_conv_bwd.restype = None
            lib.sso_conv_update.argtypes = [i64] * 3 + [dp] * 4 + [c_int] + [dp]
            lib.sso_conv_update.restype = None
            lib.sso_ssd_fwd.argtypes = [i64] * 6 + [dp] * 7 + [c_int] + [dp] * 3 + [i64, i64]
            lib.sso_ssd_fwd.restype = c_int
            lib.sso_ssd_bwd.argtypes = [i64] * 6 + [dp] * 7 + [c_int] + [dp] * 11 + [i64, i64]
            lib.sso_ssd_bwd.restype = c_int
            _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _split(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    edges = [n * i // parts for i in range(parts + 1)]
    return [(edges[i], edges[i + 1]) for i in range(parts)]


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
        h0=None, threads: int = 1):
    """Forward scan.  Returns ``(y, last_state)`` as float64 arrays.

    u, delta, z: (batch, dim, L); A: (dim, N); B, C: (batch, N, L);
    D, delta_bias: (dim,); h0: (batch, dim, N) or None (zero initial state).
    """
    lib = _load()
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias, h0 = map(_f64, (D, z, delta_bias, h0))
    nb, nd, nl = u.shape
    ns = A.shape[1]
    y = np.zeros((nb, nd, nl))
    last = np.zeros((nb, nd, ns))
    args = (nb, nd, ns, nl, _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
            _p(delta_bias), int(bool(delta_softplus)), _p(h0), _p(y), _p(last))
    rows = nb * nd
    if threads <= 1 or rows < 2:
        lib.sso_fwd(*args, 0, rows)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda rg: lib.sso_fwd(*args, rg[0], rg[1]), _split(rows, threads)))
    return y, last


def bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
        dout=None, h0=None, dlast=None, threads: int = 1):
    """Backward of ``sum(dout * y) (+ sum(dlast * last_state))``.

    Returns a dict with du, ddelta, dA, dB, dC and, for the optional inputs
    that were given, dD, dz, ddelta_bias, dh0 (float64 arrays).
    """
    lib = _load()
    u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
    D, z, delta_bias, h0, dlast = map(_f64, (D, z, delta_bias, h0, dlast))
    nb, nd, nl = u.shape
    ns = A.shape[1]
    du = np.zeros((nb, nd, nl))
    ddelta = np.zeros((nb, nd, nl))
    dB = np.zeros((nb, ns, nl))
    dC = np.zeros((nb, ns, nl))
    dz = np.zeros((nb, nd, nl)) if z is not None else None
    dh0 = np.zeros((nb, nd, ns)) if h0 is not None else None
    pieces = _split(nb, threads)
    # per-piece parameter gradients, folded below in ascending batch order
    part = [(np.zeros((nd, ns)), np.zeros(nd), np.zeros(nd)) for _ in pieces]

    def run(i):
        b0, b1 = pieces[i]
        dA_i, dD_i, db_i = part[i]
        rc = lib.sso_bwd(nb, nd, ns, nl, _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
                         _p(delta_bias), int(bool(delta_softplus)), _p(h0), _p(dout),
                         _p(dlast), _p(du), _p(ddelta), _p(dA_i), _p(dB), _p(dC), _p(dD_i),
                         _p(dz), _p(db_i), _p(dh0), b0, b1)
        if rc != 0:
            raise MemoryError("oracle backward could not allocate scratch")

    if len(pieces) == 1:
        run(0)
    else:
        with ThreadPoolExecutor(len(pieces)) as ex:
            list(ex.map(run, range(len(pieces))))
    dA = np.zeros((nd, ns))
    dD = np.zeros(nd)
    dbias = np.zeros(nd)
    for dA_i, dD_i, db_i in part:
        dA += dA_i
        dD += dD_i
        dbias += db_i
    out = dict(du=du, ddelta=ddelta, dA=dA, dB=dB, dC=dC)
    if D is not None:
        out["dD"] = dD
    if z is not None:
        out["dz"] = dz
    if delta_bias is not None:
        out["ddelta_bias"] = dbias
    if h0 is not None:
        out["dh0"] = dh0
    return out


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=False, threads: int = 1):
    """One-token update.  Returns ``(new_state, y)``; the input is not modified.

    state: (batch, dim, N); u, delta, z: (batch, dim); B, C: (batch, N).
    """
    lib = _load()
    st = _f64(state).copy()
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, delta_bias = map(_f64, (D, z, delta_bias))
    nb, nd = u.shape
    ns = A.shape[1]
    y = np.zeros((nb, nd))
    args = (nb, nd, ns, _p(st), _p(u), _p(delta), _p(A), _p(B), _p(C), _p(D), _p(z),
            _p(delta_bias), int(bool(delta_softplus)), _p(y))
    rows = nb * nd
    if threads <= 1 or rows < 2:
        lib.sso_state_update(*args, 0, rows)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda rg: lib.sso_state_update(*args, rg[0], rg[1]),
                        _split(rows, threads)))
    return st, y


def conv_fwd(x, weight, bias=None, silu=True, init_state=None, threads: int = 1):
    """Causal depthwise convolution (+ SiLU).  Returns ``(out, final_state)``.

    x: (batch, dim, L); weight: (dim, K); bias: (dim,) or None;
    init_state: (batch, dim, K-1) inputs before t = 0, or None (zeros).
    final_state: (batch, dim, K-1), the last K-1 inputs.
    """
    lib = _load()
    x, weight, bias, s0 = map(_f64, (x, weight, bias, init_state))
    nb, nd, nl = x.shape
    nk = weight.shape[1]
    out = np.zeros((nb, nd, nl))
    sf = np.zeros((nb, nd, nk - 1))
    args = (nb, nd, nl, nk, _p(x), _p(weight), _p(bias), int(bool(silu)), _p(s0), _p(out),
            _p(sf))
    rows = nb * nd
    if threads <= 1 or rows < 2:
        lib.sso_conv_fwd(*args, 0, rows)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda rg: lib.sso_conv_fwd(*args, rg[0], rg[1]),
                        _split(rows, threads)))
    return out, sf


def conv_bwd(x, weight, bias=None, silu=True, init_state=None, dout=None, threads: int = 1):
    """Backward of ``sum(dout * conv_fwd(...)[0])``.

    Returns a dict with dx, dweight and, when given, dbias and dinit_state.
    """
    lib = _load()
    x, weight, bias, s0, dout = map(_f64, (x, weight, bias, init_state, dout))
    nb, nd, nl = x.shape
    nk = weight.shape[1]
    dx = np.zeros((nb, nd, nl))
    ds0 = np.zeros((nb, nd, nk - 1)) if s0 is not None else None
    pieces = _split(nb, threads)
    part = [(np.zeros((nd, nk)), np.zeros(nd)) for _ in pieces]

    def run(i):
        b0, b1 = pieces[i]
        dw_i, db_i = part[i]
        lib.sso_conv_bwd(nb, nd, nl, nk, _p(x), _p(weight), _p(bias), int(bool(silu)),
                         _p(s0), _p(dout), _p(dx), _p(dw_i), _p(db_i), _p(ds0), b0, b1)

    if len(pieces) == 1:
        run(0)
    else:
        with ThreadPoolExecutor(len(pieces)) as ex:
            list(ex.map(run, range(len(pieces))))
    dw = np.zeros((nd, nk))
    db = np.zeros(nd)
    for dw_i, db_i in part:
        dw += dw_i
        db += db_i
    out = dict(dx=dx, dweight=dw)
    if bias is not None:
        out["dbias"] = db
    if s0 is not None:
        out["dinit_state"] = ds0
    return out


def conv_update(state, x, weight, bias=None, silu=True):
    """One input per row.  Returns ``(new_state, out)``; the input is not modified.

    state: (batch, dim, K-1); x: (batch, dim); weight: (dim, K).
    """
    lib = _load()
    st = _f64(state).copy()
    x, weight, bias = map(_f64, (x, weight, bias))
    nb, nd = x.shape
    nk = weight.shape[1]
    out = np.zeros((nb, nd))
    lib.sso_conv_update(nb, nd, nk, _p(st), _p(x), _p(weight), _p(bias), int(bool(silu)),
                        _p(out))
    return st, out


def ssd_fwd(x, dt, A, B, C, D=None, dt_bias=None, softplus=True, h0=None, threads: int = 1):
    """Mamba-2 SSD forward (scalar A per head).  Returns ``(y, last_state)``.

    x: (batch, L, nheads, headdim); dt: (batch, L, nheads); A, D, dt_bias:
    (nheads,); B, C: (batch, L, ngroups, dstate); h0: (batch, nheads,
    headdim, dstate) or None.
    """
    lib = _load()
    x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
    D, dt_bias, h0 = map(_f64, (D, dt_bias, h0))
    nb, nl, nh, npd = x.shape
    ng, ns = B.shape[2], B.shape[3]
    y = np.zeros((nb, nl, nh, npd))
    last = np.zeros((nb, nh, npd, ns))
    args = (nb, nl, nh, npd, ng, ns, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(dt_bias),
            int(bool(softplus)), _p(h0), _p(y), _p(last))

    def run(rg):
        if lib.sso_ssd_fwd(*args, rg[0], rg[1]) != 0:
            raise MemoryError("oracle SSD could not allocate its state")

    pieces = _split(nb, threads)
    if len(pieces) == 1:
        run(pieces[0])
    else:
        with ThreadPoolExecutor(len(pieces)) as ex:
            list(ex.map(run, pieces))
    return y, last


def ssd_bwd(x, dt, A, B, C, D=None, dt_bias=None, softplus=True, h0=None, dy=None,
            dlast=None, threads: int = 1):
    """Backward of ``sum(dy * y) (+ sum(dlast * last_state))`` for ``ssd_fwd``.

    Returns a dict with dx, ddt (w.r.t. the raw dt), dA, dB, dC, dh0 and, for
    the optional inputs given, dD and ddt_bias.
    """
    lib = _load()
    x, dt, A, B, C, dy = map(_f64, (x, dt, A, B, C, dy))
    D, dt_bias, h0, dlast = map(_f64, (D, dt_bias, h0, dlast))
    nb, nl, nh, npd = x.shape
    ng, ns = B.shape[2], B.shape[3]
    dx = np.zeros_like(x)
    ddt = np.zeros((nb, nl, nh))
    dh0 = np.zeros((nb, nh, npd, ns))
    pieces = _split(nb, threads)
    part = [(np.zeros(nh), np.zeros((nb, nl, ng, ns)), np.zeros((nb, nl, ng, ns)), np.zeros(nh),
             np.zeros(nh)) for _ in pieces]

    def run(i):
        b0, b1 = pieces[i]
        dA_i, dB_i, dC_i, dD_i, db_i = part[i]
        rc = lib.sso_ssd_bwd(nb, nl, nh, npd, ng, ns, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                             _p(dt_bias), int(bool(softplus)), _p(h0), _p(dy), _p(dlast), _p(dx),
                             _p(ddt), _p(dA_i), _p(dB_i), _p(dC_i), _p(dD_i), _p(db_i), _p(dh0),
                             b0, b1)
        if rc != 0:
            raise MemoryError("oracle SSD backward could not allocate its states")

    if len(pieces) == 1:
        run(0)
    else:
        with ThreadPoolExecutor(len(pieces)) as ex:
            list(ex.map(run, range(len(pieces))))
    dA = np.zeros(nh)
    dB = np.zeros((nb, nl, ng, ns))
    dC = np.zeros((nb, nl, ng, ns))
    dD = np.zeros(nh)
    dbias = np.zeros(nh)
    for dA_i, dB_i, dC_i, dD_i, db_i in part:
        dA += dA_i
        dB += dB_i      # disjoint batch entries per piece
        dC += dC_i
        dD += dD_i
        dbias += db_i
    out = dict(dx=dx, ddt=ddt, dA=dA, dB=dB, dC=dC, dh0=dh0)
    if D is not None:
        out["dD"] = dD
    if dt_bias is not None:
        out["ddt_bias"] = dbias
    return out
