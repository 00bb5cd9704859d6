"""C ABI contract tests that need no GPU.

libss.so must load, export every function include/ss.h declares, report its
ABI version, and reject bad arguments on the host -- with a status and a
message naming the argument -- before anything reaches the device.  Every
call below either fails validation or has nothing to enqueue, so no HIP
call is made.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_scan_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss.h")
EINVAL, EUNSUP = binding.SS_EINVAL, binding.SS_EUNSUPPORTED
FAKE = 0x10000          # a 16-byte aligned non-null address (never dereferenced)
MISALIGNED = 0x10004
FAKE2 = 0x40000000     # another one, far from FAKE (no overlap of small tensors)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.lib_path()):
        from selective_state_space_scan_amd import build
        build.build()
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = re.findall(r"^\w[\w\s\*]*?\b(ss_\w+)\s*\(", open(HEADER).read(), flags=re.M)
    assert set(names) >= {"ss_fwd", "ss_bwd", "ss_bwd_workspace_size", "ss_state_update",
                          "ss_last_error", "ss_abi_version", "ss_fwd_conv", "ss_bwd_conv"}
    for n in names:
        assert hasattr(lib, n), f"libss.so does not export {n}"


def test_abi_version(lib):
    assert lib.ss_abi_version() == 12


def test_scan_regime_setting(lib):
    assert binding.scan_regime() == binding.SS_SCAN_AUTO
    try:
        for r in (binding.SS_SCAN_SEQUENTIAL, binding.SS_SCAN_SEGMENTED, binding.SS_SCAN_AUTO):
            binding.set_scan_regime(r)
            assert binding.scan_regime() == r
        binding.set_scan_regime(binding.SS_SCAN_SEGMENTED)
        assert lib.ss_set_scan_regime(3) == binding.SS_EINVAL
        assert b"regime" in lib.ss_last_error()
        assert binding.scan_regime() == binding.SS_SCAN_SEGMENTED   # unchanged by the refusal
    finally:
        binding.set_scan_regime(binding.SS_SCAN_AUTO)


def test_scan_regime_sizes_the_workspaces(lib):
    """Time segments need summary space: at 1 x 1536 x 2048 only the
    segmented regime cuts time, at 8192 steps the automatic one does too,
    and the sequential one never does."""
    def sizes(L):
        return (int(lib.ss_fwd_workspace_size(1, 1536, 16, L)),
                int(lib.ss_bwd_workspace_size(1, 1536, 16, L, binding.SS_BF16)))
    try:
        seq = {}
        for r in (binding.SS_SCAN_SEQUENTIAL, binding.SS_SCAN_AUTO, binding.SS_SCAN_SEGMENTED):
            binding.set_scan_regime(r)
            seq[r] = {L: sizes(L) for L in (512, 2048, 8192)}
    finally:
        binding.set_scan_regime(binding.SS_SCAN_AUTO)
    S, A, G = binding.SS_SCAN_SEQUENTIAL, binding.SS_SCAN_AUTO, binding.SS_SCAN_SEGMENTED
    assert seq[A][2048] == seq[S][2048] and seq[A][512] == seq[S][512]
    assert seq[G][512] == seq[S][512]                   # too short to cut
    assert seq[G][2048][0] > seq[S][2048][0]             # the forward's summaries
    assert seq[A][8192][0] > seq[S][8192][0] and seq[G][8192][0] >= seq[A][8192][0]


def test_ckpt_size(lib):
    lib.ss_ckpt_size.restype = ctypes.c_size_t
    lib.ss_ckpt_size.argtypes = [ctypes.c_int64] * 4
    # block states (256-byte aligned), then the pre-gate output
    assert lib.ss_ckpt_size(2, 32, 16, 64) == 2 * 32 * 4 * 16 * 4 + 2 * 32 * 64 * 4
    assert lib.ss_ckpt_size(2, 32, 16, 65) == 2 * 32 * 5 * 16 * 4 + 2 * 32 * 65 * 4
    assert lib.ss_ckpt_size(1, 1, 16, 1) == 256 + 4
    assert lib.ss_ckpt_size(2, 32, 16, 0) == 0
    # the block states are 16 wide for any dstate up to 16
    assert lib.ss_ckpt_size(2, 32, 8, 64) == lib.ss_ckpt_size(2, 32, 16, 64)
    # above 16: 16 states per slice; up to 64 states (slices in the lane)
    # still the pre-gate output after them, above 64 none
    assert lib.ss_ckpt_size(2, 32, 17, 64) == 2 * 2 * 32 * 4 * 16 * 4 + 2 * 32 * 64 * 4
    assert lib.ss_ckpt_size(2, 32, 64, 64) == 4 * 2 * 32 * 4 * 16 * 4 + 2 * 32 * 64 * 4
    assert lib.ss_ckpt_size(2, 32, 65, 64) == 5 * 2 * 32 * 4 * 16 * 4
    assert lib.ss_ckpt_size(2, 32, 256, 64) == 16 * 2 * 32 * 4 * 16 * 4
    assert lib.ss_ckpt_size(2, 32, 257, 64) == 0


def test_bwd_misaligned_ckpt(lib):
    assert _bwd(lib, ckpt=MISALIGNED) == EINVAL and "ckpt" in _msg(lib)


def _fwd(lib, batch=2, dim=32, dstate=16, seqlen=64, io=0, u=FAKE, delta=FAKE, A=FAKE, B=FAKE,
         C=FAKE, D=None, z=None, bias=None, h0=None, out=FAKE, last=None, ckpt=None, ws=None,
         ws_bytes=0):
    return lib.ss_fwd(batch, dim, dstate, seqlen, io, u, delta, A, B, C, D, z, bias, 1, h0, out,
                      last, ckpt, ws, ws_bytes, None)


def _msg(lib):
    return lib.ss_last_error().decode()


@pytest.mark.parametrize("arg", ["u", "delta", "A", "B", "C", "out"])
def test_fwd_null_required_pointer(lib, arg):
    assert _fwd(lib, **{arg: None}) == EINVAL
    assert arg in _msg(lib)


@pytest.mark.parametrize("arg", ["u", "A", "D", "z", "bias", "h0", "last", "ckpt"])
def test_fwd_misaligned_pointer(lib, arg):
    assert _fwd(lib, **{arg: MISALIGNED}) == EINVAL
    name = {"bias": "delta_bias", "last": "last_state"}.get(arg, arg)
    assert name in _msg(lib) and "aligned" in _msg(lib)


@pytest.mark.parametrize("kw,status,word", [
    (dict(batch=-1), EINVAL, "batch"), (dict(dim=-3), EINVAL, "dim"),
    (dict(seqlen=-1), EINVAL, "seqlen"), (dict(dstate=0), EINVAL, "dstate"),
    (dict(dstate=257), EUNSUP, "dstate"), (dict(dstate=1000), EUNSUP, "dstate"),
    (dict(io=7), EINVAL, "io_dtype"), (dict(batch=70000), EUNSUP, "batch"),
    (dict(seqlen=(1 << 26) + 1), EUNSUP, "seqlen"),
])
def test_fwd_bad_sizes(lib, kw, status, word):
    assert _fwd(lib, **kw) == status
    assert word in _msg(lib)


def test_fwd_empty_batch_is_a_noop(lib):
    # nothing to compute and no state to write: succeeds without touching the device
    assert _fwd(lib, batch=0, u=None, delta=None, B=None, C=None, out=None) == 0
    assert _msg(lib) == ""
    assert _fwd(lib, dim=0, u=None, delta=None, A=None, B=None, C=None, out=None) == 0


def test_fwd_last_state_must_not_alias_h0(lib):
    assert _fwd(lib, h0=FAKE, last=FAKE) == EINVAL
    assert "alias" in _msg(lib)


def _bwd(lib, batch=2, dim=32, dstate=16, seqlen=64, D=None, z=None, bias=None, dD=None, dz=None,
         dbias=None, ws=FAKE, ws_bytes=None, ckpt=None, **over):
    args = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, dout=FAKE, du=FAKE, ddelta=FAKE,
                dA=FAKE, dB=FAKE, dC=FAKE)
    args.update(over)
    if ws_bytes is None:
        ws_bytes = lib.ss_bwd_workspace_size(batch, dim, dstate, seqlen, 0)
    return lib.ss_bwd(batch, dim, dstate, seqlen, 0, args["u"], args["delta"], args["A"],
                      args["B"], args["C"], D, z, bias, 1, None, args["dout"], None, args["du"],
                      args["ddelta"], args["dA"], args["dB"], args["dC"], dD, dz, dbias, None,
                      ckpt, ws, ws_bytes, None)


@pytest.mark.parametrize("arg", ["u", "delta", "dout", "du", "ddelta", "dA", "dB", "dC", "A"])
def test_bwd_null_required_pointer(lib, arg):
    assert _bwd(lib, **{arg: None}) == EINVAL
    assert arg in _msg(lib)


@pytest.mark.parametrize("kw,word", [
    (dict(D=FAKE), "dD"), (dict(dD=FAKE), "dD"), (dict(z=FAKE), "dz"), (dict(dz=FAKE), "dz"),
    (dict(bias=FAKE), "ddelta_bias"), (dict(dbias=FAKE), "ddelta_bias"),
])
def test_bwd_gradient_presence_matches_input(lib, kw, word):
    assert _bwd(lib, **kw) == EINVAL
    assert word in _msg(lib)


def test_bwd_workspace_checks(lib):
    need = lib.ss_bwd_workspace_size(2, 32, 16, 64, 0)
    assert need > 0
    assert _bwd(lib, ws_bytes=need - 1) == EINVAL and "workspace_bytes" in _msg(lib)
    assert _bwd(lib, ws=None) == EINVAL and "workspace" in _msg(lib)
    assert _bwd(lib, ws=MISALIGNED) == EINVAL and "aligned" in _msg(lib)


def test_workspace_size_is_monotone_and_zero_when_invalid(lib):
    base = lib.ss_bwd_workspace_size(2, 32, 16, 64, 0)
    assert lib.ss_bwd_workspace_size(4, 32, 16, 64, 0) > base
    assert lib.ss_bwd_workspace_size(2, 64, 16, 64, 0) > base
    assert lib.ss_bwd_workspace_size(2, 32, 16, 128, 0) > base
    # internal buffers are 16 states wide for any dstate up to 16
    assert lib.ss_bwd_workspace_size(2, 32, 8, 64, 0) == base
    # above 16 states: per-slice partials and (slice, batch, dim, L) buffers
    assert lib.ss_bwd_workspace_size(2, 32, 17, 64, 0) > 2 * base
    assert lib.ss_bwd_workspace_size(2, 32, 257, 64, 0) == 0
    assert lib.ss_bwd_workspace_size(-1, 32, 16, 64, 0) == 0


def test_decode_checks(lib):
    st = lib.ss_state_update(4, 32, 16, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                             1, FAKE, None)
    assert st == EINVAL and "state" in _msg(lib)
    st = lib.ss_state_update(4, 32, 257, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                             1, FAKE, None)
    assert st == EUNSUP and "dstate" in _msg(lib)
    assert lib.ss_state_update(0, 32, 16, 1, None, None, None, None, None, None, None, None,
                               None, 1, None, None) == 0


def test_error_message_is_per_thread(lib):
    import threading
    assert _fwd(lib, u=None) == EINVAL
    seen = {}

    def other():
        seen["msg"] = lib.ss_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "u" in _msg(lib)


# ---------------------------------------------------------------------------
# causal convolution
# ---------------------------------------------------------------------------
def _cfwd(lib, batch=2, dim=8, seqlen=64, width=4, io=0, x=FAKE, w=FAKE, bias=None, init=None,
          out=FAKE, final=None):
    return lib.ss_conv1d_fwd(batch, dim, seqlen, width, io, x, w, bias, 1, init, out, final, None)


def _cbwd(lib, batch=2, dim=8, seqlen=64, width=4, x=FAKE, w=FAKE, bias=None, dout=FAKE, dx=FAKE,
          dw=FAKE, dbias=None, dinit=None):
    return lib.ss_conv1d_bwd(batch, dim, seqlen, width, 0, x, w, bias, 1, None, dout, dx, dw,
                             dbias, dinit, None)


@pytest.mark.parametrize("arg", ["x", "w", "out"])
def test_conv_fwd_null_required_pointer(lib, arg):
    assert _cfwd(lib, **{arg: None}) == EINVAL and _msg(lib).startswith(
        {"w": "weight"}.get(arg, arg))


@pytest.mark.parametrize("kw,status,word", [
    (dict(width=0), EINVAL, "width"), (dict(width=5), EUNSUP, "width"),
    (dict(seqlen=-1), EINVAL, "seqlen"), (dict(seqlen=(1 << 26) + 1), EUNSUP, "seqlen"),
    (dict(io=2), EINVAL, "io_dtype"), (dict(x=MISALIGNED), EINVAL, "aligned"),
])
def test_conv_fwd_bad_arguments(lib, kw, status, word):
    assert _cfwd(lib, **kw) == status and word in _msg(lib)


def test_conv_fwd_windows_must_not_overlap(lib):
    # (2 * 8 * 3) floats per window: a final window 16 bytes into the initial one overlaps it
    assert _cfwd(lib, init=FAKE, final=FAKE + 16) == EINVAL and "overlap" in _msg(lib)


def test_conv_empty_shapes_are_noops(lib):
    assert _cfwd(lib, batch=0, x=None, out=None) == 0
    assert _cbwd(lib, dim=0, x=None, w=None, dout=None, dx=None, dw=None) == 0
    assert lib.ss_conv1d_update(0, 8, 4, 0, None, None, None, None, 1, None, None) == 0


def test_conv_bwd_checks(lib):
    assert _cbwd(lib, bias=FAKE) == EINVAL and "dbias" in _msg(lib)
    assert _cbwd(lib, dbias=FAKE) == EINVAL and "dbias" in _msg(lib)
    assert _cbwd(lib, dw=None) == EINVAL and "dweight" in _msg(lib)
    assert _cbwd(lib, dout=None) == EINVAL and "dout" in _msg(lib)
    assert _cbwd(lib, width=5) == EUNSUP and "width" in _msg(lib)


def test_conv_update_checks(lib):
    st = lib.ss_conv1d_update(2, 8, 4, 0, None, FAKE, FAKE, None, 1, FAKE, None)
    assert st == EINVAL and "state" in _msg(lib)
    st = lib.ss_conv1d_update(2, 8, 5, 0, FAKE, FAKE, FAKE, None, 1, FAKE, None)
    assert st == EUNSUP and "width" in _msg(lib)


def _fwd_conv(lib, batch=2, dim=32, dstate=16, seqlen=64, io=0, x=FAKE, w=FAKE, width=4,
              cb=None, init=None, delta=FAKE, out=FAKE2, final=None):
    lib.ss_fwd_conv.argtypes = ([ctypes.c_int64] * 4 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                                + [ctypes.c_int64] + [ctypes.c_void_p] + [ctypes.c_int]
                                + [ctypes.c_void_p] * 8 + [ctypes.c_int] + [ctypes.c_void_p] * 6
                                + [ctypes.c_size_t, ctypes.c_void_p])
    return lib.ss_fwd_conv(batch, dim, dstate, seqlen, io, x, w, width, cb, 1, init, delta, FAKE,
                           FAKE, FAKE, None, None, None, 1, None, out, None, final, None, None, 0,
                           None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(width=5), EUNSUP, "width"), (dict(width=0), EINVAL, "width"),
    (dict(dstate=80), EUNSUP, "64"), (dict(dstate=300), EUNSUP, "dstate"),
    (dict(w=None), EINVAL, "conv_weight"), (dict(x=None), EINVAL, "x"),
    (dict(w=MISALIGNED), EINVAL, "aligned"), (dict(out=FAKE), EINVAL, "overlap x"),
    (dict(init=FAKE, final=FAKE), EINVAL, "conv_final"), (dict(seqlen=-1), EINVAL, "seqlen"),
])
def test_fwd_conv_checks(lib, kw, status, word):
    assert _fwd_conv(lib, **kw) == status
    assert word in _msg(lib)


def _bwd_conv(lib, batch=2, dim=32, dstate=16, seqlen=64, io=0, x=FAKE, w=FAKE, width=4,
              cb=None, dx=FAKE2, dw=FAKE, dcb=None):
    lib.ss_bwd_conv.argtypes = ([ctypes.c_int64] * 4 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                                + [ctypes.c_int64] + [ctypes.c_void_p] + [ctypes.c_int]
                                + [ctypes.c_void_p] * 8 + [ctypes.c_int] + [ctypes.c_void_p] * 17
                                + [ctypes.c_size_t, ctypes.c_void_p])
    # x, weight, width, bias, silu, init, delta, A, B, C, D, z, delta_bias, softplus, h0,
    # dout, dlast, dx, dweight, dbias, dinit, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
    # ckpt, workspace
    return lib.ss_bwd_conv(batch, dim, dstate, seqlen, io, x, w, width, cb, 1, None, FAKE, FAKE,
                           FAKE, FAKE, None, None, None, 1, None, FAKE, None, dx, dw, dcb, None,
                           FAKE, FAKE, FAKE, FAKE, None, None, None, None, None, FAKE, 1 << 40,
                           None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(width=5), EUNSUP, "width"), (dict(dstate=17), EUNSUP, "16 states"),
    (dict(dx=None), EINVAL, "dx"), (dict(dw=None), EINVAL, "dconv_weight"),
    (dict(w=None), EINVAL, "conv_weight"), (dict(x=None), EINVAL, "x"),
    (dict(dcb=FAKE), EINVAL, "dconv_bias"), (dict(dx=FAKE), EINVAL, "overlap x"),
])
def test_bwd_conv_checks(lib, kw, status, word):
    assert _bwd_conv(lib, **kw) == status
    assert word in _msg(lib)


def test_fwd_workspace(lib):
    # no workspace up to 64 states (the slices of a row run in the same
    # lanes); above, one f32 partial per slice and element
    assert lib.ss_fwd_workspace_size(2, 32, 16, 64) == 0
    assert lib.ss_fwd_workspace_size(2, 32, 17, 64) == 0
    assert lib.ss_fwd_workspace_size(2, 32, 64, 64) == 0
    assert lib.ss_fwd_workspace_size(2, 32, 65, 64) == 5 * 2 * 32 * 64 * 4
    assert lib.ss_fwd_workspace_size(2, 32, 256, 64) == 16 * 2 * 32 * 64 * 4
    assert lib.ss_fwd_workspace_size(2, 32, 257, 64) == 0
    need = lib.ss_fwd_workspace_size(2, 32, 80, 64)
    assert _fwd(lib, dstate=80) == EINVAL and "workspace" in _msg(lib)
    assert _fwd(lib, dstate=80, ws=FAKE, ws_bytes=need - 1) == EINVAL and "workspace_bytes" in _msg(lib)
    assert _fwd(lib, dstate=80, ws=MISALIGNED, ws_bytes=need) == EINVAL and "aligned" in _msg(lib)
    # time segments: the segment summaries, 2 x slices x (nseg - 1) x batch
    # x dim x 16 floats (64 channels, 8192 steps: 8 segments; 12288 channels
    # fill the chip without them; fewer than 8192 steps never take them)
    assert lib.ss_fwd_workspace_size(1, 12288, 16, 8192) == 0
    assert lib.ss_fwd_workspace_size(1, 64, 16, 8191) == 0
    assert lib.ss_fwd_workspace_size(1, 64, 16, 8192) == 2 * 7 * 64 * 16 * 4
    assert lib.ss_fwd_workspace_size(3, 64, 16, 8192) == 3 * 2 * 7 * 64 * 16 * 4



# ---------------------------------------------------------------------------
# Mamba-2 SSD
# ---------------------------------------------------------------------------
def _ssd(lib, batch=2, seqlen=64, nheads=4, headdim=64, ngroups=1, dstate=128, io=1, x=FAKE,
         dt=FAKE, A=FAKE, B=FAKE, C=FAKE, out=FAKE, h0=None, last=None, ckpt=None):
    return lib.ss_ssd_fwd(batch, seqlen, nheads, headdim, ngroups, dstate, io, x, dt, A, B, C,
                          None, None, 1, h0, out, last, ckpt, None)


@pytest.mark.parametrize("kw,status,word", [
    (dict(io=0), EUNSUP, "bf16"), (dict(headdim=24), EUNSUP, "headdim"),
    (dict(dstate=16), EUNSUP, "dstate"), (dict(dstate=256), EUNSUP, "dstate"),
    (dict(ngroups=3), EINVAL, "ngroups"), (dict(ngroups=0), EINVAL, "ngroups"),
    (dict(seqlen=-1), EINVAL, "seqlen"), (dict(x=None), EINVAL, "x"),
    (dict(B=MISALIGNED), EINVAL, "aligned"), (dict(A=None), EINVAL, "A"),
])
def test_ssd_bad_arguments(lib, kw, status, word):
    assert _ssd(lib, **kw) == status and word in _msg(lib)


def test_ssd_dt_needs_only_element_alignment(lib):
    # validation passes for a dt at a 2-byte offset; the call then has nothing to run
    assert _ssd(lib, batch=0, dt=FAKE + 2) == 0
    assert _ssd(lib, dt=FAKE + 1) == EINVAL and "dt" in _msg(lib)


def test_ssd_ckpt_size_and_checks(lib):
    lib.ss_ssd_ckpt_size.restype = ctypes.c_size_t
    # one f32 dstate x headdim state per (batch, head, chunk of 64 steps)
    assert lib.ss_ssd_ckpt_size(2, 130, 4, 64, 128) == 2 * 4 * 3 * 128 * 64 * 4
    assert lib.ss_ssd_ckpt_size(2, 0, 4, 64, 128) == 0
    assert lib.ss_ssd_ckpt_size(2, 64, 4, 64, 256) == 0
    assert _ssd(lib, ckpt=MISALIGNED) == EINVAL and "ckpt" in _msg(lib)
    assert _ssd(lib, h0=FAKE, ckpt=FAKE + 256) == EINVAL and "overlap" in _msg(lib)


def test_ssd_state_overlap_and_empty(lib):
    assert _ssd(lib, h0=FAKE, last=FAKE + 256) == EINVAL and "overlap" in _msg(lib)
    assert _ssd(lib, batch=0, x=None, dt=None, B=None, C=None, out=None) == 0
    assert _ssd(lib, nheads=0, A=None, x=None, dt=None, B=None, C=None, out=None) == 0



def test_ssd_bwd_checks(lib):
    def bwd(**kw):
        a = dict(batch=2, seqlen=64, nheads=4, headdim=64, ngroups=1, dstate=128, io=1, x=FAKE,
                 dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, bias=None, h0=None, dout=FAKE, dlast=None,
                 dx=FAKE, ddt=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dbias=None, dh0=None,
                 ckpt=None, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return lib.ss_ssd_bwd(a["batch"], a["seqlen"], a["nheads"], a["headdim"], a["ngroups"],
                              a["dstate"], a["io"], a["x"], a["dt"], a["A"], a["B"], a["C"],
                              a["D"], a["bias"], 1, a["h0"], a["dout"], a["dlast"], a["dx"],
                              a["ddt"], a["dA"], a["dB"], a["dC"], a["dD"], a["dbias"], a["dh0"],
                              a["ckpt"], a["ws"], a["ws_bytes"], None)
    assert bwd(dout=None) == EINVAL and "dout" in _msg(lib)
    assert bwd(ckpt=MISALIGNED) == EINVAL and "ckpt" in _msg(lib)
    assert bwd(batch=1024, nheads=1024, seqlen=1 << 20) == EUNSUP and "seqlen / 64" in _msg(lib)
    assert bwd(D=FAKE) == EINVAL and "dD" in _msg(lib)
    assert bwd(io=0) == EUNSUP and "bf16" in _msg(lib)
    need = lib.ss_ssd_bwd_workspace_size(2, 64, 4, 64, 1, 128)
    assert need > 0
    assert bwd(ws_bytes=need - 1) == EINVAL and "workspace_bytes" in _msg(lib)
    assert bwd(ws=None) == EINVAL and "workspace" in _msg(lib)
    assert lib.ss_ssd_bwd_workspace_size(2, 64, 4, 64, 1, 256) == 0
    # nothing to launch without heads (an empty batch still zeroes dA on the device)
    assert bwd(nheads=0, A=None, dA=None, x=None, B=None, C=None, dout=None, dx=None, dB=None,
               dC=None) == 0


# ---------------------------------------------------------------------------
# launch grids: HIP takes at most 2^32 - 1 work-items along a grid dimension;
# shapes past it are refused on the host as unsupported, not left to fail at
# launch
# ---------------------------------------------------------------------------
def test_scan_grid_limit(lib):
    # 2^28 + 16 channels fit the dim limit but not 16 channels per 256 threads
    dim = (1 << 28) + 16
    assert _fwd(lib, batch=1, dim=dim, seqlen=16) == EUNSUP and "2^32" in _msg(lib)
    assert _bwd(lib, batch=1, dim=dim, seqlen=16, ws_bytes=1 << 60) == EUNSUP
    assert "2^32" in _msg(lib)
    # the largest dim whose grid fits passes the grid check (and fails later, on
    # the missing workspace-free pointers it is not given)
    assert _fwd(lib, batch=1, dim=(1 << 28) - 16, seqlen=16, u=None) == EINVAL


def test_slice_combine_and_fold_grid_limits(lib):
    # several state slices: one elementwise combine pass over batch * dim * seqlen
    assert _fwd(lib, batch=65535, dim=1 << 16, dstate=32, seqlen=1 << 14) == EUNSUP
    assert "combine" in _msg(lib)
    # the backward's fold: batch * dstate * seqlen / 4 items
    assert _bwd(lib, batch=65535, dim=16, seqlen=1 << 26, ws_bytes=1 << 60) == EUNSUP
    assert "fold" in _msg(lib)


def test_decode_grid_limit(lib):
    # one grid row per batch entry: at most 65535 of them
    st = lib.ss_state_update(1 << 20, 1 << 11, 16, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                             None, None, 1, FAKE, None)
    assert st == EUNSUP and "65535" in _msg(lib)


def test_conv_and_ssd_grid_limits(lib):
    # the convolution's backward takes one 128-thread block per channel
    assert _cbwd(lib, batch=1, dim=1 << 26, seqlen=16) == EUNSUP and "2^32" in _msg(lib)
    # the SSD kernels take one block of up to 1024 threads per (batch, head)
    assert _ssd(lib, batch=1 << 12, nheads=1 << 12) == EUNSUP and "2^32" in _msg(lib)
    assert _ssd(lib, batch=1 << 10, nheads=1 << 12) == EUNSUP and "2^32" in _msg(lib)


def test_bwd_noalloc_validates_like_ss_bwd(lib):
    binding.load()   # sets the argument types
    assert lib.ss_bwd_noalloc_max_scratch() == 96 << 20

    def call(**over):
        a = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, dout=FAKE, du=FAKE, ddelta=FAKE,
                 dA=FAKE, dB=FAKE, dC=FAKE, D=None, dD=None, ckpt=None, batch=2, dim=32, seqlen=64)
        a.update(over)
        return lib.ss_bwd_noalloc(a["batch"], a["dim"], 16, a["seqlen"], 0, a["u"], a["delta"],
                                  a["A"], a["B"], a["C"], a["D"], None, None, 1, None, a["dout"],
                                  None, a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"],
                                  None, None, None, a["ckpt"], None)
    assert call(u=None) == EINVAL and "u" in _msg(lib)
    assert call(D=FAKE) == EINVAL and "dD" in _msg(lib)
    assert call(ckpt=MISALIGNED) == EINVAL and "ckpt" in _msg(lib)
    assert call(dim=(1 << 28) + 16, seqlen=16) == EUNSUP and "2^32" in _msg(lib)
    # nothing to run: succeeds without touching the device
    assert call(batch=0, u=None, delta=None, dout=None, du=None, ddelta=None, B=None, C=None,
                dB=None, dC=None, dA=None, A=None, dim=0) == 0
