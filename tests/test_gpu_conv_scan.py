"""GPU parity of the convolution fused into the scan (ss_fwd_conv).

Two checks per shape:
- the fused call gives the same bits as the convolution kernel followed by
  the scan on its output (out, last_state, the saved block states and
  pre-gate output, and the convolution's final window), which is what lets
  a training step run its backward through ss_bwd and ss_conv1d_bwd;
- the chain against the oracle: the f64 convolution, its output stored in
  the io dtype (u is an io tensor between the two layers), then the f64
  scan.

Shapes span several chunks and a ragged tail, the scalar-load path (rows
not 16-byte aligned), ragged channel counts, widths 1-4 with and without
SiLU, bias and initial window, 2-4 state slices in the lane, time segments
(8192 steps over 64 channels), and the full 8 x 1536 x 2048 bf16 forward.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import ORACLE_THREADS, DEV, dev_inputs, require_gpu, say, to_dev, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu


def conv_params(dim, width, batch, seed, bias=True, init=True):
    """Seeded convolution parameters with the distributions of the
    convolution workloads: weight and bias U(-1/sqrt(width), 1/sqrt(width)),
    initial window N(0, 1)."""
    rng = np.random.default_rng(seed)
    lim = 1.0 / np.sqrt(width)
    w = rng.uniform(-lim, lim, (dim, width)).astype(np.float32)
    b = rng.uniform(-lim, lim, dim).astype(np.float32) if bias else None
    h = rng.standard_normal((batch, dim, width - 1)).astype(np.float32) if init else None
    return w, b, h


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def as_io(u64, io):
    """The convolution's output as the io dtype stores it (u is an io tensor
    between the two layers): bf16 values are rounded to nearest even."""
    if io != "bf16":
        return u64
    return widen(ssin.bf16_bits(u64.astype(np.float32)))


def ckpt_parts(ck, batch, dim, N, L):
    """The written parts of a saved record: the block states of every slice,
    then (one slice only) the pre-gate output at the next 64-float boundary;
    the padding between them is never written."""
    slices = (N + 15) // 16
    n_states = slices * batch * dim * ((L + 15) // 16) * 16
    parts = [ck[:n_states]]
    if slices == 1:
        off = (n_states + 63) // 64 * 64
        parts.append(ck[off:off + batch * dim * L])
    return parts


CASES = [
    # batch, dim, dstate, L, io, width, silu, bias, init
    (2, 40, 16, 100, "f32", 4, True, True, True),
    (1, 17, 16, 33, "f32", 4, True, False, False),     # scalar path, ragged channels
    (2, 24, 16, 96, "bf16", 4, True, True, True),       # bf16, 16-byte slots
    (2, 40, 16, 136, "bf16", 3, True, True, False),     # ragged dim and tail
    (2, 24, 16, 70, "bf16", 2, False, True, True),      # scalar path, no SiLU
    (2, 32, 16, 64, "f32", 1, True, True, False),       # width 1: pointwise
    (2, 32, 40, 96, "bf16", 4, True, True, True),       # three slices in the lane
    (2, 48, 64, 70, "f32", 4, True, True, True),        # four slices, scalar path
    (2, 20, 5, 64, "f32", 4, True, True, True),         # fewer than 16 states
    (2, 64, 16, 8192, "bf16", 4, True, True, True),     # time segments
    (1, 40, 16, 9001, "f32", 3, True, True, True),      # time segments, scalar path
]


@pytest.mark.parametrize("batch,dim,N,L,io,width,silu,bias,init", CASES)
def test_fused_conv_scan(batch, dim, N, L, io, width, silu, bias, init):
    require_gpu()
    w = ssin.custom("fwd", batch, dim, N, L, io, seed=3 * dim + N + L + width)
    arr = ssin.make(w)
    say(f"fused conv {w.name} width {width} silu {silu}")
    d = dev_inputs(arr)
    cw, cb, ch = conv_params(dim, width, batch, seed=L + width, bias=bias, init=init)
    cw_d, cb_d, ch_d = to_dev(cw), to_dev(cb), to_dev(ch)
    h0 = torch.randn(batch, dim, N, device=DEV)
    x = d["u"]
    # the chain: convolution kernel, then the scan on its output
    u, fin_ref = binding.ss_conv1d_fwd(x, cw_d, cb_d, silu, ch_d, return_final_state=True)
    ck_ref = binding.ss_ckpt_empty(x, dstate=N)
    y_ref, last_ref = binding.ss_fwd(u, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                     d["delta_bias"], True, h0=h0, return_last_state=True,
                                     ckpt=ck_ref)
    # fused
    last = torch.empty_like(last_ref)
    fin = torch.empty_like(fin_ref)
    ck = binding.ss_ckpt_empty(x, dstate=N)
    y = binding.ss_fwd_conv(x, cw_d, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True, conv_bias=cb_d, conv_silu=silu,
                            conv_init=ch_d, h0=h0, last_state=last, conv_final=fin, ckpt=ck)
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(y_ref)), "out differs from the unfused chain"
    assert torch.equal(last, last_ref), "last_state differs from the unfused chain"
    for a, r in zip(ckpt_parts(ck, batch, dim, N, L), ckpt_parts(ck_ref, batch, dim, N, L)):
        assert torch.equal(a, r), "saved record differs from the unfused chain"
    assert torch.equal(fin, fin_ref), "conv_final differs from ss_conv1d_fwd's final_state"
    # against the oracle: f64 convolution, then the f64 scan
    xs = widen(arr["u"])
    u64, _ = oracle.conv_fwd(xs, cw.astype(np.float64),
                             None if cb is None else cb.astype(np.float64), silu,
                             None if ch is None else ch.astype(np.float64),
                             threads=ORACLE_THREADS)
    x64 = {k: widen(v) for k, v in arr.items()}
    ry, rl = oracle.fwd(as_io(u64, io), x64["delta"], x64["A"], x64["B"], x64["C"], x64["D"], x64["z"],
                        x64["delta_bias"], True, h0.cpu().numpy().astype(np.float64),
                        threads=ORACLE_THREADS)
    e = assert_close(to_host(y), ry, TOL[io], "out vs oracle chain")
    assert_close(to_host(last), rl, TOL[io], "last_state vs oracle chain")
    say(f"  err {e:.3e}")


def test_fused_conv_scan_full_size_rows_do_not_depend_on_batch():
    """The c1 bf16 forward shape (8 x 1536 x 2048) with a width-4 SiLU
    convolution: bit-equal to the unfused chain, every element against the
    oracle chain, and each batch entry alone equal to the same entry inside
    the batch."""
    require_gpu()
    w = ssin.WORKLOADS["mamba130m_fwd_bf16_8x1536x2048"]
    arr = ssin.make(w)
    d = dev_inputs(arr)
    cw, cb, _ = conv_params(w.dim, 4, w.batch, seed=11, init=False)
    cw_d, cb_d = to_dev(cw), to_dev(cb)
    x = d["u"]
    u = binding.ss_conv1d_fwd(x, cw_d, cb_d, True)
    y_ref = binding.ss_fwd(u, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                           d["delta_bias"], True)
    y = binding.ss_fwd_conv(x, cw_d, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True, conv_bias=cb_d)
    torch.cuda.synchronize()
    assert torch.equal(bits(y), bits(y_ref))
    for bi in (0, 5):
        one = {k: (v[bi:bi + 1].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
               for k, v in d.items()}
        ya = binding.ss_fwd_conv(one["u"], cw_d, one["delta"], one["A"], one["B"], one["C"],
                                 one["D"], one["z"], one["delta_bias"], True, conv_bias=cb_d)
        torch.cuda.synchronize()
        assert torch.equal(bits(ya[0]), bits(y[bi])), f"entry {bi}"
    say("fused conv full: oracle chain on the whole workload")
    x64 = {k: widen(v) for k, v in arr.items()}
    u64, _ = oracle.conv_fwd(x64["u"], cw.astype(np.float64), cb.astype(np.float64), True,
                             None, threads=ORACLE_THREADS)
    ry, _ = oracle.fwd(as_io(u64, "bf16"), x64["delta"], x64["A"], x64["B"], x64["C"], x64["D"], x64["z"],
                       x64["delta_bias"], True, threads=ORACLE_THREADS)
    e = assert_close(to_host(y), ry, TOL["bf16"], "out vs oracle chain")
    say(f"  err {e:.3e}")


def test_fused_conv_scan_zero_length_and_empty():
    require_gpu()
    w = ssin.custom("fwd", 2, 32, 16, 0, "f32", seed=2)
    d = dev_inputs(ssin.make(w))
    cw, cb, ch = conv_params(32, 4, 2, seed=1)
    h0 = torch.randn(2, 32, 16, device=DEV)
    last = torch.empty(2, 32, 16, device=DEV)
    fin = torch.empty(2, 32, 3, device=DEV)
    binding.ss_fwd_conv(d["u"], to_dev(cw), d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], True, conv_bias=to_dev(cb), conv_init=to_dev(ch), h0=h0,
                        last_state=last, conv_final=fin)
    torch.cuda.synchronize()
    assert torch.equal(last, h0)
    # seqlen 0: the final window is the initial one
    assert torch.equal(fin, to_dev(ch))


BWD_CASES = [
    # batch, dim, dstate, L, io, width, silu, bias, init
    (2, 40, 16, 100, "f32", 4, True, True, True),
    (1, 17, 16, 33, "f32", 4, True, False, False),     # scalar path, ragged channels
    (2, 24, 16, 96, "bf16", 4, True, True, True),
    (2, 40, 16, 136, "bf16", 3, True, True, False),     # ragged dim and tail
    (2, 24, 16, 70, "bf16", 2, False, True, True),      # scalar path, no SiLU
    (2, 32, 16, 64, "f32", 1, True, True, False),       # width 1
    (2, 20, 5, 64, "f32", 4, True, True, True),         # fewer than 16 states
    (8, 1544, 16, 64, "f32", 4, True, True, True),      # 48-channel reverse workgroups
    (2, 64, 16, 8192, "bf16", 4, True, True, True),     # time segments (boundary fix-up)
    (1, 40, 16, 9001, "f32", 3, True, True, True),      # time segments, scalar path
]

SCAN_KEYS = ("ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


@pytest.mark.parametrize("batch,dim,N,L,io,width,silu,bias,init", BWD_CASES)
def test_fused_conv_scan_backward(batch, dim, N, L, io, width, silu, bias, init):
    """ss_bwd_conv against the oracle chain (f64 convolution, its output
    stored in the io dtype, f64 scan and its backward, f64 convolution
    backward of the scan's du), and its scan gradients bit-equal to ss_bwd
    on the convolution kernel's u -- with and without the forward's saved
    record."""
    require_gpu()
    w = ssin.custom("bwd", batch, dim, N, L, io, seed=5 * dim + N + L + width)
    arr = ssin.make(w)
    say(f"fused conv bwd {w.name} width {width} silu {silu}")
    d = dev_inputs(arr)
    cw, cb, ch = conv_params(dim, width, batch, seed=2 * L + width, bias=bias, init=init)
    cw_d, cb_d, ch_d = to_dev(cw), to_dev(cb), to_dev(ch)
    rng = np.random.default_rng(L + width)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    dl = rng.standard_normal((batch, dim, N)).astype(np.float32)
    h0_d, dl_d = to_dev(h0), to_dev(dl)
    x = d["u"]
    u = binding.ss_conv1d_fwd(x, cw_d, cb_d, silu, ch_d)
    ck = binding.ss_ckpt_empty(x, dstate=N)
    binding.ss_fwd_conv(x, cw_d, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], True, conv_bias=cb_d, conv_silu=silu, conv_init=ch_d,
                        h0=h0_d, ckpt=ck)
    runs = {}
    for saved in (False, True):
        runs[saved] = binding.ss_bwd_conv(
            x, cw_d, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"], True,
            d["dout"], conv_bias=cb_d, conv_silu=silu, conv_init=ch_d, h0=h0_d, dlast=dl_d,
            want_dconv_init=True, ckpt=ck if saved else None)
        ref = binding.ss_bwd(u, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                             d["delta_bias"], True, d["dout"], h0=h0_d, dlast=dl_d,
                             ckpt=ck if saved else None)
        torch.cuda.synchronize()
        for k in SCAN_KEYS:
            if k in ref:
                assert torch.equal(bits(runs[saved][k]), bits(ref[k])), f"{k} saved={saved}"
    for k in runs[False]:
        assert torch.equal(bits(runs[False][k]), bits(runs[True][k])), f"{k} with saved record"
    g = runs[False]
    # the oracle chain
    x64 = {k: widen(v) for k, v in arr.items()}
    u64, _ = oracle.conv_fwd(x64["u"], cw.astype(np.float64),
                             None if cb is None else cb.astype(np.float64), silu,
                             None if ch is None else ch.astype(np.float64),
                             threads=ORACLE_THREADS)
    rs = oracle.bwd(as_io(u64, io), x64["delta"], x64["A"], x64["B"], x64["C"], x64["D"],
                    x64["z"], x64["delta_bias"], True, x64["dout"], h0.astype(np.float64),
                    dl.astype(np.float64), threads=ORACLE_THREADS)
    win = ch if ch is not None else np.zeros((batch, dim, width - 1), np.float32)
    rc = oracle.conv_bwd(x64["u"], cw.astype(np.float64),
                         None if cb is None else cb.astype(np.float64), silu,
                         win.astype(np.float64), rs["du"], threads=ORACLE_THREADS)
    checks = [("dx", rc["dx"], TOL[io]), ("dconv_weight", rc["dweight"], TOL["f32"]),
              ("dconv_init", rc["dinit_state"], TOL["f32"])]
    if cb is not None:
        checks.append(("dconv_bias", rc["dbias"], TOL["f32"]))
    for k in SCAN_KEYS:
        if k in rs and k in g:
            checks.append((k, rs[k], TOL["f32"] if k in ("dA", "dD", "ddelta_bias", "dh0")
                           else TOL[io]))
    for k, r, tol in checks:
        e = assert_close(to_host(g[k]), r, tol, f"{k} vs oracle chain")
        say(f"  {k} err {e:.3e}")


def test_fused_conv_scan_backward_rows_do_not_depend_on_batch():
    """Per-entry gradients (dx, ddelta, dz, dB, dC, the initial window's) of
    a batch entry run alone equal the same entry inside the batch, with time
    segments, and two calls give the same bits."""
    require_gpu()
    w = ssin.custom("bwd", 3, 64, 16, 8192, "bf16", seed=79)
    d = dev_inputs(ssin.make(w))
    cw, cb, ch = conv_params(64, 4, 3, seed=9)
    cw_d, cb_d, ch_d = to_dev(cw), to_dev(cb), to_dev(ch)

    def run(dd, init):
        return binding.ss_bwd_conv(dd["u"], cw_d, dd["delta"], dd["A"], dd["B"], dd["C"],
                                   dd["D"], dd["z"], dd["delta_bias"], True, dd["dout"],
                                   conv_bias=cb_d, conv_init=init)
    g1, g2 = run(d, ch_d), run(d, ch_d)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(bits(g1[k]), bits(g2[k])), f"{k} not deterministic"
    per_entry = ("u", "delta", "B", "C", "z", "dout")
    for bi in (0, 2):
        one = {k: (v[bi:bi + 1].contiguous() if k in per_entry else v) for k, v in d.items()}
        ga = run(one, ch_d[bi:bi + 1].contiguous())
        torch.cuda.synchronize()
        for k in ("dx", "ddelta", "dz", "dB", "dC", "dconv_init"):
            assert torch.equal(bits(ga[k]), bits(g1[k][bi:bi + 1])), f"{k} entry {bi}"


def test_fused_conv_scan_backward_zero_length():
    """seqlen 0: dlast passes through to dh0, the initial window and the
    parameter gradients are zero."""
    require_gpu()
    w = ssin.custom("bwd", 2, 32, 16, 0, "f32", seed=3)
    d = dev_inputs(ssin.make(w))
    cw, cb, ch = conv_params(32, 4, 2, seed=2)
    dl = torch.randn(2, 32, 16, device=DEV)
    g = binding.ss_bwd_conv(d["u"], to_dev(cw), d["delta"], d["A"], d["B"], d["C"], d["D"],
                            d["z"], d["delta_bias"], True, d["dout"], conv_bias=to_dev(cb),
                            conv_init=to_dev(ch), dlast=dl, want_dh0=True)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dl)
    for k in ("dconv_weight", "dconv_bias", "dconv_init", "dA", "dD", "ddelta_bias"):
        assert torch.count_nonzero(g[k]).item() == 0, k
