"""The segmented scan regime (ss_set_scan_regime(SS_SCAN_SEGMENTED)): time
segments for narrow calls from 1024 steps on, which the automatic regime
keeps sequential below 8192 steps.  Each regime is its own bit family
(mamba-rs GEMM-modes page, "What is guaranteed": the sequential and the
parallel scan regimes): checked against the f64 oracle element by element,
run to run and batch entry by batch entry bit for bit."""
import contextlib

import numpy as np
import pytest
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import ORACLE_THREADS, DEV, dev_inputs, oracle_fwd, require_gpu, say, to_dev, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu

KEYS = ["du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0"]


@contextlib.contextmanager
def regime(r):
    binding.set_scan_regime(r)
    try:
        yield
    finally:
        binding.set_scan_regime(binding.SS_SCAN_AUTO)


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def run_fwd(d, w, h0=None):
    return binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"), d.get("z"),
                          d.get("delta_bias"), w.softplus, h0=h0, return_last_state=True)


def run_bwd(d, w, h0=None, dlast=None, ckpt=None):
    return binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"), d.get("z"),
                          d.get("delta_bias"), w.softplus, d["dout"], h0=h0, dlast=dlast,
                          want_dh0=True, ckpt=ckpt)


# batch, dim, dstate, seqlen, io: 3, 4 and 3 segments (the last ragged)
CASES = [
    (2, 64, 16, 1536, "f32"),
    (1, 48, 16, 2100, "bf16"),
    (2, 40, 5, 1100, "f32"),
]


@pytest.mark.parametrize("batch,dim,N,L,io", CASES)
def test_segmented_regime_against_the_oracle(batch, dim, N, L, io):
    require_gpu()
    w = ssin.custom("bwd", batch, dim, N, L, io, seed=7 * dim + L)
    arr = ssin.make(w)
    say(f"segmented regime {w.name}")
    d = dev_inputs(arr)
    rng = np.random.default_rng(L)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    dl = rng.standard_normal((batch, dim, N)).astype(np.float32)
    with regime(binding.SS_SCAN_SEGMENTED):
        y, last = run_fwd(d, w, h0=to_dev(h0))
        g = run_bwd(d, w, h0=to_dev(h0), dlast=to_dev(dl))
        ck = binding.ss_ckpt_empty(d["u"], dstate=N)
        binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], w.softplus, h0=to_dev(h0), ckpt=ck)
        g2 = run_bwd(d, w, h0=to_dev(h0), dlast=to_dev(dl), ckpt=ck)
    with regime(binding.SS_SCAN_SEQUENTIAL):
        _, lasts = run_fwd(d, w, h0=to_dev(h0))
    torch.cuda.synchronize()
    ry, rl = oracle_fwd(arr, w.softplus, h0=h0.astype(np.float64))
    assert_close(to_host(y), ry, TOL[io], "y")
    assert_close(to_host(last), rl, TOL["f32"], "last_state")
    x = {k: widen(v) for k, v in arr.items()}
    ref = oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"),
                     x.get("delta_bias"), w.softplus, x["dout"], h0.astype(np.float64),
                     dl.astype(np.float64), threads=ORACLE_THREADS)
    for k in KEYS:
        tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias", "dh0") else TOL[io]
        e = assert_close(to_host(g[k]), ref[k], tol, f"{k} segmented regime")
        say(f"  {k} err {e:.3e}")
    # the forward's saved record gives the bits of recomputing it
    for k in g:
        assert torch.equal(bits(g[k]), bits(g2[k])), f"{k} with the saved record"
    # the regime took effect: the segmented forward is another bit family
    # (seen in the f32 final state; a bf16 output can round to the same bits)
    assert not torch.equal(last, lasts)


def test_segmented_regime_batch_invariant_and_deterministic():
    require_gpu()
    w = ssin.custom("bwd", 3, 64, 16, 2048, "bf16", seed=91)
    d = dev_inputs(ssin.make(w))
    h0 = torch.randn(3, 64, 16, device=DEV)
    dl = torch.randn(3, 64, 16, device=DEV)
    per_entry = ("u", "delta", "B", "C", "z", "dout")
    with regime(binding.SS_SCAN_SEGMENTED):
        y1, l1 = run_fwd(d, w, h0=h0)
        y2, l2 = run_fwd(d, w, h0=h0)
        g1 = run_bwd(d, w, h0=h0, dlast=dl)
        g2 = run_bwd(d, w, h0=h0, dlast=dl)
        torch.cuda.synchronize()
        assert torch.equal(bits(y1), bits(y2)) and torch.equal(l1, l2)
        for k in g1:
            assert torch.equal(bits(g1[k]), bits(g2[k])), f"{k} not deterministic"
        for bi in range(w.batch):
            one = {k: (v[bi:bi + 1].contiguous() if k in per_entry else v) for k, v in d.items()}
            ya, la = run_fwd(one, w, h0=h0[bi:bi + 1].contiguous())
            ga = run_bwd(one, w, h0=h0[bi:bi + 1].contiguous(), dlast=dl[bi:bi + 1].contiguous())
            torch.cuda.synchronize()
            assert torch.equal(bits(ya[0]), bits(y1[bi])), f"y entry {bi}"
            assert torch.equal(la[0], l1[bi]), f"last_state entry {bi}"
            for k in ("du", "ddelta", "dz", "dB", "dC", "dh0"):
                assert torch.equal(bits(g1[k][bi:bi + 1]), bits(ga[k])), f"{k} entry {bi}"


def test_segmented_regime_leaves_short_and_wide_calls_sequential():
    """Below 1024 steps, and for calls whose batch entry already fills the
    chip (3072 wavefronts: 12288 channels), the segmented regime gives the
    sequential bits."""
    require_gpu()
    for (batch, dim, L) in ((2, 64, 1000), (1, 12288, 1024)):
        w = ssin.custom("fwd", batch, dim, 16, L, "bf16", seed=dim + L)
        d = dev_inputs(ssin.make(w))
        with regime(binding.SS_SCAN_SEGMENTED):
            ya, la = run_fwd(d, w)
        with regime(binding.SS_SCAN_SEQUENTIAL):
            yb, lb = run_fwd(d, w)
        torch.cuda.synchronize()
        assert torch.equal(bits(ya), bits(yb)) and torch.equal(la, lb), f"{batch}x{dim}x{L}"


def test_segmented_regime_fused_convolution_matches_the_separate_calls():
    """In the segmented regime too, the convolution fused into the scan
    gives the bits of the separate convolution followed by the scan, forward
    and backward (the fused backward's scan gradients, and its record-based
    run the recomputing one's)."""
    require_gpu()
    batch, dim, N, L, width = 2, 40, 16, 2100, 4
    w = ssin.custom("bwd", batch, dim, N, L, "bf16", seed=4 * dim + L)
    d = dev_inputs(ssin.make(w))
    rng = np.random.default_rng(L)
    lim = 1.0 / np.sqrt(width)
    cw = to_dev(rng.uniform(-lim, lim, (dim, width)).astype(np.float32))
    cb = to_dev(rng.uniform(-lim, lim, dim).astype(np.float32))
    ch = to_dev(rng.standard_normal((batch, dim, width - 1)).astype(np.float32))
    x = d["u"]
    with regime(binding.SS_SCAN_SEGMENTED):
        u = binding.ss_conv1d_fwd(x, cw, cb, True, ch)
        yf = binding.ss_fwd_conv(x, cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                 d["delta_bias"], True, conv_bias=cb, conv_init=ch)
        ys = binding.ss_fwd(u, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True)
        ck = binding.ss_ckpt_empty(x, dstate=N)
        binding.ss_fwd_conv(x, cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True, conv_bias=cb, conv_init=ch, ckpt=ck)
        gf = binding.ss_bwd_conv(x, cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                 d["delta_bias"], True, d["dout"], conv_bias=cb, conv_init=ch)
        gk = binding.ss_bwd_conv(x, cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                 d["delta_bias"], True, d["dout"], conv_bias=cb, conv_init=ch,
                                 ckpt=ck)
        gs = binding.ss_bwd(u, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True, d["dout"])
    torch.cuda.synchronize()
    assert torch.equal(bits(yf), bits(ys))
    for k in ("ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias"):
        assert torch.equal(bits(gf[k]), bits(gs[k])), k
    for k in gf:
        assert torch.equal(bits(gf[k]), bits(gk[k])), f"{k} with the saved record"
