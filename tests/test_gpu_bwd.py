"""GPU parity of the backward (ss_bwd through the C ABI) with the oracle.

Small shapes are compared element by element for every gradient; they span
several chunks, ragged time tails and channel counts, the scalar-load path,
each optional input on and off, an initial state with its gradient and a
gradient on the last state.  The full-size workload runs in the benchmark's
launch configuration and is checked on sampled rows (du, ddelta, dz), one
whole batch entry (dB, dC) and sampled channels (dA, dD, ddelta_bias), plus
run-to-run bit equality.
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

KEYS = ["du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0"]


def run_bwd(d, w, h0=None, dlast=None, want_dh0=False):
    return binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"), d.get("z"),
                          d.get("delta_bias"), w.softplus, d["dout"], h0=h0, dlast=dlast,
                          want_dh0=want_dh0)


def oracle_bwd(arr, w, h0=None, dlast=None, threads=8):
    x = {k: widen(v) for k, v in arr.items()}
    return oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"),
                      x.get("delta_bias"), w.softplus, x["dout"], h0, dlast, threads=threads)


SMALL = [
    (2, 40, 100, "f32", {}),
    (1, 17, 33, "f32", {}),
    (2, 32, 64, "f32", dict(has_z=False)),
    (2, 32, 64, "f32", dict(has_D=False)),
    (2, 32, 64, "f32", dict(has_bias=False)),
    (2, 32, 64, "f32", dict(softplus=False)),
    (3, 16, 1, "f32", {}),
    (2, 24, 70, "bf16", {}),                      # bf16 rows not 16-byte aligned (scalar path)
    (2, 24, 96, "bf16", {}),                      # bf16, 16-byte slots
    (2, 40, 136, "bf16", {}),                     # bf16, 16-byte slots, ragged dim and tail
    # Enough 48-channel groups to fill a 256-CU device: these take the
    # 12-wavefront reverse pass (the first with a last group of 8 channels).
    (8, 1544, 64, "f32", {}),
    (8, 1536, 96, "bf16", {}),
]


@pytest.mark.parametrize("batch,dim,L,io,flags", SMALL)
def test_bwd_small_elementwise(batch, dim, L, io, flags):
    require_gpu()
    w = ssin.custom("bwd", batch, dim, 16, L, io, seed=7 * batch + dim + L, **flags)
    arr = ssin.make(w)
    if not w.softplus:
        arr["delta"] = (np.abs(ssin.widen(arr["delta"])) + 0.05).astype(np.float32)
        if "delta_bias" in arr:
            arr["delta_bias"] = np.linspace(0.0, 0.1, dim).astype(np.float32)
    say(f"bwd small {w.name}")
    d = dev_inputs(arr)
    rng = np.random.default_rng(9)
    h0 = rng.standard_normal((batch, dim, 16)).astype(np.float32)
    dl = rng.standard_normal((batch, dim, 16)).astype(np.float32)
    for use_state in (False, True):
        g = run_bwd(d, w, h0=to_dev(h0) if use_state else None,
                    dlast=to_dev(dl) if use_state else None, want_dh0=True)
        torch.cuda.synchronize()
        ref = oracle_bwd(arr, w, h0=h0.astype(np.float64) if use_state else None,
                         dlast=dl.astype(np.float64) if use_state else None)
        if not use_state:
            # gradient at a zero initial state: the oracle reports it when h0 is given
            ref["dh0"] = oracle_bwd(arr, w, h0=np.zeros((batch, dim, 16)))["dh0"]
        for k in KEYS:
            if k not in ref:
                assert k not in g
                continue
            tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias", "dh0") else TOL[io]
            assert_close(to_host(g[k]), ref[k], tol, f"{k} state={use_state}")


@pytest.mark.parametrize("batch,dim,L,io", [(2, 40, 100, "f32"), (1, 33, 70, "bf16"),
                                             (2, 24, 96, "bf16"), (2, 16, 17, "f32"),
                                             (8, 1544, 64, "f32")])
def test_bwd_with_forward_checkpoints_is_bit_identical(batch, dim, L, io):
    """Checkpoints saved by the forward give the same bits as recomputing them."""
    require_gpu()
    w = ssin.custom("bwd", batch, dim, 16, L, io, seed=L + dim)
    arr = ssin.make(w)
    d = dev_inputs(arr)
    h0 = torch.randn(batch, dim, 16, device=DEV)
    ck = binding.ss_ckpt_empty(d["u"])
    binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                   True, h0=h0, ckpt=ck)
    g1 = binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], True, d["dout"], h0=h0)
    g2 = binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], True, d["dout"], h0=h0, ckpt=ck)
    torch.cuda.synchronize()
    for k in g1:
        a, b2 = g1[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), k


@pytest.mark.parametrize("dim,L,io", [(1536, 64, "f32"), (1544, 96, "bf16")])
def test_bwd_rows_do_not_depend_on_batch(dim, L, io):
    """A batch entry's du, ddelta, dz, dB and dC are the same bits run alone
    as inside a batch of 8.  On a 256-CU device the batch of 8 takes the
    48-channel reverse pass and the single entry the 16-channel one, so this
    also pins their common order of the sums over channels."""
    require_gpu()
    w = ssin.custom("bwd", 8, dim, 16, L, io, seed=dim + L)
    d = dev_inputs(ssin.make(w))
    g = run_bwd(d, w)
    per_entry = ("u", "delta", "B", "C", "z", "dout")
    for bi in (0, 5):
        one = {k: (v[bi:bi + 1].contiguous() if k in per_entry else v) for k, v in d.items()}
        g1 = run_bwd(one, w)
        torch.cuda.synchronize()
        for k in ("du", "ddelta", "dz", "dB", "dC"):
            a, b1 = g[k][bi:bi + 1], g1[k]
            if a.dtype == torch.bfloat16:
                a, b1 = a.view(torch.int16), b1.view(torch.int16)
            assert torch.equal(a, b1), f"{k} entry {bi}"


@pytest.mark.parametrize("batch,dim,N,L,io", [(2, 40, 1, 64, "f32"), (2, 40, 5, 96, "bf16"),
                                              (2, 24, 12, 70, "f32"), (8, 1544, 8, 64, "f32"),
                                              (2, 40, 17, 64, "f32"), (2, 40, 48, 96, "bf16"),
                                              (2, 24, 100, 70, "f32"), (2, 40, 256, 32, "f32"),
                                              (8, 1544, 64, 64, "f32")])
def test_bwd_smaller_dstate(batch, dim, N, L, io):
    """d_state other than 16, every gradient against the oracle (the
    1544-channel shapes take the 48-channel reverse pass; above 16 states the
    slices run one launch each and chain their du and ddelta sums up to 64
    states, and go through the combine kernel above), and a backward with
    the forward's saved record giving the same bits as one that recomputes
    it."""
    require_gpu()
    w = ssin.custom("bwd", batch, dim, N, L, io, seed=17 * N + L + dim)
    arr = ssin.make(w)
    say(f"bwd dstate {w.name}")
    d = dev_inputs(arr)
    rng = np.random.default_rng(N + 1)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    dl = rng.standard_normal((batch, dim, N)).astype(np.float32)
    g = run_bwd(d, w, h0=to_dev(h0), dlast=to_dev(dl), want_dh0=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(arr, w, h0=h0.astype(np.float64), dlast=dl.astype(np.float64))
    for k in KEYS:
        if k not in ref:
            continue
        tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias", "dh0") else TOL[io]
        assert_close(to_host(g[k]), ref[k], tol, f"{k} N={N}")
    ck = binding.ss_ckpt_empty(d["u"], dstate=N)
    binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                   w.softplus, h0=to_dev(h0), ckpt=ck)
    g2 = binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], w.softplus, d["dout"], h0=to_dev(h0), dlast=to_dev(dl),
                        want_dh0=True, ckpt=ck)
    torch.cuda.synchronize()
    for k in g:
        a, b2 = g[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), f"{k} with saved record"


@pytest.mark.parametrize("batch,dim,N,L,io", [(2, 40, 40, 96, "f32"), (2, 24, 100, 70, "bf16"),
                                              (8, 1544, 33, 64, "f32")])
def test_bwd_slices_without_gate(batch, dim, N, L, io):
    """Without z no slice needs dz partials, so at any d_state above 16 the
    slices chain their du and ddelta sums launch after launch (the last adds
    D dy): every gradient against the oracle, and the same bits on a second
    call."""
    require_gpu()
    w = ssin.custom("bwd", batch, dim, N, L, io, seed=31 * N + L, has_z=False)
    arr = ssin.make(w)
    say(f"bwd no gate {w.name}")
    d = dev_inputs(arr)
    g = run_bwd(d, w)
    g2 = run_bwd(d, w)
    torch.cuda.synchronize()
    ref = oracle_bwd(arr, w)
    for k in KEYS:
        if k not in ref:
            continue
        tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias") else TOL[io]
        assert_close(to_host(g[k]), ref[k], tol, f"{k} N={N}")
    for k in g:
        a, b2 = g[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), f"{k} differs between calls"


def test_bwd_zero_length_passes_dlast_through():
    require_gpu()
    w = ssin.custom("bwd", 2, 32, 16, 0, "f32", seed=4)
    d = dev_inputs(ssin.make(w))
    dl = torch.randn(2, 32, 16, device=DEV)
    g = run_bwd(d, w, dlast=dl, want_dh0=True)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dl)
    for k in ("dA", "dD", "ddelta_bias"):
        assert torch.count_nonzero(g[k]).item() == 0


def test_bwd_full_size_whole_tensors():
    """The backward workload at full size (8 x 1536 x 2048, f32), in the
    launch configuration the benchmark times, against the oracle on every
    element of every gradient."""
    require_gpu()
    w = ssin.WORKLOADS["mamba130m_bwd_f32_8x1536x2048"]
    say("bwd full: generating inputs")
    arr = ssin.make(w)
    d = dev_inputs(arr)
    say("bwd full: running twice")
    g1 = run_bwd(d, w)
    g2 = run_bwd(d, w)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), f"{k} not deterministic"
    x = {k: widen(v) for k, v in arr.items()}
    tol = TOL["f32"]
    say(f"bwd full: oracle on the whole workload ({ORACLE_THREADS} threads)")
    ref = oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                     x["delta_bias"], True, x["dout"], threads=ORACLE_THREADS)
    for k in ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddelta_bias"):
        e = assert_close(to_host(g1[k]), ref[k], tol, k)
        say(f"  {k} err {e:.3e}")


# Long sequences over few channels: the backward cuts time into the
# forward's segments (block states after the forward's summary pass, the
# reverse pass after an adjoint summary pass).
SEGMENTED = [
    # batch, dim, dstate, L, io
    (2, 64, 16, 8192, "f32"),        # 8 segments of 1024 steps
    (2, 48, 16, 8229, "bf16"),       # segments of 1088 steps, a short ragged last one
    (1, 40, 16, 9001, "f32"),        # rows not 16-byte aligned (scalar path), ragged channels
    (2, 32, 40, 8300, "bf16"),       # three 16-state slices x 8 segments
]


@pytest.mark.parametrize("batch,dim,N,L,io", SEGMENTED)
def test_bwd_time_segments_elementwise(batch, dim, N, L, io):
    """Every gradient against the oracle, with an initial state and a
    gradient on the last state, and the forward's saved record giving the
    same bits as recomputing the block states."""
    require_gpu()
    w = ssin.custom("bwd", batch, dim, N, L, io, seed=batch + dim + N + L)
    arr = ssin.make(w)
    say(f"bwd segmented {w.name}")
    d = dev_inputs(arr)
    rng = np.random.default_rng(L + 3)
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32)
    dl = rng.standard_normal((batch, dim, N)).astype(np.float32)
    g = run_bwd(d, w, h0=to_dev(h0), dlast=to_dev(dl), want_dh0=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(arr, w, h0=h0.astype(np.float64), dlast=dl.astype(np.float64),
                     threads=ORACLE_THREADS)
    for k in KEYS:
        if k not in ref:
            continue
        tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias", "dh0") else TOL[io]
        e = assert_close(to_host(g[k]), ref[k], tol, f"{k} segmented")
        say(f"  {k} err {e:.3e}")
    ck = binding.ss_ckpt_empty(d["u"], dstate=N)
    binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                   w.softplus, h0=to_dev(h0), ckpt=ck)
    g2 = binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], w.softplus, d["dout"], h0=to_dev(h0), dlast=to_dev(dl),
                        want_dh0=True, ckpt=ck)
    torch.cuda.synchronize()
    for k in g:
        a, b2 = g[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), f"{k} with saved record"


def test_bwd_time_segments_batch_invariant_and_deterministic():
    """Segmented backward: run-to-run bit equality, and each batch entry's
    du, ddelta, dz, dB, dC and dh0 the same bits run alone as inside the
    batch (the segment count depends on dim, dstate and seqlen only)."""
    require_gpu()
    w = ssin.custom("bwd", 3, 64, 16, 8192, "bf16", seed=78)
    d = dev_inputs(ssin.make(w))
    h0 = torch.randn(3, 64, 16, device=DEV)
    dl = torch.randn(3, 64, 16, device=DEV)
    g1 = run_bwd(d, w, h0=h0, dlast=dl, want_dh0=True)
    g2 = run_bwd(d, w, h0=h0, dlast=dl, want_dh0=True)
    torch.cuda.synchronize()
    for k in g1:
        a, b2 = g1[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), f"{k} not deterministic"
    per_entry = ("u", "delta", "B", "C", "z", "dout")
    for bi in range(w.batch):
        one = {k: (v[bi:bi + 1].contiguous() if k in per_entry else v) for k, v in d.items()}
        ga = run_bwd(one, w, h0=h0[bi:bi + 1].contiguous(), dlast=dl[bi:bi + 1].contiguous(),
                     want_dh0=True)
        torch.cuda.synchronize()
        for k in ("du", "ddelta", "dz", "dB", "dC", "dh0"):
            a, b1 = g1[k][bi:bi + 1], ga[k]
            if a.dtype == torch.bfloat16:
                a, b1 = a.view(torch.int16), b1.view(torch.int16)
            assert torch.equal(a, b1), f"{k} entry {bi}"


def test_bwd_long_sequence_full_size_whole_tensors():
    """One long bf16 sequence (1 x 1536 x 16384), the shape the time segments
    serve, in the launch configuration the benchmark times: every element of
    every gradient against the oracle, the same bits twice, and the
    forward's saved record giving the same bits as recomputing it."""
    require_gpu()
    w = ssin.WORKLOADS["mamba130m_long_bf16_1x1536x16384"]
    say("bwd long: generating inputs")
    arr = ssin.make(w)
    d = dev_inputs(arr)
    say("bwd long: running")
    g1 = run_bwd(d, w)
    g2 = run_bwd(d, w)
    ck = binding.ss_ckpt_empty(d["u"])
    binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                   True, ckpt=ck)
    g3 = binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                        d["delta_bias"], True, d["dout"], ckpt=ck)
    torch.cuda.synchronize()
    for k in g1:
        a, b2, b3 = g1[k], g2[k], g3[k]
        if a.dtype == torch.bfloat16:
            a, b2, b3 = a.view(torch.int16), b2.view(torch.int16), b3.view(torch.int16)
        assert torch.equal(a, b2), f"{k} not deterministic"
        assert torch.equal(a, b3), f"{k} with saved record"
    x = {k: widen(v) for k, v in arr.items()}
    say(f"bwd long: oracle on the whole workload ({ORACLE_THREADS} threads)")
    ref = oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                     x["delta_bias"], True, x["dout"], threads=ORACLE_THREADS)
    for k in ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddelta_bias"):
        tol = TOL["f32"] if k in ("dA", "dD", "ddelta_bias") else TOL[w.io]
        e = assert_close(to_host(g1[k]), ref[k], tol, k)
        say(f"  {k} err {e:.3e}")
