"""GPU parity of the forward scan (ss_fwd through the C ABI) with the oracle.

Small shapes are compared element by element; they span several 32-step
chunks, ragged time tails (including lengths whose rows are not 16-byte
aligned), ragged channel counts, every optional input switched on and off,
an initial state, and the empty and single-step cases.  The named workloads
run at their full size in the launch configuration the benchmark times and
are checked on every element.  Determinism (same bits twice) and batch
invariance (a row alone == the same row inside the batch, bit for bit) are
checked exactly.
"""
import numpy as np
import pytest
import torch

from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import ORACLE_THREADS, DEV, dev_inputs, oracle_fwd, require_gpu, say, to_dev, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu


def run_fwd(d, w, h0=None, last=False):
    return binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"), d.get("z"),
                          d.get("delta_bias"), w.softplus, h0=h0, return_last_state=last)


SMALL = [
    # batch, dim, L, io, flags
    (2, 40, 100, "f32", {}),                      # ragged dim, ragged tail, aligned rows
    (1, 17, 33, "f32", {}),                       # rows not 16-byte aligned (scalar path)
    (3, 16, 64, "bf16", {}),
    (2, 48, 75, "bf16", {}),                      # bf16 rows not 16-byte aligned
    (1, 32, 96, "f32", dict(has_z=False)),
    (1, 32, 96, "f32", dict(has_D=False)),
    (1, 32, 96, "f32", dict(has_bias=False)),
    (1, 32, 96, "f32", dict(softplus=False)),
    (1, 32, 96, "bf16", dict(has_z=False, has_D=False, has_bias=False)),
    (2, 16, 1, "f32", {}),                        # single step
    (1, 8, 31, "f32", {}),                        # fewer rows than a workgroup, one chunk
    # many workgroups: a last group of 8 channels and a ragged tail; no z
    (8, 1544, 100, "f32", {}),
    (8, 1536, 128, "bf16", dict(has_z=False)),
]


@pytest.mark.parametrize("batch,dim,L,io,flags", SMALL)
def test_fwd_small_elementwise(batch, dim, L, io, flags):
    require_gpu()
    w = ssin.custom("fwd", batch, dim, 16, L, io, seed=batch * 1000 + dim + L, **flags)
    if not w.softplus:
        # without softplus keep delta positive so the recurrence decays
        arr = ssin.make(w)
        arr["delta"] = (np.abs(ssin.widen(arr["delta"])) + 0.05).astype(np.float32)
        if io == "bf16":
            arr["delta"] = ssin.bf16_bits(arr["delta"])
        if "delta_bias" in arr:
            arr["delta_bias"] = np.linspace(0.0, 0.1, dim).astype(np.float32)
    else:
        arr = ssin.make(w)
    say(f"fwd small {w.name}")
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal((batch, dim, 16)).astype(np.float32)
    d = dev_inputs(arr)
    for use_h0 in (False, True):
        y, last = run_fwd(d, w, h0=to_dev(h0) if use_h0 else None, last=True)
        torch.cuda.synchronize()
        ry, rl = oracle_fwd(arr, w.softplus, h0=h0.astype(np.float64) if use_h0 else None)
        assert_close(to_host(y), ry, TOL[io], f"y h0={use_h0}")
        assert_close(to_host(last), rl, TOL["f32"], f"last_state h0={use_h0}")


@pytest.mark.parametrize("N,io,L", [(1, "f32", 70), (4, "bf16", 64), (7, "f32", 100),
                                    (12, "bf16", 40), (17, "f32", 70), (32, "bf16", 64),
                                    (64, "f32", 100), (100, "bf16", 40), (256, "f32", 48)])
def test_fwd_smaller_dstate(N, io, L):
    """d_state other than 16: the kernels keep 16 state lanes and the unused
    ones must add nothing (scalar and 16-byte load paths); above 16 the
    states run in 16-state slices whose sums a combine kernel adds."""
    require_gpu()
    w = ssin.custom("fwd", 2, 40, N, L, io, seed=31 * N + L)
    arr = ssin.make(w)
    say(f"fwd dstate {w.name}")
    d = dev_inputs(arr)
    h0 = np.random.default_rng(N).standard_normal((2, 40, N)).astype(np.float32)
    for use_h0 in (False, True):
        y, last = run_fwd(d, w, h0=to_dev(h0) if use_h0 else None, last=True)
        torch.cuda.synchronize()
        ry, rl = oracle_fwd(arr, w.softplus, h0=h0.astype(np.float64) if use_h0 else None)
        assert_close(to_host(y), ry, TOL[io], f"y N={N} h0={use_h0}")
        assert_close(to_host(last), rl, TOL["f32"], f"last_state N={N} h0={use_h0}")


def test_fwd_empty_and_zero_length():
    require_gpu()
    w = ssin.custom("fwd", 2, 32, 16, 0, "f32", seed=3)
    arr = ssin.make(w)
    d = dev_inputs(arr)
    h0 = torch.randn(2, 32, 16, device=DEV)
    y, last = run_fwd(d, w, h0=h0, last=True)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(last, h0)          # no steps: the state is the initial state
    y, last = run_fwd(d, w, last=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(last).item() == 0
    w0 = ssin.custom("fwd", 0, 32, 16, 64, "f32", seed=3)
    d0 = dev_inputs(ssin.make(w0))
    y = run_fwd(d0, w0)
    torch.cuda.synchronize()
    assert y.shape == (0, 32, 64)


def test_fwd_tiny_named_workload_elementwise():
    require_gpu()
    w = ssin.WORKLOADS["tiny_fwd_f32_1x64x256"]
    arr = ssin.make(w)
    say(f"fwd {w.name}")
    y = run_fwd(dev_inputs(arr), w)
    torch.cuda.synchronize()
    ry, _ = oracle_fwd(arr, w.softplus)
    e = assert_close(to_host(y), ry, TOL[w.io], w.name)
    say(f"  max err {e:.3e}")


@pytest.mark.parametrize("name", ["mamba130m_fwd_bf16_8x1536x2048",
                                  "mamba2p8b_fwd_bf16_4x5120x4096",
                                  # one long sequence: the time-segmented scan
                                  "mamba130m_long_bf16_1x1536x16384"])
def test_fwd_full_size_whole_tensors_deterministic(name):
    """A named forward workload at full size, in the launch configuration the
    benchmark times: every element of y and of last_state against the
    oracle, the same bits twice, and every batch entry alone equal to the
    same entry inside the batch."""
    require_gpu()
    w = ssin.WORKLOADS[name]
    say(f"fwd full {name}: generating inputs")
    arr = ssin.make(w)
    d = dev_inputs(arr)
    say(f"fwd full {name}: running twice")
    y1, l1 = run_fwd(d, w, last=True)
    y2, l2 = run_fwd(d, w, last=True)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "forward not deterministic"
    assert torch.equal(l1, l2)
    say(f"fwd full {name}: oracle on the whole workload ({ORACLE_THREADS} threads)")
    ry, rl = oracle_fwd(arr, w.softplus, threads=ORACLE_THREADS)
    e = assert_close(to_host(y1), ry, TOL[w.io], f"{name} y")
    el = assert_close(to_host(l1), rl, TOL["f32"], f"{name} last_state")
    say(f"  max err y {e:.3e}, last_state {el:.3e}")
    del ry, rl
    # batch invariance: every batch entry alone gives the same bits as inside the batch
    for b in range(w.batch):
        one = {k: (v[b:b + 1] if k in ("u", "delta", "z", "B", "C") else v) for k, v in d.items()}
        ya, la = run_fwd(one, w, last=True)
        torch.cuda.synchronize()
        assert torch.equal(ya[0].view(torch.int16), y1[b].view(torch.int16)), f"batch row {b}"
        assert torch.equal(la[0], l1[b])


def test_fwd_wide_state_rows_do_not_depend_on_batch():
    """With several state slices a row's output is still the same bits alone
    and inside a batch."""
    require_gpu()
    w = ssin.custom("fwd", 4, 48, 64, 160, "bf16", seed=5)
    arr = ssin.make(w)
    d = dev_inputs(arr)
    y, last = run_fwd(d, w, last=True)
    for bi in (0, 3):
        one = {k: (v[bi:bi + 1].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
               for k, v in d.items()}
        y1, l1 = run_fwd(one, w, last=True)
        torch.cuda.synchronize()
        assert torch.equal(y1[0].view(torch.int16), y[bi].view(torch.int16)), f"y entry {bi}"
        assert torch.equal(l1[0], last[bi]), f"last_state entry {bi}"


# Long sequences over few channels take the time-segmented scan (chosen from
# dim, dstate and seqlen only): a summary pass per segment, then every segment
# from the state its predecessors' (decay, end state) pairs give.  Seqlen
# 8192 and up with fewer than 3072 wavefronts per batch entry; 64 channels
# give 8 segments of 1024+ steps.
SEGMENTED = [
    # batch, dim, dstate, L, io
    (2, 64, 16, 8192, "f32"),        # 8 segments of 1024 steps
    (2, 48, 16, 8229, "bf16"),       # ragged: segments of 1088 steps, a short ragged last one
    (1, 40, 16, 9001, "f32"),        # rows not 16-byte aligned (scalar path), ragged channels
    (2, 32, 40, 8300, "bf16"),       # three 16-state slices x 8 segments
]


@pytest.mark.parametrize("batch,dim,N,L,io", SEGMENTED)
def test_fwd_time_segments_elementwise(batch, dim, N, L, io):
    require_gpu()
    w = ssin.custom("fwd", batch, dim, N, L, io, seed=batch + dim + N + L)
    arr = ssin.make(w)
    say(f"fwd segmented {w.name}")
    d = dev_inputs(arr)
    h0 = np.random.default_rng(L).standard_normal((batch, dim, N)).astype(np.float32)
    for use_h0 in (False, True):
        y, last = run_fwd(d, w, h0=to_dev(h0) if use_h0 else None, last=True)
        torch.cuda.synchronize()
        ry, rl = oracle_fwd(arr, w.softplus, h0=h0.astype(np.float64) if use_h0 else None)
        e = assert_close(to_host(y), ry, TOL[io], f"y h0={use_h0}")
        assert_close(to_host(last), rl, TOL["f32"], f"last_state h0={use_h0}")
        say(f"  h0={use_h0} max err {e:.3e}")


def test_fwd_time_segments_batch_invariant_and_deterministic():
    require_gpu()
    w = ssin.custom("fwd", 3, 64, 16, 8192, "bf16", seed=77)
    d = dev_inputs(ssin.make(w))
    y1, l1 = run_fwd(d, w, last=True)
    y2, l2 = run_fwd(d, w, last=True)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(l1, l2)
    for b in range(w.batch):
        one = {k: (v[b:b + 1].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
               for k, v in d.items()}
        ya, la = run_fwd(one, w, last=True)
        torch.cuda.synchronize()
        assert torch.equal(ya[0].view(torch.int16), y1[b].view(torch.int16)), f"entry {b}"
        assert torch.equal(la[0], l1[b]), f"last_state entry {b}"
