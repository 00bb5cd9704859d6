"""GPU parity of the one-token state update (ss_state_update via the C ABI).

The decode workload runs at its full size against the oracle element by
element; every batch entry stepped alone must give the same bits as inside
the batch; the call must be deterministic; and a scan over L steps followed
by one state update must agree with a scan over L + 1 steps.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import DEV, dev_inputs, require_gpu, say, to_dev, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu


def step(d, w, state):
    return binding.ss_state_update(state, d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"),
                                   d.get("z"), d.get("delta_bias"), w.softplus)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_full_size_and_batch_invariance(io):
    require_gpu()
    base = ssin.WORKLOADS["decode_bf16_256x5120"]
    w = base if io == "bf16" else ssin.custom("decode", 256, 5120, 16, 1, "f32", seed=base.seed)
    say(f"decode {w.name}")
    arr = ssin.make(w)
    d = dev_inputs(arr)
    st = to_dev(arr["state"])
    st2 = st.clone()
    y = step(d, w, st)
    y2 = step(d, w, st2)
    torch.cuda.synchronize()
    assert torch.equal(st, st2) and torch.equal(y.view(torch.int16) if io == "bf16" else y,
                                                y2.view(torch.int16) if io == "bf16" else y2)
    x = {k: widen(v) for k, v in arr.items()}
    rs, ry = oracle.state_update(x["state"], x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                 x["z"], x["delta_bias"], True, threads=8)
    e1 = assert_close(to_host(y), ry, TOL[io], "y")
    e2 = assert_close(to_host(st), rs, TOL["f32"], "state")
    say(f"  err y {e1:.3e} state {e2:.3e}")
    for b in range(w.batch):
        one = {k: (v[b:b + 1] if k in ("u", "delta", "z", "B", "C") else v) for k, v in d.items()}
        s1 = to_dev(arr["state"][b:b + 1])
        y1 = step(one, w, s1)
        torch.cuda.synchronize()
        assert torch.equal(s1[0], st[b]), f"state row {b}"
        if io == "bf16":
            assert torch.equal(y1[0].view(torch.int16), y[b].view(torch.int16)), f"y row {b}"
        else:
            assert torch.equal(y1[0], y[b]), f"y row {b}"


@pytest.mark.parametrize("N,io", [(1, "f32"), (6, "bf16"), (13, "f32"), (17, "f32"),
                                  (64, "bf16"), (100, "f32"), (256, "bf16")])
def test_decode_smaller_dstate(N, io):
    """d_state below 16 (element loads, unused state lanes held at zero)."""
    require_gpu()
    w = ssin.custom("decode", 8, 40, N, 1, io, seed=N)
    arr = ssin.make(w)
    d = dev_inputs(arr)
    st = to_dev(arr["state"])
    y = step(d, w, st)
    torch.cuda.synchronize()
    x = {k: widen(v) for k, v in arr.items()}
    rs, ry = oracle.state_update(x["state"], x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"],
                                 x["z"], x["delta_bias"], True, threads=8)
    assert_close(to_host(y), ry, TOL[io], f"y N={N}")
    assert_close(to_host(st), rs, TOL["f32"], f"state N={N}")


def test_decode_ragged_rows_and_flags():
    require_gpu()
    for flags in ({}, dict(has_z=False, has_D=False, has_bias=False)):
        w = ssin.custom("decode", 3, 37, 16, 1, "f32", seed=21, **flags)
        arr = ssin.make(w)
        d = dev_inputs(arr)
        st = to_dev(arr["state"])
        y = step(d, w, st)
        torch.cuda.synchronize()
        x = {k: widen(v) for k, v in arr.items()}
        rs, ry = oracle.state_update(x["state"], x["u"], x["delta"], x["A"], x["B"], x["C"],
                                     x.get("D"), x.get("z"), x.get("delta_bias"), True)
        assert_close(to_host(y), ry, TOL["f32"], "y")
        assert_close(to_host(st), rs, TOL["f32"], "state")


def test_scan_then_step_equals_longer_scan():
    require_gpu()
    w = ssin.custom("fwd", 2, 48, 16, 65, "f32", seed=33)
    arr = ssin.make(w)
    d = dev_inputs(arr)
    L = 64
    first = {k: (v[..., :L].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
             for k, v in d.items()}
    y_full = binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                            d["delta_bias"], True)
    _, last = binding.ss_fwd(first["u"], first["delta"], d["A"], first["B"], first["C"], d["D"],
                             first["z"], d["delta_bias"], True, return_last_state=True)
    tok = {k: (v[..., L].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
           for k, v in d.items()}
    y_step = binding.ss_state_update(last, tok["u"], tok["delta"], d["A"], tok["B"], tok["C"],
                                     d["D"], tok["z"], d["delta_bias"], True)
    torch.cuda.synchronize()
    assert_close(to_host(y_step), to_host(y_full[..., L]), 1e-5, "step after scan")
