"""GPU parity of the Mamba-2 SSD forward (ss_ssd_fwd via the C ABI).

The chunked matrix-core kernel is compared with the double-precision
oracle's recurrence element by element: shapes with a ragged last chunk,
one or several groups, every supported head size and state size, with and
without D, dt bias, softplus and an initial state, sequences of one step
and of none, and the full Mamba-2 130M layer shape (8 x 2048, 24 heads of
64, d_state 128).  Results must be the same bits between calls and for a
batch entry alone or inside the batch, and a sequence continued from its
last state must agree with the whole.

Tolerance: the bf16 bound (2e-2 on the shared error metric) for the bf16
output; the f32 bound for the final state, an f32 output whose products take
their on-chip operands as bf16 high and low parts (measured 1e-5 at full
size).
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import dev_inputs, require_gpu, say, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu


def _run(d, softplus=True, h0=None):
    return binding.ss_ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"),
                              d.get("dt_bias"), softplus, h0=h0, return_last_state=True)


def _oracle(arr, softplus=True, h0=None, threads=8):
    w = {k: widen(v) for k, v in arr.items()}
    return oracle.ssd_fwd(w["x"], w["dt"], w["A"], w["B"], w["C"], w.get("D"), w.get("dt_bias"),
                          softplus, h0, threads=threads)


SMALL = [
    # batch, seqlen, nheads, headdim, ngroups, dstate, flags
    (2, 130, 4, 64, 1, 128, dict(has_h0=True)),   # ragged last chunk, initial state
    (1, 64, 3, 32, 3, 64, {}),                    # one group per head, one full chunk
    (2, 200, 6, 16, 2, 32, dict(has_D=False)),    # two groups
    (1, 1, 2, 48, 1, 96, dict(has_h0=True)),      # a single step
    (3, 97, 2, 64, 2, 64, dict(has_bias=False)),
    (1, 300, 8, 32, 4, 128, dict(has_h0=True)),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:6])))
@pytest.mark.parametrize("softplus", [True, False])
def test_ssd_small_parity(shape, softplus):
    require_gpu()
    b, L, H, P, G, N, flags = shape
    w = ssin.ssd_custom(b, L, H, P, G, N, seed=L + N + H, **flags)
    say(f"ssd {w.name} softplus={softplus}")
    arr = ssin.make_ssd(w)
    if not softplus:
        # without softplus the step is dt_raw + bias itself, which must not
        # be negative (exp(dt A) > 1 would grow the state without bound):
        # take |dt_raw| / 10 and no bias
        arr["dt"] = ssin.bf16_bits(0.1 * np.abs(ssin.widen(arr["dt"])))
        arr.pop("dt_bias", None)
    d = dev_inputs(arr)
    y, last = _run(d, softplus, h0=d.get("h0"))
    torch.cuda.synchronize()
    ry, rl = _oracle(arr, softplus, h0=arr.get("h0"))
    assert_close(to_host(y), ry, TOL["bf16"], "y")
    # last_state is an f32 output: the state and its sums stay f32 on chip
    assert_close(to_host(last), rl, TOL["f32"], "last_state")


def test_ssd_empty_sequence():
    require_gpu()
    w = ssin.ssd_custom(2, 0, 4, 64, 1, 128, seed=2, has_h0=True)
    d = dev_inputs(ssin.make_ssd(w))
    y, last = _run(d, h0=d["h0"])
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(last, d["h0"])


def test_ssd_full_size():
    require_gpu()
    w = ssin.SSD_WORKLOADS["mamba2_130m_ssd_bf16_8x2048x24x64_n128"]
    say(f"ssd full size {w.name}")
    arr = ssin.make_ssd(w)
    d = dev_inputs(arr)
    y, last = _run(d)
    y2, last2 = _run(d)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "y differs between calls"
    assert torch.equal(last, last2), "last_state differs between calls"
    ry, rl = _oracle(arr)
    e1 = assert_close(to_host(y), ry, TOL["bf16"], "y")
    e2 = assert_close(to_host(last), rl, TOL["f32"], "last_state")
    say(f"  err y {e1:.3e} last_state {e2:.3e}")


def test_ssd_rows_do_not_depend_on_batch():
    require_gpu()
    w = ssin.ssd_custom(4, 150, 6, 64, 2, 128, seed=9, has_h0=True)
    arr = ssin.make_ssd(w)
    d = dev_inputs(arr)
    y, last = _run(d, h0=d["h0"])
    for bi in (0, 3):
        one = {k: (v[bi:bi + 1].contiguous() if k in ("x", "dt", "B", "C", "h0") else v)
               for k, v in d.items()}
        y1, l1 = _run(one, h0=one["h0"])
        torch.cuda.synchronize()
        assert torch.equal(y1[0].view(torch.int16), y[bi].view(torch.int16)), f"y entry {bi}"
        assert torch.equal(l1[0], last[bi]), f"last_state entry {bi}"


@pytest.mark.parametrize("split", [64, 100])
def test_ssd_continues_from_last_state(split):
    require_gpu()
    w = ssin.ssd_custom(2, 256, 4, 64, 1, 128, seed=split)
    arr = ssin.make_ssd(w)
    d = dev_inputs(arr)
    y, last = _run(d)
    first = {k: (v[:, :split].contiguous() if k in ("x", "dt", "B", "C") else v)
             for k, v in d.items()}
    rest = {k: (v[:, split:].contiguous() if k in ("x", "dt", "B", "C") else v)
            for k, v in d.items()}
    y1, l1 = _run(first)
    y2, l2 = _run(rest, h0=l1)
    torch.cuda.synchronize()
    assert_close(to_host(torch.cat([y1, y2], dim=1)), to_host(y), TOL["bf16"], "y continued")
    assert_close(to_host(l2), to_host(last), TOL["bf16"], "last_state continued")
