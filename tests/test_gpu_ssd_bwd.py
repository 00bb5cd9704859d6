"""GPU parity of the Mamba-2 SSD backward (ss_ssd_bwd via the C ABI).

Every gradient is compared with the double-precision oracle's
back-propagation through time, element by element: one group (a single
selective-scan backward over the batch) and several groups (one call per
batch entry and group), every supported head and state size, with and
without D, dt bias, softplus, an initial state and a gradient on the final
state, L = 1 and L = 0, and the full Mamba-2 130M layer shape.  Results must
be the same bits between calls, and the per-batch-entry gradients the same
bits alone and inside a batch.

Tolerances: the bf16 bound (2e-2) for the bf16 outputs dx, ddt, dB, dC; the
f32 bound (1e-4) for dA, dD, ddt_bias and dh0, which stay in f32.
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

BF16_KEYS = ("dx", "ddt", "dB", "dC")
F32_KEYS = ("dA", "dD", "ddt_bias", "dh0")


def _run(d, softplus=True, use_dlast=True):
    return binding.ss_ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"),
                              d.get("dt_bias"), softplus, h0=d.get("h0"), dout=d["dout"],
                              dlast=d["dlast"] if use_dlast else None, want_dh0=True)


def _oracle(arr, softplus=True, use_dlast=True, threads=8):
    w = {k: widen(v) for k, v in arr.items()}
    return oracle.ssd_bwd(w["x"], w["dt"], w["A"], w["B"], w["C"], w.get("D"), w.get("dt_bias"),
                          softplus, w.get("h0"), w["dout"], w["dlast"] if use_dlast else None,
                          threads=threads)


def _compare(g, ref, tag):
    errs = {}
    for k in BF16_KEYS + F32_KEYS:
        if k in ref and k in g:
            tol = TOL["bf16"] if k in BF16_KEYS else TOL["f32"]
            errs[k] = assert_close(to_host(g[k]), ref[k], tol, f"{tag} {k}")
    return errs


SMALL = [
    # batch, seqlen, nheads, headdim, ngroups, dstate, flags
    (2, 130, 4, 64, 1, 128, dict(has_h0=True)),
    (1, 64, 3, 32, 3, 64, {}),                     # one group per head: per-(entry, group) calls
    (2, 200, 6, 16, 2, 32, dict(has_D=False)),
    (1, 1, 2, 48, 1, 96, dict(has_h0=True)),
    (3, 97, 2, 64, 2, 64, dict(has_bias=False)),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:6])))
@pytest.mark.parametrize("softplus", [True, False])
def test_ssd_bwd_small_parity(shape, softplus):
    require_gpu()
    b, L, H, P, G, N, flags = shape
    w = ssin.ssd_custom(b, L, H, P, G, N, seed=L + N + H + 7, bwd=True, **flags)
    say(f"ssd bwd {w.name} softplus={softplus}")
    arr = ssin.make_ssd(w)
    if not softplus:
        # without softplus dt must not be negative (see the forward's tests)
        arr["dt"] = ssin.bf16_bits(0.1 * np.abs(ssin.widen(arr["dt"])))
        arr.pop("dt_bias", None)
    d = dev_inputs(arr)
    g = _run(d, softplus)
    torch.cuda.synchronize()
    _compare(g, _oracle(arr, softplus), w.name)


def test_ssd_bwd_empty_sequence_passes_dlast_through():
    require_gpu()
    w = ssin.ssd_custom(2, 0, 4, 64, 1, 128, seed=3, has_h0=True, bwd=True)
    d = dev_inputs(ssin.make_ssd(w))
    g = _run(d)
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], d["dlast"])
    assert not g["dA"].any() and not g["dD"].any() and not g["ddt_bias"].any()


def test_ssd_bwd_empty_batch_zeroes_parameter_gradients():
    require_gpu()
    w = ssin.ssd_custom(1, 64, 4, 64, 1, 128, seed=5, bwd=True)
    d = {k: (v[:0].contiguous() if k in ("x", "dt", "B", "C", "dout", "dlast", "h0") else v)
         for k, v in dev_inputs(ssin.make_ssd(w)).items()}
    g = _run(d)
    torch.cuda.synchronize()
    assert g["dx"].numel() == 0 and g["dB"].numel() == 0
    for k in ("dA", "dD", "ddt_bias"):
        assert g[k].shape == (4,) and not g[k].any(), k


@pytest.mark.parametrize("shape", [(2, 130, 4, 64, 1, 128), (3, 97, 6, 48, 2, 96),
                                   (1, 64, 2, 16, 1, 32)])
def test_ssd_bwd_from_forward_checkpoint(shape):
    # the forward's saved chunk states are the states pass's: same bits
    require_gpu()
    b, L, H, P, G, N = shape
    w = ssin.ssd_custom(b, L, H, P, G, N, seed=L + P, has_h0=True, bwd=True)
    d = dev_inputs(ssin.make_ssd(w))
    say(f"ssd bwd from checkpoint {w.name}")
    ck = binding.ss_ssd_ckpt_empty(d["x"], N)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dt_bias"], True)
    y0, l0 = binding.ss_ssd_fwd(*args, h0=d["h0"], return_last_state=True)
    y1, l1 = binding.ss_ssd_fwd(*args, h0=d["h0"], return_last_state=True, ckpt=ck)
    g0 = _run(d)
    g1 = binding.ss_ssd_bwd(*args, h0=d["h0"], dout=d["dout"], dlast=d["dlast"], want_dh0=True,
                            ckpt=ck)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)) and torch.equal(l0, l1)
    for k in g0:
        a, c = g0[k], g1[k]
        if a.dtype == torch.bfloat16:
            a, c = a.view(torch.int16), c.view(torch.int16)
        assert torch.equal(a, c), k


def test_ssd_bwd_full_size():
    require_gpu()
    w = ssin.SSD_WORKLOADS["mamba2_130m_ssd_bwd_bf16_8x2048x24x64_n128"]
    say(f"ssd bwd full size {w.name}")
    arr = ssin.make_ssd(w)
    d = dev_inputs(arr)
    g = _run(d)
    g2 = _run(d)
    torch.cuda.synchronize()
    for k in g:
        a, b2 = g[k], g2[k]
        if a.dtype == torch.bfloat16:
            a, b2 = a.view(torch.int16), b2.view(torch.int16)
        assert torch.equal(a, b2), f"{k} differs between calls"
    errs = _compare(g, _oracle(arr), w.name)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_ssd_bwd_rows_do_not_depend_on_batch():
    require_gpu()
    w = ssin.ssd_custom(4, 150, 4, 64, 1, 64, seed=11, has_h0=True, bwd=True)
    arr = ssin.make_ssd(w)
    d = dev_inputs(arr)
    g = _run(d)
    per_entry = ("x", "dt", "B", "C", "h0", "dout", "dlast")
    for bi in (0, 3):
        one = {k: (v[bi:bi + 1].contiguous() if k in per_entry else v) for k, v in d.items()}
        g1 = _run(one)
        torch.cuda.synchronize()
        for k in ("dx", "ddt", "dB", "dC", "dh0"):
            a, b1 = g[k][bi:bi + 1], g1[k]
            if a.dtype == torch.bfloat16:
                a, b1 = a.view(torch.int16), b1.view(torch.int16)
            assert torch.equal(a, b1), f"{k} entry {bi}"
