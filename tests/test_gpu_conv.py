"""GPU parity of the causal depthwise convolution (ss_conv1d_* via the C ABI).

Forward, backward and the decode step are compared with the double-precision
oracle element by element: at sizes that span several segments and end in
a ragged one, on both the 16-byte vector path and the per-element path
(lengths that are not a multiple of the vector), for every width 1..4, with
and without bias, initial window and SiLU, and at the full Mamba-130M shape
(8 x 1536 x 2048, width 4).  Results must be bit-identical between calls
and whatever the batch size, a sequence cut in two and continued from the
final window must give the same bits as the whole, and a decode step must
continue a forward pass.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import dev_inputs, require_gpu, say, to_dev, to_host, widen
from metrics import TOL, assert_close

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run(w, d, silu=True, want_dinit=False):
    out, fin = binding.ss_conv1d_fwd(d["x"], d["weight"], d.get("bias"), silu, d.get("init"),
                                     return_final_state=True)
    g = binding.ss_conv1d_bwd(d["x"], d["weight"], d.get("bias"), silu, d.get("init"), d["dout"],
                              want_dinit_state=want_dinit)
    torch.cuda.synchronize()
    return out, fin, g


def _oracle(arr, silu=True, threads=8):
    x = {k: widen(v) for k, v in arr.items()}
    ro, rf = oracle.conv_fwd(x["x"], x["weight"], x.get("bias"), silu, x.get("init"),
                             threads=threads)
    rg = oracle.conv_bwd(x["x"], x["weight"], x.get("bias"), silu, x.get("init"), x["dout"],
                         threads=threads)
    return ro, rf, rg


def _compare(w, arr, out, fin, g, silu=True, tag=""):
    ro, rf, rg = _oracle(arr, silu)
    tol = TOL[w.io]
    errs = {"out": assert_close(to_host(out), ro, tol, f"{tag} out"),
            "dx": assert_close(to_host(g["dx"]), rg["dx"], tol, f"{tag} dx"),
            "dweight": assert_close(to_host(g["dweight"]), rg["dweight"], TOL["f32"],
                                    f"{tag} dweight")}
    # the final window is a copy of inputs: exact
    np.testing.assert_array_equal(to_host(fin), rf, err_msg=f"{tag} final_state")
    if "bias" in arr:
        errs["dbias"] = assert_close(to_host(g["dbias"]), rg["dbias"], TOL["f32"], f"{tag} dbias")
    if "dinit_state" in g:
        ref = rg.get("dinit_state")
        if ref is None:  # gradient at a zero window: the oracle with explicit zeros
            x = {k: widen(v) for k, v in arr.items()}
            ref = oracle.conv_bwd(x["x"], x["weight"], x.get("bias"), silu,
                                  np.zeros(g["dinit_state"].shape), x["dout"])["dinit_state"]
        errs["dinit"] = assert_close(to_host(g["dinit_state"]), ref, TOL["f32"], f"{tag} dinit")
    return errs


SMALL = [
    # batch, dim, seqlen, width, io, flags
    (2, 37, 4160, 4, "f32", dict(has_init=True)),   # vector path, 3 segments, ragged tail
    (3, 21, 1000, 4, "bf16", {}),                   # vector path, one partial segment
    (2, 19, 4104, 4, "bf16", dict(has_init=True)),  # vector path, bf16, 3 segments
    (2, 17, 2051, 3, "f32", {}),                    # element path, 2 segments
    (2, 9, 37, 2, "bf16", dict(has_init=True)),     # element path, bf16
    (1, 5, 8, 1, "f32", dict(has_bias=False)),      # width 1
    (2, 6, 2, 4, "f32", dict(has_init=True)),       # seqlen < width - 1
    (1, 3, 4, 4, "f32", dict(has_init=True)),       # one vector
    (2, 4, 2048, 4, "f32", dict(has_bias=False)),   # exactly one segment
    (2, 4, 2052, 4, "bf16", dict(has_init=True)),   # element path (2052 % 8 != 0)
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}k{s[3]}{s[4]}")
@pytest.mark.parametrize("silu", [True, False])
def test_conv_small_parity(shape, silu):
    require_gpu()
    b, dm, L, K, io, flags = shape
    w = ssin.conv_custom(b, dm, L, K, io, seed=L + K, **flags)
    say(f"conv {w.name} silu={silu}")
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    out, fin, g = _run(w, d, silu, want_dinit=True)
    _compare(w, arr, out, fin, g, silu, w.name)


def test_conv_empty_sequence():
    require_gpu()
    w = ssin.conv_custom(2, 5, 0, 4, "f32", seed=3, has_init=True)
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    out, fin, g = _run(w, d, True)
    assert out.numel() == 0
    assert torch.equal(fin, d["init"])
    assert not g["dweight"].any() and not g["dbias"].any() and not g["dinit_state"].any()


@pytest.mark.parametrize("name", ["mamba130m_conv_f32_8x1536x2048",
                                  "mamba130m_conv_bf16_8x1536x2048"])
def test_conv_full_size(name):
    require_gpu()
    w = ssin.CONV_WORKLOADS[name]
    say(f"conv full size {name}")
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    out, fin, g = _run(w, d, True)
    out2, fin2, g2 = _run(w, d, True)
    for a, b_, n in ((out, out2, "out"), (g["dx"], g2["dx"], "dx"),
                     (g["dweight"], g2["dweight"], "dweight"), (g["dbias"], g2["dbias"], "dbias")):
        assert torch.equal(_bits(a), _bits(b_)), f"{n} differs between calls"
    errs = _compare(w, arr, out, fin, g, True, name)
    say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_conv_rows_do_not_depend_on_batch():
    require_gpu()
    w = ssin.conv_custom(6, 24, 3000, 4, "bf16", seed=77, has_init=True)
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    out, fin, g = _run(w, d, True)
    for b in (0, 5):
        one = {k: (v[b:b + 1] if k in ("x", "dout", "init") else v) for k, v in d.items()}
        o1, f1, g1 = _run(w, one, True)
        assert torch.equal(_bits(o1[0]), _bits(out[b])), f"out row {b}"
        assert torch.equal(_bits(g1["dx"][0]), _bits(g["dx"][b])), f"dx row {b}"
        assert torch.equal(g1["dinit_state"][0], g["dinit_state"][b]), f"dinit row {b}"
        assert torch.equal(f1[0], fin[b])


@pytest.mark.parametrize("io,split", [("f32", 2048), ("f32", 1001), ("bf16", 4096)])
def test_conv_continues_from_final_window(io, split):
    require_gpu()
    w = ssin.conv_custom(2, 16, 6144, 4, io, seed=split, has_init=True)
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    whole, fin = binding.ss_conv1d_fwd(d["x"], d["weight"], d["bias"], True, d["init"],
                                       return_final_state=True)
    a, s1 = binding.ss_conv1d_fwd(d["x"][:, :, :split].contiguous(), d["weight"], d["bias"], True,
                                  d["init"], return_final_state=True)
    b, s2 = binding.ss_conv1d_fwd(d["x"][:, :, split:].contiguous(), d["weight"], d["bias"], True,
                                  s1, return_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch.cat([a, b], dim=2)), _bits(whole))
    assert torch.equal(s2, fin)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_conv_decode_full_size(io):
    require_gpu()
    base = ssin.CONV_WORKLOADS["conv_decode_bf16_256x5120"]
    w = base if io == "bf16" else ssin.ConvWorkload("conv_decode_f32_256x5120", 256, 5120, 1, 4,
                                                    "f32", decode=True, seed=base.seed)
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    st = to_dev(arr["state"])
    y = binding.ss_conv1d_update(st, d["x"], d["weight"], d["bias"], True)
    torch.cuda.synchronize()
    x = {k: widen(v) for k, v in arr.items()}
    rs, ry = oracle.conv_update(x["state"], x["x"], x["weight"], x["bias"], True)
    assert_close(to_host(y), ry, TOL[io], "decode out")
    np.testing.assert_array_equal(to_host(st), rs)


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_decode_continues_forward(K):
    require_gpu()
    w = ssin.conv_custom(3, 40, 129, K, "f32", seed=K, has_init=True)
    arr = ssin.make_conv(w)
    d = dev_inputs(arr)
    L = 128
    full, fin_full = binding.ss_conv1d_fwd(d["x"], d["weight"], d["bias"], True, d["init"],
                                           return_final_state=True)
    _, st = binding.ss_conv1d_fwd(d["x"][:, :, :L].contiguous(), d["weight"], d["bias"], True,
                                  d["init"], return_final_state=True)
    y = binding.ss_conv1d_update(st, d["x"][:, :, L].contiguous(), d["weight"], d["bias"], True)
    torch.cuda.synchronize()
    assert_close(to_host(y), to_host(full[:, :, L]), TOL["f32"], "decode vs forward")
    assert torch.equal(st, fin_full)
