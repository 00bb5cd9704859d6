"""Pins of the oracle's causal depthwise convolution against things other than itself.

The reading pinned here: a per-channel causal convolution of width K over
time, out_t = act(bias + sum_k w[k] x_{t-(K-1)+k}), with the K-1 inputs
before t = 0 taken from an initial window (zeros when none is given), the
last K-1 inputs kept as the final window, and SiLU as the optional
activation; the Mamba block of the state-spaces/mamba README ("Usage")
sets this width with d_conv = 4.  Expected values come from library
routines that compute the same convolution by other means (numpy's full
convolution with the taps reversed, torch's grouped conv1d with left
padding, torch autograd), from impulse responses, from brute-force central
differences, and from structural facts (continuation from the final
window, the decode step reproducing the sequence).  A wrong tap order, a
dropped bias, a window read at the wrong offset, or a wrong SiLU derivative
fails at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _silu(p):
    return p / (1.0 + np.exp(-p))


def _case(seed, nb=2, nd=3, nl=11, nk=4):
    r = _rng(seed)
    return (r.standard_normal((nb, nd, nl)), r.standard_normal((nd, nk)) * 0.5,
            r.standard_normal(nd) * 0.3)


@pytest.mark.parametrize("nk", [2, 3, 4])
def test_impulse_response_is_reversed_taps(nk):
    # A unit input at t0 reaches out_{t0+j} through tap K-1-j and nothing else.
    nl, t0 = 12, 5
    w = np.arange(1.0, nk + 1.0)[None, :] * np.array([[1.0], [-0.5]])
    x = np.zeros((1, 2, nl))
    x[:, :, t0] = 1.0
    out, _ = oracle.conv_fwd(x, w, None, silu=False)
    for d in range(2):
        expect = np.zeros(nl)
        expect[t0:t0 + nk] = w[d, ::-1]
        np.testing.assert_array_equal(out[0, d], expect)


@pytest.mark.parametrize("nk", [1, 2, 4])
def test_matches_numpy_full_convolution(nk):
    x, w, b = _case(1, nk=nk)
    out, _ = oracle.conv_fwd(x, w, b, silu=False)
    for bi in range(x.shape[0]):
        for d in range(x.shape[1]):
            ref = np.convolve(x[bi, d], w[d, ::-1])[: x.shape[2]] + b[d]
            np.testing.assert_allclose(out[bi, d], ref, rtol=1e-14, atol=1e-14)


def test_silu_applied_to_torch_grouped_conv1d():
    # torch's conv1d is a cross-correlation; padding K-1 on both ends and
    # keeping the first L outputs makes it causal with taps in input order.
    x, w, b = _case(2, nb=3, nd=5, nl=17)
    nk = w.shape[1]
    pre = torch.nn.functional.conv1d(torch.from_numpy(x), torch.from_numpy(w)[:, None, :],
                                     torch.from_numpy(b), padding=nk - 1, groups=w.shape[0])
    ref = torch.nn.functional.silu(pre[..., : x.shape[2]]).numpy()
    out, _ = oracle.conv_fwd(x, w, b, silu=True)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_width_one_is_elementwise():
    x, w, b = _case(3, nk=1)
    out, sf = oracle.conv_fwd(x, w, b, silu=True)
    np.testing.assert_allclose(out, _silu(w[None, :, 0:1] * x + b[None, :, None]),
                               rtol=1e-14, atol=1e-15)
    assert sf.shape == (x.shape[0], x.shape[1], 0)


def test_zero_input_gives_activation_of_bias():
    _, w, b = _case(4)
    out, sf = oracle.conv_fwd(np.zeros((2, 3, 7)), w, b, silu=True)
    np.testing.assert_allclose(out, np.broadcast_to(_silu(b)[None, :, None], out.shape),
                               rtol=1e-15, atol=0)
    assert not sf.any()


def test_initial_window_equals_prepended_inputs():
    x, w, b = _case(5)
    nk = w.shape[1]
    s0 = _rng(6).standard_normal((x.shape[0], x.shape[1], nk - 1))
    out, sf = oracle.conv_fwd(x, w, b, silu=True, init_state=s0)
    out_cat, sf_cat = oracle.conv_fwd(np.concatenate([s0, x], axis=2), w, b, silu=True)
    np.testing.assert_allclose(out, out_cat[:, :, nk - 1:], rtol=1e-15, atol=0)
    np.testing.assert_array_equal(sf, sf_cat)


@pytest.mark.parametrize("nl", [1, 2, 3, 9])
def test_final_window_is_last_inputs(nl):
    x, w, b = _case(7, nl=nl)
    nk = w.shape[1]
    s0 = _rng(8).standard_normal((x.shape[0], x.shape[1], nk - 1))
    _, sf = oracle.conv_fwd(x, w, b, init_state=s0)
    np.testing.assert_array_equal(sf, np.concatenate([s0, x], axis=2)[:, :, -(nk - 1):])
    _, sf0 = oracle.conv_fwd(x, w, b)
    np.testing.assert_array_equal(
        sf0, np.concatenate([np.zeros_like(s0), x], axis=2)[:, :, -(nk - 1):])


@pytest.mark.parametrize("split", [1, 2, 5, 10])
def test_scan_continues_from_final_window(split):
    x, w, b = _case(9)
    out, sf = oracle.conv_fwd(x, w, b, silu=True)
    o1, s1 = oracle.conv_fwd(x[:, :, :split], w, b, silu=True)
    o2, s2 = oracle.conv_fwd(x[:, :, split:], w, b, silu=True, init_state=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), out, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(s2, sf)


@pytest.mark.parametrize("silu", [False, True])
def test_decode_steps_reproduce_the_sequence(silu):
    x, w, b = _case(10, nl=8)
    nk = w.shape[1]
    s0 = _rng(11).standard_normal((x.shape[0], x.shape[1], nk - 1))
    out, sf = oracle.conv_fwd(x, w, b, silu=silu, init_state=s0)
    st = s0
    for t in range(x.shape[2]):
        st_next, o = oracle.conv_update(st, x[:, :, t], w, b, silu=silu)
        np.testing.assert_allclose(o, out[:, :, t], rtol=1e-15, atol=0)
        st = st_next
    np.testing.assert_array_equal(st, sf)


def test_decode_width_one_has_no_state():
    _, w, b = _case(12, nk=1)
    x = _rng(13).standard_normal((2, 3))
    st, o = oracle.conv_update(np.zeros((2, 3, 0)), x, w, b, silu=True)
    np.testing.assert_allclose(o, _silu(w[:, 0] * x + b), rtol=1e-15, atol=0)
    assert st.shape == (2, 3, 0)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def _loss(x, w, b, s0, dout, silu):
    out, _ = oracle.conv_fwd(x, w, b, silu=silu, init_state=s0)
    return float(np.sum(out * dout))


def _central(fn, arr, eps=1e-6):
    g = np.zeros_like(arr)
    if arr.size == 0:
        return g
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        keep = arr[i]
        arr[i] = keep + eps
        fp = fn()
        arr[i] = keep - eps
        fm = fn()
        arr[i] = keep
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("nk", [1, 3, 4])
def test_backward_matches_central_differences(silu, nk):
    x, w, b = _case(20 + nk, nb=2, nd=2, nl=6, nk=nk)
    s0 = _rng(30 + nk).standard_normal((2, 2, nk - 1))
    dout = _rng(40 + nk).standard_normal(x.shape)
    g = oracle.conv_bwd(x, w, b, silu=silu, init_state=s0, dout=dout)
    f = lambda: _loss(x, w, b, s0, dout, silu)  # noqa: E731
    for name, arr in (("dx", x), ("dweight", w), ("dbias", b), ("dinit_state", s0)):
        np.testing.assert_allclose(g[name], _central(f, arr), rtol=1e-6, atol=1e-8,
                                   err_msg=name)


def test_backward_matches_torch_autograd():
    x, w, b = _case(50, nb=3, nd=4, nl=13)
    nk = w.shape[1]
    s0 = _rng(51).standard_normal((3, 4, nk - 1))
    dout = _rng(52).standard_normal(x.shape)
    tx, tw, tb, ts = (torch.tensor(a, requires_grad=True) for a in (x, w, b, s0))
    pre = torch.nn.functional.conv1d(torch.cat([ts, tx], dim=2), tw[:, None, :], tb,
                                     groups=4)
    (torch.nn.functional.silu(pre) * torch.from_numpy(dout)).sum().backward()
    g = oracle.conv_bwd(x, w, b, silu=True, init_state=s0, dout=dout)
    for name, t in (("dx", tx), ("dweight", tw), ("dbias", tb), ("dinit_state", ts)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-12, atol=1e-13,
                                   err_msg=name)


def test_backward_without_window_or_bias():
    x, w, _ = _case(60)
    dout = _rng(61).standard_normal(x.shape)
    g = oracle.conv_bwd(x, w, None, silu=True, dout=dout)
    assert set(g) == {"dx", "dweight"}
    f = lambda: _loss(x, w, None, None, dout, True)  # noqa: E731
    np.testing.assert_allclose(g["dx"], _central(f, x), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g["dweight"], _central(f, w), rtol=1e-6, atol=1e-8)


def test_backward_threads_fold_in_batch_order():
    x, w, b = _case(70, nb=5, nd=3, nl=9)
    dout = _rng(71).standard_normal(x.shape)
    g1 = oracle.conv_bwd(x, w, b, dout=dout, threads=1)
    g3 = oracle.conv_bwd(x, w, b, dout=dout, threads=3)
    np.testing.assert_array_equal(g1["dx"], g3["dx"])
    np.testing.assert_allclose(g1["dweight"], g3["dweight"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(g1["dbias"], g3["dbias"], rtol=1e-14, atol=1e-14)
