"""Pins of the oracle's backward (reverse-time BPTT through the state).

The forward is pinned in test_oracle_pins.py; here the backward is checked
against it: central finite differences of the loss sum(dout * y)
(+ sum(dlast * last_state)) for every input element on tiny shapes, an
adjoint (directional-derivative) identity on a larger shape, hand-derived
one-step gradients, and additivity of the parameter gradients over the
batch.  A dropped term (say the B u part of d delta), a wrong sign or a
decay applied at the wrong step fails the finite differences.
"""
import math

import numpy as np
import pytest

from oracle import oracle


def _problem(seed, nb=2, nd=3, ns=4, nl=7, z=True, D=True, bias=True, h0=False,
             dlast=False, softplus=True):
    """Random problem; without softplus, delta and bias are drawn positive so
    that delta * A stays negative (a decaying, well-conditioned scan)."""
    r = np.random.default_rng(seed)
    delta = (0.5 * r.standard_normal((nb, nd, nl)) if softplus
             else r.uniform(0.05, 0.8, (nb, nd, nl)))
    p = dict(
        u=r.standard_normal((nb, nd, nl)), delta=delta,
        A=-r.uniform(0.3, 3.0, (nd, ns)), B=r.standard_normal((nb, ns, nl)),
        C=r.standard_normal((nb, ns, nl)))
    p["D"] = r.standard_normal(nd) if D else None
    p["z"] = r.standard_normal((nb, nd, nl)) if z else None
    if bias:
        p["delta_bias"] = (np.log(np.expm1(r.uniform(1e-3, 1e-1, nd))) if softplus
                           else r.uniform(0.0, 0.1, nd))
    else:
        p["delta_bias"] = None
    p["h0"] = r.standard_normal((nb, nd, ns)) if h0 else None
    dout = r.standard_normal((nb, nd, nl))
    dl = r.standard_normal((nb, nd, ns)) if dlast else None
    return p, dout, dl


def _loss(p, dout, dlast, softplus):
    y, last = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                         p["delta_bias"], softplus, p["h0"])
    val = float(np.sum(dout * y))
    if dlast is not None:
        val += float(np.sum(dlast * last))
    return val


GRAD_NAME = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "z": "dz", "delta_bias": "ddelta_bias", "h0": "dh0"}


def _check_fd(p, dout, dlast, softplus):
    g = oracle.bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                   p["delta_bias"], softplus, dout, p["h0"], dlast)
    for name, grad_key in GRAD_NAME.items():
        if p.get(name) is None:
            assert grad_key not in g
            continue
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            h = 1e-6 * max(1.0, abs(old))
            x[idx] = old + h
            lp = _loss(p, dout, dlast, softplus)
            x[idx] = old - h
            lm = _loss(p, dout, dlast, softplus)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(np.max(np.abs(fd)), 1e-3)
        err = np.max(np.abs(g[grad_key] - fd)) / scale
        assert err < 2e-7, f"{grad_key}: max error {err:.3e} (scale {scale:.3e})"


@pytest.mark.parametrize("softplus", [True, False])
def test_fd_all_inputs_with_every_option(softplus):
    p, dout, dl = _problem(1, h0=True, dlast=True, softplus=softplus)
    _check_fd(p, dout, dl, softplus)


@pytest.mark.parametrize(
    "opts",
    [dict(z=False), dict(D=False), dict(bias=False), dict(z=False, D=False, bias=False)],
    ids=["no_z", "no_D", "no_bias", "bare"])
def test_fd_optional_inputs_absent(opts):
    p, dout, dl = _problem(2, nb=1, nd=2, ns=3, nl=6, **opts)
    _check_fd(p, dout, dl, softplus=True)


def test_adjoint_identity_larger_shape():
    """<grad, v> equals the directional derivative of the loss along v."""
    p, dout, _ = _problem(3, nb=2, nd=5, ns=16, nl=48)
    g = oracle.bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                   p["delta_bias"], True, dout)
    r = np.random.default_rng(4)
    v = {k: r.standard_normal(p[k].shape) for k in GRAD_NAME if p.get(k) is not None}
    pred = sum(float(np.sum(g[GRAD_NAME[k]] * v[k])) for k in v)
    eps = 1e-5

    def at(s):
        q = {k: (p[k] + s * v[k] if k in v else p[k]) for k in p}
        return _loss(q, dout, None, True)

    fd = (at(eps) - at(-eps)) / (2 * eps)
    assert pred == pytest.approx(fd, rel=1e-7)


def test_one_step_closed_form_gradients():
    """L = 1 with an initial state, written out by hand:
    h = a h0 + dl B u, a = exp(dl A); pre = sum C h + D u; y = pre silu(z)."""
    r = np.random.default_rng(5)
    ns = 5
    A = -r.uniform(0.5, 2.0, (1, ns))
    B, C, h0 = r.standard_normal(ns), r.standard_normal(ns), r.standard_normal(ns)
    u, raw, z, D, dout = r.standard_normal(5)
    g = oracle.bwd(np.full((1, 1, 1), u), np.full((1, 1, 1), raw), A,
                   B.reshape(1, ns, 1), C.reshape(1, ns, 1), np.array([D]),
                   np.full((1, 1, 1), z), None, False, np.full((1, 1, 1), dout),
                   h0.reshape(1, 1, ns))
    dl = raw                     # no bias, no softplus
    a = np.exp(dl * A[0])
    h = a * h0 + dl * B * u
    pre = float(C @ h) + D * u
    sig = 1.0 / (1.0 + math.exp(-z))
    dy = dout * z * sig
    assert g["dz"][0, 0, 0] == pytest.approx(dout * pre * (sig + z * sig * (1 - sig)), rel=1e-12)
    assert g["dD"][0] == pytest.approx(dy * u, rel=1e-12)
    np.testing.assert_allclose(g["dC"][0, :, 0], dy * h, rtol=1e-12)
    np.testing.assert_allclose(g["dB"][0, :, 0], dy * C * dl * u, rtol=1e-12)
    assert g["du"][0, 0, 0] == pytest.approx(dy * (dl * float(C @ B) + D), rel=1e-12)
    assert g["ddelta"][0, 0, 0] == pytest.approx(
        dy * float(np.sum(C * (A[0] * a * h0 + B * u))), rel=1e-12)
    np.testing.assert_allclose(g["dA"][0], dy * C * dl * a * h0, rtol=1e-12)
    np.testing.assert_allclose(g["dh0"][0, 0], dy * C * a, rtol=1e-12)


def test_parameter_grads_add_over_batch():
    p, dout, _ = _problem(6, nb=3, nd=4, ns=5, nl=10)
    kw = lambda q: (q["A"], q["B"], q["C"], q["D"], q["z"], q["delta_bias"])  # noqa: E731
    full = oracle.bwd(p["u"], p["delta"], *kw(p), True, dout)
    acc = {k: 0.0 for k in ("dA", "dD", "ddelta_bias")}
    for b in range(3):
        q = dict(p)
        for k in ("u", "delta", "B", "C", "z"):
            q[k] = p[k][b:b + 1]
        part = oracle.bwd(q["u"], q["delta"], *kw(q), True, dout[b:b + 1])
        for k in acc:
            acc[k] = acc[k] + part[k]
        np.testing.assert_allclose(full["dB"][b], part["dB"][0], rtol=1e-13)
        np.testing.assert_allclose(full["du"][b], part["du"][0], rtol=1e-13)
    for k in acc:
        np.testing.assert_allclose(full[k], acc[k], rtol=1e-12, atol=1e-14)


def test_threaded_batches_match_single_thread():
    p, dout, _ = _problem(8, nb=4, nd=3, ns=4, nl=9)
    args = (p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
            True, dout)
    g1 = oracle.bwd(*args)
    g2 = oracle.bwd(*args, threads=2)
    for k in g1:
        np.testing.assert_allclose(g1[k], g2[k], rtol=1e-14, atol=1e-15)
