"""Pins of the oracle's Mamba-2 SSD forward and backward against things other than itself.

The reading pinned here (the pages name SSD without printing it): per
batch and head a headdim x d_state state, H_t = exp(dt_t A_h) H_{t-1} +
dt_t x_t B_t^T, y_t = H_t C_t + D_h x_t, B and C shared by the heads of a
group (heads grouped contiguously).  Expected values come from

  * the quadratic ("dual") form of the same map, evaluated with numpy in
    f64: y_t = sum_{s<=t} exp(cum_t - cum_s) (C_t . B_s) dt_s x_s +
    exp(cum_t) H_{-1} C_t + D x_t, cum_t the running sum of dt A -- a
    different algorithm (no recurrence) that must agree to rounding;
  * the Mamba-1 oracle, which is pinned on its own: with one group, SSD is
    the selective scan with one channel per (head, column), delta shared by
    the columns of a head and A[d, n] = A_h for every n;
  * structural facts: continuation from the last state, no decay and no
    input at dt = 0.

The backward (back-propagation through time) is pinned to central
differences of the forward for every input, with and without softplus and
with two groups, and, with one group, to the Mamba-1 oracle's backward with
the tied parameters' gradients summed.

A wrong decay sign, a dropped dt on the input, C and B exchanged, a wrong
head-to-group map, a dropped D term, an ignored initial state, a missing
adjoint carry, dB without dt, dA without the decay, or dC from the
previous state fails at least one of them.
"""
import numpy as np
import pytest

from oracle import oracle


def _case(seed, nb=2, nl=23, nh=4, npd=3, ng=2, ns=5, h0=True):
    r = np.random.default_rng(seed)
    return dict(x=r.standard_normal((nb, nl, nh, npd)),
                dt=0.5 * r.standard_normal((nb, nl, nh)),
                A=-np.exp(r.uniform(-1.0, 1.0, nh)),
                B=r.standard_normal((nb, nl, ng, ns)),
                C=r.standard_normal((nb, nl, ng, ns)),
                D=r.standard_normal(nh),
                dt_bias=r.uniform(-1.0, 0.5, nh),
                h0=r.standard_normal((nb, nh, npd, ns)) if h0 else None)


def _quadratic(c, softplus=True):
    x, B, C = c["x"], c["B"], c["C"]
    nb, nl, nh, npd = x.shape
    ng = B.shape[2]
    dt = c["dt"] + c["dt_bias"][None, None, :]
    if softplus:
        dt = np.logaddexp(0.0, dt)
    cum = np.cumsum(dt * c["A"][None, None, :], axis=1)           # (b, t, h)
    gi = np.arange(nh) // (nh // ng)
    Bh, Ch = B[:, :, gi, :], C[:, :, gi, :]                       # (b, t, h, n)
    G = np.einsum("bthn,bshn->bhts", Ch, Bh)                      # C_t . B_s
    seg = cum.transpose(0, 2, 1)[:, :, :, None] - cum.transpose(0, 2, 1)[:, :, None, :]
    mask = np.tril(np.ones((nl, nl), dtype=bool))
    Lm = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)   # exp(cum_t - cum_s), s <= t
    W = G * Lm * dt.transpose(0, 2, 1)[:, :, None, :]             # times dt_s
    y = np.einsum("bhts,bshp->bthp", W, x)
    if c.get("h0") is not None:
        y += np.einsum("bth,bthn,bhpn->bthp", np.exp(cum), Ch, c["h0"])
    return y + c["D"][None, None, :, None] * x


def _run(c, softplus=True):
    return oracle.ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["dt_bias"],
                          softplus, c.get("h0"))


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("ng,h0", [(1, False), (2, True), (4, True)])
def test_matches_quadratic_dual_form(softplus, ng, h0):
    c = _case(ng + 10 * h0, ng=ng, h0=h0)
    y, _ = _run(c, softplus)
    np.testing.assert_allclose(y, _quadratic(c, softplus), rtol=1e-10, atol=1e-10)


def test_one_group_is_the_selective_scan():
    c = _case(3, nb=2, nl=31, nh=3, npd=4, ng=1, ns=6)
    y, last = _run(c)
    nb, nl, nh, npd = c["x"].shape
    ns = c["B"].shape[3]
    # channel d = (head, column); delta, A and D follow the head
    u = c["x"].reshape(nb, nl, nh * npd).transpose(0, 2, 1)
    delta = np.repeat(c["dt"], npd, axis=2).transpose(0, 2, 1)
    A = np.repeat(c["A"], npd)[:, None] * np.ones((1, ns))
    Bs = c["B"][:, :, 0, :].transpose(0, 2, 1)
    Cs = c["C"][:, :, 0, :].transpose(0, 2, 1)
    D = np.repeat(c["D"], npd)
    bias = np.repeat(c["dt_bias"], npd)
    h0 = c["h0"].reshape(nb, nh * npd, ns)
    ys, ls = oracle.fwd(u, delta, A, Bs, Cs, D, None, bias, True, h0)
    np.testing.assert_allclose(y.reshape(nb, nl, nh * npd).transpose(0, 2, 1), ys,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(last.reshape(nb, nh * npd, ns), ls, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [1, 9, 22])
def test_continues_from_last_state(split):
    c = _case(4)
    y, last = _run(c)
    a = dict(c, x=c["x"][:, :split], dt=c["dt"][:, :split], B=c["B"][:, :split],
             C=c["C"][:, :split])
    y1, l1 = _run(a)
    b = dict(c, x=c["x"][:, split:], dt=c["dt"][:, split:], B=c["B"][:, split:],
             C=c["C"][:, split:], h0=l1)
    y2, l2 = _run(b)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l2, last, rtol=1e-12, atol=1e-12)


def test_zero_step_keeps_the_state():
    # dt = 0 without softplus or bias: no decay, no input; y = h0 C + D x
    c = _case(5)
    c["dt"] = np.zeros_like(c["dt"])
    c["dt_bias"] = np.zeros_like(c["dt_bias"])
    y, last = _run(c, softplus=False)
    nh, ng = c["x"].shape[2], c["B"].shape[2]
    Ch = c["C"][:, :, np.arange(nh) // (nh // ng), :]
    ref = np.einsum("bthn,bhpn->bthp", Ch, c["h0"]) + c["D"][None, None, :, None] * c["x"]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(last, c["h0"])


def test_threads_split_batch_only():
    c = _case(6, nb=5)
    y1, l1 = oracle.ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["dt_bias"], True,
                            c["h0"], threads=1)
    y3, l3 = oracle.ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["dt_bias"], True,
                            c["h0"], threads=3)
    np.testing.assert_array_equal(y1, y3)
    np.testing.assert_array_equal(l1, l3)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def _loss(c, dy, dlast, softplus=True):
    y, last = _run(c, softplus)
    return float(np.sum(y * dy) + np.sum(last * dlast))


def _central(fn, arr, eps=1e-6):
    g = np.zeros_like(arr)
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


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("ng", [1, 2])
def test_backward_matches_central_differences(softplus, ng):
    c = _case(40 + ng, nb=2, nl=7, nh=2, npd=2, ng=ng, ns=3)
    if not softplus:
        c["dt"] = np.abs(c["dt"])
        c["dt_bias"] = np.zeros_like(c["dt_bias"])
    r = np.random.default_rng(50 + ng)
    dy = r.standard_normal(c["x"].shape)
    dlast = r.standard_normal(c["h0"].shape)
    g = oracle.ssd_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["dt_bias"], softplus,
                       c["h0"], dy, dlast)
    f = lambda: _loss(c, dy, dlast, softplus)  # noqa: E731
    for name, key in (("dx", "x"), ("ddt", "dt"), ("dA", "A"), ("dB", "B"), ("dC", "C"),
                      ("dD", "D"), ("ddt_bias", "dt_bias"), ("dh0", "h0")):
        np.testing.assert_allclose(g[name], _central(f, c[key]), rtol=1e-6, atol=1e-7,
                                   err_msg=name)


def test_backward_one_group_is_the_selective_scan_backward():
    c = _case(60, nb=2, nl=19, nh=3, npd=4, ng=1, ns=5)
    nb, nl, nh, npd = c["x"].shape
    ns = c["B"].shape[3]
    r = np.random.default_rng(61)
    dy = r.standard_normal(c["x"].shape)
    dlast = r.standard_normal(c["h0"].shape)
    g = oracle.ssd_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], c["dt_bias"], True,
                       c["h0"], dy, dlast)
    u = c["x"].reshape(nb, nl, nh * npd).transpose(0, 2, 1)
    delta = np.repeat(c["dt"], npd, axis=2).transpose(0, 2, 1)
    A = np.repeat(c["A"], npd)[:, None] * np.ones((1, ns))
    Bs = c["B"][:, :, 0, :].transpose(0, 2, 1)
    Cs = c["C"][:, :, 0, :].transpose(0, 2, 1)
    D = np.repeat(c["D"], npd)
    bias = np.repeat(c["dt_bias"], npd)
    s6 = oracle.bwd(u, delta, A, Bs, Cs, D, None, bias, True,
                    dy.reshape(nb, nl, nh * npd).transpose(0, 2, 1),
                    c["h0"].reshape(nb, nh * npd, ns), dlast.reshape(nb, nh * npd, ns))
    tie = lambda a: a.reshape(nh, npd, *a.shape[1:]).sum(axis=1)  # noqa: E731
    np.testing.assert_allclose(g["dx"], s6["du"].transpose(0, 2, 1).reshape(c["x"].shape),
                               rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["ddt"], s6["ddelta"].reshape(nb, nh, npd, nl).sum(axis=2)
                               .transpose(0, 2, 1), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dA"], tie(s6["dA"]).sum(axis=1), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dB"][:, :, 0, :], s6["dB"].transpose(0, 2, 1), rtol=1e-11,
                               atol=1e-11)
    np.testing.assert_allclose(g["dC"][:, :, 0, :], s6["dC"].transpose(0, 2, 1), rtol=1e-11,
                               atol=1e-11)
    np.testing.assert_allclose(g["dD"], tie(s6["dD"]), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["ddt_bias"], tie(s6["ddelta_bias"]), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dh0"].reshape(nb, nh * npd, ns), s6["dh0"], rtol=1e-11,
                               atol=1e-11)
