"""Pins of the double-precision oracle against things other than itself.

Every check here runs on the CPU.  The expected values come from closed
forms (special values of softplus and silu, one-step and pure-decay
formulas, geometric series), a brute-force time-invariant convolution that
evaluates each kernel tap directly, hand-derived worked examples stored
under ``tests/golden/``, and structural facts (linearity, causality,
continuation of a scan from its last state).  Each is chosen so that a
plausible slip in the oracle -- a dropped term, a wrong sign, a transposed
B/C index, a decay taken per step instead of from the accumulated delta --
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN2 = math.log(2.0)


def _fwd(u, delta, A, B, C, D=None, z=None, bias=None, softplus=False, h0=None):
    return oracle.fwd(u, delta, A, B, C, D, z, bias, softplus, h0)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# delta preparation: softplus and bias, read off through a single step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize(
    "raw,bias,softplus,expect",
    [
        (0.0, 0.0, True, LN2),                       # softplus(0) = ln 2
        (math.log(math.e - 1.0), 0.0, True, 1.0),    # softplus(ln(e - 1)) = 1
        (0.0, math.log(math.expm1(0.05)), True, 0.05),  # bias = softplus^-1(0.05)
        (60.0, 0.0, True, 60.0),                     # softplus(x) -> x for large x
        (-60.0, 0.0, True, math.exp(-60.0)),         # softplus(x) -> e^x for very negative x
        (0.3, -0.2, False, 0.1),                     # no softplus: raw + bias
        (-0.7, 0.0, False, -0.7),
    ],
)
def test_delta_preparation(raw, bias, softplus, expect):
    # A = 0 (no decay), B = C = u = 1, zero initial state: y_0 = delta itself.
    one = np.ones((1, 1, 1))
    y, last = _fwd(one, np.full((1, 1, 1), raw), np.zeros((1, 1)), one, one,
                   bias=np.array([bias]), softplus=softplus)
    assert y[0, 0, 0] == pytest.approx(expect, rel=1e-13, abs=0)
    assert last[0, 0, 0] == pytest.approx(expect, rel=1e-13, abs=0)


@pytest.mark.parametrize(
    "zval,expect",
    [
        (0.0, 0.0),
        (1.0, math.e / (1.0 + math.e)),              # silu(1) = e / (1 + e)
        (-1.0, -1.0 / (1.0 + math.e)),               # silu(-1) = -1 / (1 + e)
        (math.log(3.0), math.log(3.0) * 0.75),       # sigmoid(ln 3) = 3/4
        (-40.0, -40.0 * math.exp(-40.0) / (1 + math.exp(-40.0))),
    ],
)
def test_gate_values(zval, expect):
    # C = 0 removes the state; D = 2, u = 1.5 gives y = 3 * silu(z).
    y, _ = _fwd(np.full((1, 1, 1), 1.5), np.ones((1, 1, 1)), -np.ones((1, 1)),
                np.ones((1, 1, 1)), np.zeros((1, 1, 1)), D=np.array([2.0]),
                z=np.full((1, 1, 1), zval))
    assert y[0, 0, 0] == pytest.approx(3.0 * expect, rel=1e-13, abs=1e-300)


# ---------------------------------------------------------------------------
# hand-derived worked examples (tests/golden)
# ---------------------------------------------------------------------------
def _tok(t):
    table = {"ln2": LN2, "-ln2": -LN2, "-ln4": -math.log(4.0), "1/ln2": 1 / LN2,
             "-1/ln2": -1 / LN2}
    if t in table:
        return table[t]
    if t.startswith("e^"):
        return math.exp(float(t[2:]))
    return float(t)


def _golden_cases():
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, "fwd_worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    cases.append(cur)
                cur = {}
                continue
            k, v = line.split(":", 1)
            cur[k.strip()] = v.split()
    if cur:
        cases.append(cur)
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"][0])
def test_golden_worked_examples(case):
    nb, nd, ns, nl = (int(case[k][0]) for k in ("batch", "dim", "dstate", "seqlen"))
    arr = {k: np.array([_tok(t) for t in case[k]]) for k in case
           if k not in ("name", "batch", "dim", "dstate", "seqlen", "softplus")}
    y, last = _fwd(arr["u"].reshape(nb, nd, nl), arr["delta"].reshape(nb, nd, nl),
                   arr["A"].reshape(nd, ns), arr["B"].reshape(nb, ns, nl),
                   arr["C"].reshape(nb, ns, nl), D=arr.get("D"),
                   z=arr["z"].reshape(nb, nd, nl) if "z" in arr else None,
                   softplus=bool(int(case["softplus"][0])))
    np.testing.assert_allclose(y.ravel(), arr["y"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(last.ravel(), arr["last_state"], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# brute-force time-invariant convolution
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lti_bruteforce_convolution(seed):
    """Constant delta, B, C per row: y_t = sum_k K_k u_{t-k} + D u_t with
    K_k = sum_n C_n exp(k delta A_n) delta B_n, each tap evaluated directly."""
    r = _rng(seed)
    nb, nd, ns, nl = 2, 3, 5, 37
    A = -r.uniform(0.05, 2.0, (nd, ns))
    dconst = r.uniform(0.05, 1.5, (nb, nd))
    Bc, Cc = r.standard_normal((nb, ns)), r.standard_normal((nb, ns))
    D = r.standard_normal(nd)
    u = r.standard_normal((nb, nd, nl))
    delta = np.repeat(dconst[:, :, None], nl, axis=2)
    B = np.repeat(Bc[:, :, None], nl, axis=2)
    C = np.repeat(Cc[:, :, None], nl, axis=2)
    y, last = _fwd(u, delta, A, B, C, D=D)
    for b in range(nb):
        for d in range(nd):
            dl = dconst[b, d]
            K = np.array([sum(Cc[b, n] * math.exp(k * dl * A[d, n]) * dl * Bc[b, n]
                              for n in range(ns)) for k in range(nl)])
            for t in range(nl):
                ref = sum(K[k] * u[b, d, t - k] for k in range(t + 1)) + D[d] * u[b, d, t]
                assert y[b, d, t] == pytest.approx(ref, rel=1e-11, abs=1e-12)
            for n in range(ns):
                ref = sum(math.exp((nl - 1 - s) * dl * A[d, n]) * dl * Bc[b, n] * u[b, d, s]
                          for s in range(nl))
                assert last[b, d, n] == pytest.approx(ref, rel=1e-11, abs=1e-13)


# ---------------------------------------------------------------------------
# pure decay after an impulse, with time-varying delta, B and C
# ---------------------------------------------------------------------------
def test_impulse_decays_with_accumulated_delta():
    """u_0 = 1, u_t = 0 afterwards: h_t[n] = exp(A_n * sum_{j=1..t} delta_j)
    * delta_0 * B[n, 0]; y_t = sum_n C[n, t] h_t[n].  N != L and B, C vary in
    both n and t, so a transposed index or a per-step decay would show."""
    r = _rng(7)
    nb, nd, ns, nl = 2, 3, 6, 11
    A = -r.uniform(0.1, 3.0, (nd, ns))
    delta = r.uniform(0.01, 0.8, (nb, nd, nl))
    B = r.standard_normal((nb, ns, nl))
    C = r.standard_normal((nb, ns, nl))
    u = np.zeros((nb, nd, nl))
    u[:, :, 0] = 1.0
    y, last = _fwd(u, delta, A, B, C)
    for b in range(nb):
        for d in range(nd):
            for t in range(nl):
                s = delta[b, d, 1:t + 1].sum()
                h = [math.exp(A[d, n] * s) * delta[b, d, 0] * B[b, n, 0] for n in range(ns)]
                ref = sum(C[b, n, t] * h[n] for n in range(ns))
                assert y[b, d, t] == pytest.approx(ref, rel=1e-12, abs=1e-15)
                if t == nl - 1:
                    np.testing.assert_allclose(last[b, d], h, rtol=1e-12)


def test_scalar_geometric_series():
    """N = 1, constant decay a = exp(delta A): h_t = sum_s a^(t-s) delta B_s u_s,
    with the powers taken by repeated multiplication."""
    r = _rng(3)
    nl, dl, a_cont = 25, 0.37, -1.3
    u = r.standard_normal(nl)
    B = r.standard_normal(nl)
    C = r.standard_normal(nl)
    y, _ = _fwd(u.reshape(1, 1, nl), np.full((1, 1, nl), dl), np.array([[a_cont]]),
                B.reshape(1, 1, nl), C.reshape(1, 1, nl))
    a = math.exp(dl * a_cont)
    for t in range(nl):
        h, p = 0.0, 1.0
        for s in range(t, -1, -1):
            h += p * dl * B[s] * u[s]
            p *= a
        assert y[0, 0, t] == pytest.approx(C[t] * h, rel=1e-12, abs=1e-15)


# ---------------------------------------------------------------------------
# structural invariants
# ---------------------------------------------------------------------------
def _random_problem(seed, nb=2, nd=4, ns=6, nl=19):
    r = _rng(seed)
    return dict(
        u=r.standard_normal((nb, nd, nl)), delta=0.5 * r.standard_normal((nb, nd, nl)),
        A=-r.uniform(0.5, 8.0, (nd, ns)), B=r.standard_normal((nb, ns, nl)),
        C=r.standard_normal((nb, ns, nl)), D=r.standard_normal(nd),
        z=r.standard_normal((nb, nd, nl)),
        bias=np.log(np.expm1(r.uniform(1e-3, 1e-1, nd))))


def test_linear_in_u_without_gate():
    p = _random_problem(11)
    r = _rng(12)
    u2 = r.standard_normal(p["u"].shape)
    args = (p["delta"], p["A"], p["B"], p["C"])
    kw = dict(D=p["D"], bias=p["bias"], softplus=True)
    y1, _ = _fwd(p["u"], *args, **kw)
    y2, _ = _fwd(u2, *args, **kw)
    y12, _ = _fwd(2.0 * p["u"] - 3.0 * u2, *args, **kw)
    np.testing.assert_allclose(y12, 2.0 * y1 - 3.0 * y2, rtol=1e-10, atol=1e-12)


def test_causal():
    p = _random_problem(13)
    kw = dict(D=p["D"], z=p["z"], bias=p["bias"], softplus=True)
    y1, _ = _fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], **kw)
    u = p["u"].copy()
    u[:, :, 9:] += 1.0
    dl = p["delta"].copy()
    dl[:, :, 9:] -= 0.4
    y2, _ = _fwd(u, dl, p["A"], p["B"], p["C"], **kw)
    np.testing.assert_array_equal(y1[:, :, :9], y2[:, :, :9])
    assert np.all(y1[:, :, 9:] != y2[:, :, 9:])


def test_zero_C_leaves_gated_skip():
    p = _random_problem(14)
    y, _ = _fwd(p["u"], p["delta"], p["A"], p["B"], np.zeros_like(p["C"]), D=p["D"],
                z=p["z"], bias=p["bias"], softplus=True)
    z = p["z"]
    expect = p["D"][None, :, None] * p["u"] * z / (1.0 + np.exp(-z))
    np.testing.assert_allclose(y, expect, rtol=1e-13, atol=1e-15)


def test_continuation_from_last_state():
    """Scanning [0, L1) and then [L1, L) from the carried state equals one scan."""
    p = _random_problem(15, nl=30)
    kw = dict(D=p["D"], bias=p["bias"], softplus=True)
    y, last = _fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], z=p["z"], **kw)
    cut = 13
    sl = lambda a, s: a[:, :, s]  # noqa: E731
    ya, la = _fwd(sl(p["u"], slice(0, cut)), sl(p["delta"], slice(0, cut)), p["A"],
                  sl(p["B"], slice(0, cut)), sl(p["C"], slice(0, cut)),
                  z=sl(p["z"], slice(0, cut)), **kw)
    yb, lb = _fwd(sl(p["u"], slice(cut, None)), sl(p["delta"], slice(cut, None)), p["A"],
                  sl(p["B"], slice(cut, None)), sl(p["C"], slice(cut, None)),
                  z=sl(p["z"], slice(cut, None)), h0=la, **kw)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=2), y, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lb, last, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# one-token state update
# ---------------------------------------------------------------------------
def test_state_update_one_step_closed_form():
    r = _rng(21)
    nb, nd, ns = 3, 5, 4
    st = r.standard_normal((nb, nd, ns))
    u, dr, z = (r.standard_normal((nb, nd)) for _ in range(3))
    A = -r.uniform(0.5, 4.0, (nd, ns))
    B, C = r.standard_normal((nb, ns)), r.standard_normal((nb, ns))
    D = r.standard_normal(nd)
    new, y = oracle.state_update(st, u, dr, A, B, C, D, z, None, False)
    for b in range(nb):
        for d in range(nd):
            dl = dr[b, d]
            h = [math.exp(dl * A[d, n]) * st[b, d, n] + dl * B[b, n] * u[b, d]
                 for n in range(ns)]
            np.testing.assert_allclose(new[b, d], h, rtol=1e-13)
            pre = sum(C[b, n] * h[n] for n in range(ns)) + D[d] * u[b, d]
            zz = z[b, d]
            assert y[b, d] == pytest.approx(pre * zz / (1 + math.exp(-zz)), rel=1e-12)


def test_state_update_repeated_equals_scan():
    """k updates from a zero state reproduce the scan over those k steps."""
    p = _random_problem(22, nl=9)
    nb, nd, nl = p["u"].shape
    ns = p["A"].shape[1]
    y, last = _fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                   bias=p["bias"], softplus=True)
    st = np.zeros((nb, nd, ns))
    for t in range(nl):
        st, yt = oracle.state_update(st, p["u"][:, :, t], p["delta"][:, :, t], p["A"],
                                     p["B"][:, :, t], p["C"][:, :, t], p["D"],
                                     p["z"][:, :, t], p["bias"], True)
        np.testing.assert_allclose(yt, y[:, :, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st, last, rtol=1e-12, atol=1e-14)


def test_threaded_rows_match_single_thread():
    p = _random_problem(23, nb=3, nd=5)
    kw = dict(D=p["D"], z=p["z"], delta_bias=p["bias"], delta_softplus=True)
    y1, l1 = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], **kw)
    y4, l4 = oracle.fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], threads=4, **kw)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(l1, l4)
