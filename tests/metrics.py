"""Error metric used by every parity test.

Strict elementwise relative error is ill-posed where the reference crosses
zero (the silu gate and the channel sums of dB and dC produce many such
values), so each tensor is judged by

    err = max_i |x_i - r_i| / max(|r_i|, rms(r))

against 1e-4 when the inputs and outputs are float32 and 2e-2 when they are
bfloat16.  The reading is documented with the other readings of the pages.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(x)))
    den = np.maximum(np.abs(r), rms)
    return float(np.max(np.abs(x - r) / den))


def assert_close(x, r, tol, name=""):
    e = rel_err(x, r)
    assert np.all(np.isfinite(np.asarray(x, dtype=np.float64))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: error {e:.3e} > {tol:.1e}"
    return e
