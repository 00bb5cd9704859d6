"""Helpers shared by the GPU parity tests: moving seeded inputs to the
device and back, and running the oracle on the same stored values."""
import os
import sys

import numpy as np
import torch

from oracle import oracle
from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

DEV = "cuda:0"
# host threads for whole-workload oracle runs (one GPU's share of the host:
# at most 16 cores)
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "this test needs the MI355X"
    binding.load()  # fails loudly when libss.so is missing


def to_dev(a):
    """numpy (float32 or uint16 bf16 bits) -> torch tensor on the GPU."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_host(t):
    """torch tensor -> exact float64 numpy values."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return ssin.widen(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def widen(a):
    return None if a is None else ssin.widen(a).astype(np.float64)


def dev_inputs(arr):
    return {k: to_dev(v) for k, v in arr.items()}


def oracle_fwd(arr, softplus=True, h0=None, rows=None, threads=8):
    """Oracle forward on the stored inputs; rows = list of (b, d) to restrict to."""
    w = {k: widen(v) for k, v in arr.items()}
    if rows is None:
        return oracle.fwd(w["u"], w["delta"], w["A"], w["B"], w["C"], w.get("D"), w.get("z"),
                          w.get("delta_bias"), softplus, h0, threads=threads)
    ys, ls = [], []
    for b, d in rows:
        sl = lambda k: None if w.get(k) is None else w[k][b:b + 1, d:d + 1]  # noqa: E731
        y, l = oracle.fwd(sl("u"), sl("delta"), w["A"][d:d + 1], w["B"][b:b + 1],
                          w["C"][b:b + 1], None if w.get("D") is None else w["D"][d:d + 1],
                          sl("z"), None if w.get("delta_bias") is None else w["delta_bias"][d:d + 1],
                          softplus, None if h0 is None else h0[b:b + 1, d:d + 1])
        ys.append(y[0, 0])
        ls.append(l[0, 0])
    return np.stack(ys), np.stack(ls)
