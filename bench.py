#!/usr/bin/env python3
"""Benchmark of the selective scan on one MI355X.

A step is one forward (ss_fwd) and one backward (ss_bwd) over a batch of the
Mamba-130m-shaped layer: batch 8, d_inner 1536, d_state 16, L 2048, float32
inputs and outputs, z gate, D skip, delta bias and softplus, synthetic seeded
inputs already resident in HBM.  The line printed is

  value = batch * d_inner * L / (time of one step)   [elements/s]

with each library kernel also timed on its own (HIP events recorded between
the kernels on the stream they run on), the dominant kernel set against the
MI355X roofline, and the plain f64 oracle timed on a bounded sample of the
same workload on the host cores.  The forward-only and decode workloads,
the d_state 64 step, the causal convolution (width 4) that feeds the scan
and the Mamba-2 SSD forward are timed as well and reported under "detail".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan fwd+bwd elements/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
N = 16


def hip_runtime():
    names = ["libamdhip64.so.7", "libamdhip64.so"]
    import torch
    names.append(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    for n in names:
        try:
            lib = ctypes.CDLL(n)
            lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            return lib
        except OSError:
            continue
    raise RuntimeError("HIP runtime library not found")


class KernelTimer:
    """Arms libss's profiling hook with HIP events and reads back durations."""

    def __init__(self, hip, sslib, count):
        self.hip, self.ss = hip, sslib
        self.events = (ctypes.c_void_p * count)()
        for i in range(count):
            ev = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(ev)) == 0
            self.events[i] = ev
        self.count = count
        self.ss.ss_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_int]
        self.ss.ss_profile_events_used.restype = ctypes.c_int

    def arm(self):
        self.ss.ss_profile_events(ctypes.cast(self.events, ctypes.c_void_p), self.count)

    def disarm(self):
        used = self.ss.ss_profile_events_used()
        self.ss.ss_profile_events(None, 0)
        return used

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.events[i], self.events[j]) == 0
        return out.value

    def close(self):
        for i in range(self.count):
            self.hip.hipEventDestroy(self.events[i])


def algorithmic_bytes(kernel, batch, dim, L, esize):
    """Bytes each kernel must move if every tensor it reads or writes crosses
    HBM exactly once (workspace traffic excluded)."""
    E = batch * dim * L
    bc = batch * N * L * esize           # one of B, C, dB, dC
    params = dim * N * 4 + 2 * dim * 4     # A, D, delta_bias (or their gradients)
    if kernel == "ss_fwd_kernel":
        return 3 * E * esize + 2 * bc + params + E * esize
    if kernel == "ss_bwd_ckpt_kernel":
        return 2 * E * esize + bc + dim * N * 4 + dim * 4
    if kernel == "ss_bwd_reverse_kernel":
        return 4 * E * esize + 2 * bc + params + 3 * E * esize
    if kernel == "ss_bwd_fold_kernel":
        return 2 * bc + params
    if kernel == "ss_state_update_kernel":
        return 2 * batch * dim * N * 4 + 4 * batch * dim * esize + 2 * batch * N * esize + params
    raise KeyError(kernel)


def conv_algorithmic_bytes(kernel, batch, dim, L, width, esize):
    """The same count for the causal convolution kernels (width-tap weights
    and bias, and their gradients, in f32)."""
    E = batch * dim * L
    params = dim * (width + 1) * 4
    if kernel == "conv_fwd":      # x in, out
        return 2 * E * esize + params
    if kernel == "conv_bwd":      # x, dout in, dx out
        return 3 * E * esize + params
    if kernel == "conv_update":   # window in and out, x in, out
        return batch * dim * (2 * (width - 1) * 4 + 2 * esize) + params
    raise KeyError(kernel)


# Algorithmic floating-point operations per element (b, d, t) with d_state 16,
# counted from the recurrence as the oracle writes it (multiply, add = 1,
# fused multiply-add = 2, exp / log / reciprocal = 1): per state 5 for the
# forward step and 15 for the adjoint step and its sums, per element 21 for
# softplus, the gate and the element gradients.  The reverse pass of the
# step recomputes the forward states (the forward saved the pre-gate output,
# so not C h and its sum: 2 more per state otherwise).
FLOPS_PER_ELEMENT = {"ss_fwd_kernel": 16 * 7 + 11,          # 123
                     "ss_bwd_reverse_kernel": 16 * 20 + 21,  # 341
                     "ss_bwd_fold_kernel": 0}
# MI355X f32 vector peak: 256 CUs x 128 FMA lanes per clock x 2 FLOP x
# 2.4 GHz = 157.3 TFLOP/s.
ALU_PEAK_TFLOPS = 256 * 128 * 2 * 2.4e9 / 1e12

KERNEL_SOURCES = {
    "ss_fwd_kernel": ["ss_fwd.hip", "ss_tiles.h", "ss_device.h", "ss_kernels.h"],
    "ss_bwd_reverse_kernel": ["ss_bwd.hip", "ss_tiles.h", "ss_device.h", "ss_kernels.h"],
    "ss_bwd_fold_kernel": ["ss_bwd.hip", "ss_tiles.h", "ss_device.h", "ss_kernels.h"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when the summary is missing or the kernel's sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "selective_state_space_scan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("sources_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def timed_calls(hip, lib, calls, marks, iters):
    """Mean duration of each kernel of a library call: the calls rotate over
    their input sets; `marks` profiling events are recorded per call (one at
    the start and one after each kernel)."""
    import numpy as np
    import torch
    for c in calls:
        c()
    tm = KernelTimer(hip, lib, marks * iters)
    torch.cuda.synchronize()
    tm.arm()
    for i in range(iters):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    tm.disarm()
    out = [float(np.mean([tm.ms(marks * i + a, marks * i + a + 1) for i in range(iters)]))
           for a in range(marks - 1)]
    tm.close()
    return out


def wide_state_detail(hip, lib, to_dev, dev):
    """The fwd + bwd step at the Mamba-130m layer shape with d_state 64 (four
    16-state slices plus the combine kernels), f32 io."""
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin
    w = ssin.custom("bwd", 8, 1536, 64, 2048, "f32", seed=ssin.SEED_BASE + 20)
    d = {k: to_dev(v) for k, v in ssin.make(w).items()}
    y = torch.empty_like(d["u"])
    ck = binding.ss_ckpt_empty(d["u"], dstate=64)
    fws = torch.empty(binding.ss_fwd_workspace_size(w.batch, w.dim, 64, w.seqlen),
                      dtype=torch.uint8, device=dev)
    bws = torch.empty(binding.ss_bwd_workspace_size(w.batch, w.dim, 64, w.seqlen, 0),
                      dtype=torch.uint8, device=dev)

    def step():
        binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], True, out=y, ckpt=ck, workspace=fws)
        binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], True, d["dout"], workspace=bws, ckpt=ck)
    # per step: fwd [start, slices, combine]; bwd [start, reverse slices, combine, fold]
    parts = timed_calls(hip, lib, [step], 7, 5)
    names = ["fwd_slices_ms", "fwd_combine_ms", None, "bwd_reverse_slices_ms",
             "bwd_combine_ms", "bwd_fold_ms"]
    out = {n: round(v, 5) for n, v in zip(names, parts) if n}
    tot = sum(v for n, v in zip(names, parts) if n)
    out["step_kernels_ms"] = round(tot, 5)
    out["elements_per_s"] = w.elements / (tot * 1e-3)
    del d, y, ck, fws, bws
    return {"mamba130m_step_f32_8x1536x2048_dstate64": out}


def ssd_detail(hip, lib, to_dev, dev):
    """The Mamba-2 SSD at the 130M layer shape (batch 8, L 2048, 24 heads of
    64, d_state 128, one group, bf16): the forward kernel (inputs rotated over
    two copies), the backward call, and a forward + backward step in which
    the forward saves the chunk states for the backward."""
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin
    w = ssin.SSD_WORKLOADS["mamba2_130m_ssd_bf16_8x2048x24x64_n128"]
    a = ssin.make_ssd(w)
    sets = [{k: to_dev(v) for k, v in a.items()} for _ in range(2)]
    outs = [torch.empty_like(c["x"]) for c in sets]
    calls = [lambda c=c, o=o: binding.ss_ssd_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"],
                                                 c["dt_bias"], True, out=o)
             for c, o in zip(sets, outs)]
    (ms,) = timed_calls(hip, lib, calls, 2, 20)
    E = w.elements
    by = (2 * E * 2 + w.batch * w.seqlen * w.nheads * 2
          + 2 * w.batch * w.seqlen * w.ngroups * w.dstate * 2 + 3 * w.nheads * 4)
    # the chunked form's products per (batch, head, 64-step chunk): C B^T and
    # W x over the lower triangle, C H^T and the state update in full
    Q, N, P = 64, w.dstate, w.headdim
    fl = (Q * Q * N + Q * Q * P + 4 * Q * N * P) * w.batch * w.nheads * (w.seqlen // Q)
    del sets, outs
    # the backward (through the selective-scan backward), timed as a whole call
    wb = ssin.SSD_WORKLOADS["mamba2_130m_ssd_bwd_bf16_8x2048x24x64_n128"]
    db = {k: to_dev(v) for k, v in ssin.make_ssd(wb).items()}
    wsb = torch.empty(binding.ss_ssd_bwd_workspace_size(wb.batch, wb.seqlen, wb.nheads,
                                                        wb.headdim, wb.ngroups, wb.dstate),
                      dtype=torch.uint8, device=dev)

    def bwd():
        binding.ss_ssd_bwd(db["x"], db["dt"], db["A"], db["B"], db["C"], db["D"], db["dt_bias"],
                           True, dout=db["dout"], workspace=wsb)
    bwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    bms = e0.elapsed_time(e1) / 5
    # a training step: the forward saves the chunk states, the backward takes them
    ck = binding.ss_ssd_ckpt_empty(db["x"], wb.dstate)
    yb = torch.empty_like(db["x"])

    def step():
        binding.ss_ssd_fwd(db["x"], db["dt"], db["A"], db["B"], db["C"], db["D"], db["dt_bias"],
                           True, out=yb, ckpt=ck)
        binding.ss_ssd_bwd(db["x"], db["dt"], db["A"], db["B"], db["C"], db["D"], db["dt_bias"],
                           True, dout=db["dout"], workspace=wsb, ckpt=ck)
    step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        step()
    e1.record()
    torch.cuda.synchronize()
    sms = e0.elapsed_time(e1) / 5
    del db, wsb, ck, yb
    return {wb.name: {"call_ms": round(bms, 4), "elements_per_s": E / (bms * 1e-3),
                      "note": "chunked backward: states pass, reverse chunk kernel, dt, "
                              "head fold and parameter sums (one call)",
                      "fwd_bwd_step_with_ckpt_ms": round(sms, 4),
                      "fwd_bwd_step_elements_per_s": E / (sms * 1e-3)},
            w.name: {"kernel_ms": round(ms, 5), "elements_per_s": E / (ms * 1e-3),
                     "algorithmic_bytes": by,
                     "algorithmic_GBps": round(by / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac_of_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "chunk_form_TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2),
                     "bf16_dense_peak_TFLOPs": 2500.0,
                     "input_sets_rotated": 2}}


def conv_detail(hip, lib, to_dev, dev):
    """The causal convolution (width 4) in front of the scan: forward and
    backward at the Mamba-130m layer shape in bf16 and f32, and the decode
    step at 256 x 5120."""
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin
    detail = {}
    for cname, reps in (("mamba130m_conv_bf16_8x1536x2048", 4),
                        ("mamba130m_conv_f32_8x1536x2048", 2)):
        wc = ssin.CONV_WORKLOADS[cname]
        ac = ssin.make_conv(wc)
        es = 2 if wc.io == "bf16" else 4
        csets = [{k: to_dev(v) for k, v in ac.items()} for _ in range(reps)]
        couts = [torch.empty_like(c["x"]) for c in csets]
        fwd_calls = [lambda c=c, o=o: binding.ss_conv1d_fwd(c["x"], c["weight"], c["bias"],
                                                            True, out=o)
                     for c, o in zip(csets, couts)]
        bwd_calls = [lambda c=c: binding.ss_conv1d_bwd(c["x"], c["weight"], c["bias"], True,
                                                       None, c["dout"])
                     for c in csets]
        (fms,) = timed_calls(hip, lib, fwd_calls, 2, 20)
        (bms,) = timed_calls(hip, lib, bwd_calls, 2, 20)
        Ec = wc.elements
        fb = conv_algorithmic_bytes("conv_fwd", wc.batch, wc.dim, wc.seqlen, wc.width, es)
        bb = conv_algorithmic_bytes("conv_bwd", wc.batch, wc.dim, wc.seqlen, wc.width, es)
        detail[cname] = {
            "fwd_kernel_ms": round(fms, 5), "fwd_algorithmic_bytes": fb,
            "fwd_algorithmic_GBps": round(fb / (fms * 1e-3) / 1e9, 1),
            "fwd_hbm_frac_of_peak": round(fb / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_kernel_ms": round(bms, 5), "bwd_algorithmic_bytes": bb,
            "bwd_algorithmic_GBps": round(bb / (bms * 1e-3) / 1e9, 1),
            "bwd_hbm_frac_of_peak": round(bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_elements_per_s": Ec / (fms * 1e-3),
            "input_sets_rotated": reps}
        del csets, couts
    wcd = ssin.CONV_WORKLOADS["conv_decode_bf16_256x5120"]
    acd = ssin.make_conv(wcd)
    dsets = [{k: to_dev(v) for k, v in acd.items()} for _ in range(4)]
    douts = [torch.empty_like(c["x"]) for c in dsets]
    dec_calls = [lambda c=c, o=o: binding.ss_conv1d_update(c["state"], c["x"], c["weight"],
                                                           c["bias"], True, out=o)
                 for c, o in zip(dsets, douts)]
    (ums,) = timed_calls(hip, lib, dec_calls, 2, 40)
    ub = conv_algorithmic_bytes("conv_update", wcd.batch, wcd.dim, 1, wcd.width, 2)
    detail["conv_decode_bf16_256x5120"] = {
        "kernel_ms": round(ums, 5), "rows_per_s": wcd.batch * wcd.dim / (ums * 1e-3),
        "algorithmic_GBps": round(ub / (ums * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(ub / (ums * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "input_sets_rotated": 4}
    del dsets, douts
    return detail


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--conv-only", action="store_true",
                    help="time only the causal convolution kernels (prints their detail)")
    ap.add_argument("--ssd-only", action="store_true",
                    help="time only the Mamba-2 SSD kernel (prints its detail)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the selective scan's "
              "multi-GPU sharding is described in DESIGN.md but not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = "cuda:0"
    lib = binding.load()
    hip = hip_runtime()

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    if args.conv_only:
        print(json.dumps({"detail": conv_detail(hip, lib, to_dev, dev)}), flush=True)
        return
    if args.ssd_only:
        print(json.dumps({"detail": ssd_detail(hip, lib, to_dev, dev)}), flush=True)
        return

    # ---------------- the step: fwd + bwd at 8 x 1536 x 2048, f32 ----------------
    w = ssin.WORKLOADS["mamba130m_bwd_f32_8x1536x2048"]
    arr = ssin.make(w)
    d = {k: to_dev(v) for k, v in arr.items()}
    y = torch.empty_like(d["u"])
    ws = torch.empty(binding.ss_bwd_workspace_size(w.batch, w.dim, 16, w.seqlen, 0),
                     dtype=torch.uint8, device=dev)
    ck = binding.ss_ckpt_empty(d["u"])

    def step():
        # the forward saves its chunk checkpoints; the backward reuses them
        binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], True, out=y, ckpt=ck)
        return binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                              d["delta_bias"], True, d["dout"], workspace=ws, ckpt=ck)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # per step: fwd = [call start, after fwd kernel]; bwd = [call start, after reverse, after fold]
    per_step = 5
    timer = KernelTimer(hip, lib, per_step * args.steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    timer.arm()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    used = timer.disarm()
    assert used == per_step * args.steps, f"recorded {used} events"
    ms_step = t_start.elapsed_time(t_end) / args.steps
    names = ["ss_fwd_kernel", "ss_bwd_reverse_kernel", "ss_bwd_fold_kernel"]
    pairs = [(0, 1), (2, 3), (3, 4)]
    kern_ms = {n: float(np.mean([timer.ms(s * per_step + i, s * per_step + j)
                                 for s in range(args.steps)])) for n, (i, j) in zip(names, pairs)}
    timer.close()
    E = w.batch * w.dim * w.seqlen
    kb = {n: algorithmic_bytes(n, w.batch, w.dim, w.seqlen, 4) for n in names}
    step_bytes = kb["ss_fwd_kernel"] + kb["ss_bwd_reverse_kernel"] + kb["ss_bwd_fold_kernel"]
    dom = max(names, key=lambda n: kern_ms[n])
    ach = kb[dom] / (kern_ms[dom] * 1e-3) / 1e9
    tflops = FLOPS_PER_ELEMENT[dom] * E / (kern_ms[dom] * 1e-3) / 1e12
    traffic = measured_traffic(dom, "mamba130m_f32_8x1536x2048")
    kernels = {n: {"avg_ms": round(kern_ms[n], 5), "algorithmic_bytes": kb[n],
                   "algorithmic_GBps": round(kb[n] / (kern_ms[n] * 1e-3) / 1e9, 1)}
               for n in names}

    result = {
        "metric": METRIC,
        "value": E / (ms_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mamba130m-layer scan fwd+bwd, f32 io", "batch": w.batch,
                   "d_inner": w.dim, "d_state": 16, "seqlen": w.seqlen, "io_dtype": "f32",
                   "z_gate": True, "D_skip": True, "delta_bias_softplus": True},
        "hbm_GBps_algorithmic": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        # The scan kernels are limited by f32 VALU work (an exp and ~20 other
        # VALU ops per element and state in the reverse pass) and on-chip
        # latency, not by HBM: the roofline is the ALU one; the HBM view of
        # the same kernel follows beside it.
        "roofline": {"kernel": dom, "bound": "alu", "achieved": round(tflops, 2),
                     "peak": round(ALU_PEAK_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / ALU_PEAK_TFLOPS, 4), "traffic": traffic,
                     "flops_per_element": FLOPS_PER_ELEMENT[dom],
                     "hbm_algorithmic_GBps": round(ach, 1), "hbm_peak_GBps": HBM_PEAK_GBS,
                     "hbm_frac": round(ach / HBM_PEAK_GBS, 4),
                     "hbm_measured_GBps": (round(traffic / (kern_ms[dom] * 1e-3) / 1e9, 1)
                                           if traffic else None)},
        "kernels": kernels,
    }

    # ---------------- detail: forward-only and decode workloads ----------------
    if not args.no_detail:
        detail = {}
        for name, reps in (("mamba130m_fwd_bf16_8x1536x2048", 2), ("mamba2p8b_fwd_bf16_4x5120x4096", 1)):
            wf = ssin.WORKLOADS[name]
            af = ssin.make(wf)
            sets = [{k: to_dev(v) for k, v in af.items()} for _ in range(reps)]
            outs = [torch.empty_like(s["u"]) for s in sets]
            last = torch.empty(wf.batch, wf.dim, 16, device=dev) if wf.last_state else None
            del af

            def run(i):
                s = sets[i % reps]
                binding.ss_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"],
                               s["delta_bias"], True, out=outs[i % reps], last_state=last)
            for i in range(3):
                run(i)
            iters = 20
            tm = KernelTimer(hip, lib, 2 * iters)
            torch.cuda.synchronize()
            tm.arm()
            for i in range(iters):
                run(i)
            torch.cuda.synchronize()
            tm.disarm()
            ms = float(np.mean([tm.ms(2 * i, 2 * i + 1) for i in range(iters)]))
            tm.close()
            Ef = wf.batch * wf.dim * wf.seqlen
            by = algorithmic_bytes("ss_fwd_kernel", wf.batch, wf.dim, wf.seqlen, 2)
            if wf.last_state:
                by += wf.batch * wf.dim * 16 * 4
            detail[name] = {"kernel_ms": round(ms, 5), "elements_per_s": Ef / (ms * 1e-3),
                            "algorithmic_GBps": round(by / (ms * 1e-3) / 1e9, 1),
                            "hbm_frac_of_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "input_sets_rotated": reps}
            del sets, outs
        # the same fwd + bwd step with bf16 tensors
        wb = ssin.WORKLOADS["mamba130m_bwd_bf16_8x1536x2048"]
        db = {k: to_dev(v) for k, v in ssin.make(wb).items()}
        yb = torch.empty_like(db["u"])
        ckb = binding.ss_ckpt_empty(db["u"])
        wsb = torch.empty(binding.ss_bwd_workspace_size(wb.batch, wb.dim, 16, wb.seqlen, 1),
                          dtype=torch.uint8, device=dev)

        def step_bf16():
            binding.ss_fwd(db["u"], db["delta"], db["A"], db["B"], db["C"], db["D"], db["z"],
                           db["delta_bias"], True, out=yb, ckpt=ckb)
            binding.ss_bwd(db["u"], db["delta"], db["A"], db["B"], db["C"], db["D"], db["z"],
                           db["delta_bias"], True, db["dout"], workspace=wsb, ckpt=ckb)
        for _ in range(3):
            step_bf16()
        iters = 10
        tm = KernelTimer(hip, lib, per_step * iters)
        torch.cuda.synchronize()
        tm.arm()
        for _ in range(iters):
            step_bf16()
        torch.cuda.synchronize()
        tm.disarm()
        kb16 = {n: float(np.mean([tm.ms(s * per_step + i, s * per_step + j) for s in range(iters)]))
                for n, (i, j) in zip(names, pairs)}
        tm.close()
        detail["mamba130m_step_bf16_8x1536x2048"] = {
            **{n.replace("ss_", "").replace("_kernel", "") + "_ms": round(v, 5) for n, v in kb16.items()},
            "step_kernels_ms": round(sum(kb16.values()), 5),
            "elements_per_s": E / (sum(kb16.values()) * 1e-3)}
        del db, yb, ckb, wsb

        # the backward on its own (checkpoints recomputed inside ss_bwd)
        iters = 10
        tm = KernelTimer(hip, lib, 4 * iters)
        torch.cuda.synchronize()
        tm.arm()
        for _ in range(iters):
            binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                           d["delta_bias"], True, d["dout"], workspace=ws)
        torch.cuda.synchronize()
        tm.disarm()
        parts = [float(np.mean([tm.ms(4 * i + a, 4 * i + a + 1) for i in range(iters)]))
                 for a in range(3)]
        tm.close()
        detail["mamba130m_bwd_f32_8x1536x2048_standalone"] = {
            "ckpt_kernel_ms": round(parts[0], 5), "reverse_kernel_ms": round(parts[1], 5),
            "fold_kernel_ms": round(parts[2], 5), "total_ms": round(sum(parts), 5),
            "elements_per_s": E / (sum(parts) * 1e-3)}
        wd = ssin.WORKLOADS["decode_bf16_256x5120"]
        ad = ssin.make(wd)
        reps = 4
        sets = [{k: to_dev(v) for k, v in ad.items()} for _ in range(reps)]
        outs = [torch.empty_like(s["u"]) for s in sets]

        def dec(i):
            s = sets[i % reps]
            binding.ss_state_update(s["state"], s["u"], s["delta"], s["A"], s["B"], s["C"],
                                    s["D"], s["z"], s["delta_bias"], True, out=outs[i % reps])
        for i in range(4):
            dec(i)
        iters = 40
        tm = KernelTimer(hip, lib, 2 * iters)
        torch.cuda.synchronize()
        tm.arm()
        for i in range(iters):
            dec(i)
        torch.cuda.synchronize()
        tm.disarm()
        ms = float(np.mean([tm.ms(2 * i, 2 * i + 1) for i in range(iters)]))
        tm.close()
        by = algorithmic_bytes("ss_state_update_kernel", wd.batch, wd.dim, 1, 2)
        detail["decode_bf16_256x5120"] = {
            "kernel_ms": round(ms, 5), "rows_per_s": wd.batch * wd.dim / (ms * 1e-3),
            "algorithmic_GBps": round(by / (ms * 1e-3) / 1e9, 1),
            "hbm_frac_of_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "input_sets_rotated": reps}
        del sets, outs

        detail.update(wide_state_detail(hip, lib, to_dev, dev))
        detail.update(conv_detail(hip, lib, to_dev, dev))
        detail.update(ssd_detail(hip, lib, to_dev, dev))
        result["detail"] = detail

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    if not args.no_cpu_baseline:
        from oracle import oracle
        threads = min(8, os.cpu_count() or 1)
        nd = 1536  # the whole workload: 8 x 1536 x 2048 elements, about 10 s of host work
        x = {k: (v[:, :nd] if k in ("u", "delta", "z", "dout") else v).astype(np.float64)
             for k, v in arr.items()}
        x["A"], x["D"], x["delta_bias"] = (arr["A"][:nd].astype(np.float64),
                                           arr["D"][:nd].astype(np.float64),
                                           arr["delta_bias"][:nd].astype(np.float64))
        t0 = time.perf_counter()
        oracle.fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                   True, threads=threads)
        oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                   True, x["dout"], threads=threads)
        dt = time.perf_counter() - t0
        Es = w.batch * nd * w.seqlen
        result["cpu_baseline"] = {"value": Es / dt, "unit": "elements/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"fwd+bwd (f64 oracle, incl. the dB/dC sums over "
                                            f"channels) of the whole workload, {w.batch} x {nd} x "
                                            f"{w.seqlen} = {Es} elements, {threads} threads, "
                                            f"{dt:.2f} s wall"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
