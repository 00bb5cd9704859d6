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


# The sources each profiled kernel is built from: a committed summary counts
# only while their hash is the one it was measured with.
_FWD_SRC = ["ss_fwd.hip", "ss_conv_lane.h", "ss_tiles.h", "ss_device.h", "ss_kernels.h"]
_BWD_SRC = ["ss_bwd.hip", "ss_conv_lane.h", "ss_tiles.h", "ss_device.h", "ss_kernels.h"]
KERNEL_SOURCES = {
    "ss_fwd_kernel": _FWD_SRC,
    "ss_fwd_summary_kernel": _FWD_SRC,
    "ss_bwd_reverse_kernel": _BWD_SRC,
    "ss_bwd_fold_kernel": _BWD_SRC,
    "ss_bwd_ckpt_kernel": _BWD_SRC,
    "ss_bwd_adjoint_summary_kernel": _BWD_SRC,
    "ss_state_update_kernel": ["ss_state_update.hip", "ss_device.h", "ss_kernels.h"],
}


# rocprofv3 counter passes behind a committed summary: five runs of
# `rocprofv3 --pmc <pass> -- python3 bench.py --only <workload> --steps 3
# --warmup 1`, then one `--kernel-trace --stats` run with --steps 20.
PMC_PASSES = [
    "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR "
    "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_SMEM GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY "
    "SQ_WAIT_ANY SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU2 GRBM_GUI_ACTIVE",
    "SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_THREAD_CYCLES_VALU SQ_INSTS_BRANCH SQ_CYCLES "
    "SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_MISC GRBM_GUI_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
]
# Issue cost of one wave64 f32 VALU instruction in SIMD cycles, measured on
# this chip with independent FMA chains at 4-8 waves per SIMD (4.1-4.4;
# v_exp_f32 alone 8.3, but it overlaps the next plain op).  The VALU issue
# floor of a kernel is its VALU instruction count times this cost, spread
# over 1024 SIMDs at the 2.4 GHz peak clock.
VALU_ISSUE_CYCLES = 4.1
SIMDS = 1024
CLOCK_HZ = 2.4e9


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def summarize_profile(prof_dir, copy_dir, kernel, workload, title, only, sources):
    """Markdown summary of the counter passes and the kernel trace of one
    kernel (a substring of its name) in `prof_dir` (p1 .. p5 and trace, as
    written by the commands the summary quotes); `copy_dir` holds the same
    FETCH_SIZE / WRITE_SIZE passes over the 1 GiB device copy that calibrates
    them."""
    import glob
    import hashlib
    vals = {}
    meta = None
    for i in range(1, len(PMC_PASSES) + 1):
        for f in glob.glob(os.path.join(prof_dir, f"p{i}", "**", "*counter_collection.csv"),
                           recursive=True):
            for r in _read_csv(f):
                if kernel not in r["Kernel_Name"]:
                    continue
                meta = meta or r
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    cp = {}
    for i in (4, 5):
        for f in glob.glob(os.path.join(copy_dir, f"p{i}", "**", "*counter_collection.csv"),
                           recursive=True):
            for r in _read_csv(f):
                if "copyBuffer" in r["Kernel_Name"]:
                    cp.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    gib_kib = float(1 << 20)
    fs = gib_kib / max(cp["FETCH_SIZE"]) if cp.get("FETCH_SIZE") else None
    ws = gib_kib / max(cp["WRITE_SIZE"]) if cp.get("WRITE_SIZE") else None
    stats = []
    for f in glob.glob(os.path.join(prof_dir, "trace", "**", "*kernel_stats.csv"), recursive=True):
        stats += _read_csv(f)
    row = next(r for r in stats if kernel in r["Name"])
    ns = float(row["AverageNs"])
    waves = avg.get("SQ_WAVES", 0.0)
    gui = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8.0   # summed over the 8 XCDs
    out = [f"# {kernel} -- {title}", "",
           "Measured on one MI355X (gfx950) with rocprofv3; the raw profiler outputs are not committed.", "",
           "## Commands", "",
           "Counters, one run per pass (each pass fits the per-block counter limits):", ""]
    for p in PMC_PASSES:
        out.append(f"- `timeout -s KILL 120 rocprofv3 --pmc {p} -d <dir>/pN -o pN --output-format "
                   f"csv -- python3 bench.py --only {only} --steps 3 --warmup 1`")
    out += ["", f"Trace: `timeout -s KILL 120 rocprofv3 --kernel-trace --stats -d <dir>/trace -o "
                f"trace --output-format csv -- python3 bench.py --only {only} --steps 20 --warmup 3`",
            "", "Traffic calibration: the FETCH_SIZE and WRITE_SIZE passes above with "
                "`--only copy_1GiB` (a 1 GiB device copy).", "",
            "Summary: `python3 bench.py --summarize <dir> --copy-dir <copy dir> "
            f"--kernel {kernel} --only {only}`", "",
            "## Launch", "",
            f"grid {meta['Grid_Size']} work-items, workgroup {meta['Workgroup_Size']}, "
            f"LDS {meta['LDS_Block_Size']} B, VGPRs {meta['VGPR_Count']}, "
            f"SGPRs {meta['SGPR_Count']}, scratch {meta['Scratch_Size']} B", "",
            "## Trace", "",
            f"average {ns:.0f} ns over {row['Calls']} calls (min {row['MinNs']}, max {row['MaxNs']})",
            "", "## Counters (per launch)", "", "| counter | value | per wave |", "|---|---|---|"]
    for k in sorted(avg):
        pw = f"{avg[k] / waves:.1f}" if waves and k.startswith("SQ_INSTS") else ""
        out.append(f"| {k} | {avg[k]:.6g} | {pw} |")
    valu = avg.get("SQ_INSTS_VALU", 0.0)
    floor_ns = valu * VALU_ISSUE_CYCLES / SIMDS / CLOCK_HZ * 1e9
    traffic = None
    if fs and ws and "FETCH_SIZE" in avg and "WRITE_SIZE" in avg:
        traffic = int(avg["FETCH_SIZE"] * 1024 * fs + avg["WRITE_SIZE"] * 1024 * ws)
    out += ["", "## Derived", "", "| quantity | value |", "|---|---|",
            f"| kernel clock-cycles per XCD (GRBM_GUI_ACTIVE / 8) | {gui:.0f} |"]
    if gui and "SQ_ACTIVE_INST_VALU" in avg:
        out.append(f"| VALU busy (4 x SQ_ACTIVE_INST_VALU / (1024 SIMDs x cycles)) | "
                   f"{100 * 4 * avg['SQ_ACTIVE_INST_VALU'] / SIMDS / gui:.1f}% |")
    if gui and "SQ_ACTIVE_INST_LDS" in avg:
        out.append(f"| LDS instruction activity per CU (4 x SQ_ACTIVE_INST_LDS / (256 x cycles)) | "
                   f"{100 * 4 * avg['SQ_ACTIVE_INST_LDS'] / 256 / gui:.1f}% |")
    out.append(f"| VALU instructions per launch | {valu:.0f} |")
    out.append(f"| VALU issue floor ({VALU_ISSUE_CYCLES} cycles per wave64 op, {SIMDS} SIMDs, "
               f"{CLOCK_HZ / 1e9} GHz) | {floor_ns:.0f} ns = {100 * floor_ns / ns:.1f}% of the "
               f"trace time |")
    if traffic:
        out += [f"| FETCH scale (1 GiB copy) | {fs:.3f} |", f"| WRITE scale (1 GiB copy) | {ws:.3f} |",
                f"| HBM bytes per launch (scaled) | {traffic} |",
                f"| measured HBM rate | {traffic / ns:.1f} GB/s |"]
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "selective_state_space_scan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    out += ["", "## Values read by bench.py", ""]
    if traffic:
        out.append(f"traffic_bytes_per_launch: {traffic}")
    out += [f"valu_insts_per_launch: {valu:.0f}", f"trace_avg_ns: {ns:.0f}",
            f"sources_sha256_16: {h.hexdigest()[:16]}",
            "sources: " + " ".join("selective_state_space_scan_amd/csrc/" + f for f in sources)]
    return "\n".join(out) + "\n"


def profile_path(kernel, only):
    """Committed summary of `kernel` under the `--only` workload `only`."""
    return os.path.join(ROOT, "profiles", f"{kernel}__{only}.md")


def profile_value(kernel, only, key):
    """A value from the committed rocprofv3 summary of `kernel` under the
    `--only` workload `only`, or None when the summary is missing or the
    kernel's sources changed."""
    import hashlib
    path = profile_path(kernel, only)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`", "-")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "selective_state_space_scan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("sources_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def copy_ceiling_gbps(dev, iters=10):
    """Device-to-device copy rate of a 1 GiB buffer (read + write bytes per
    second): the ceiling a streaming kernel can reach on this machine."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del src, dst
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


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
    16-state slices: the forward runs them in each lane, the backward one
    launch per slice, each adding its du and ddelta to the sum so far), f32
    io."""
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
    # per step: fwd [start, scan]; bwd [start, reverse slices, fold]
    parts = timed_calls(hip, lib, [step], 5, 5)
    names = ["fwd_ms", None, "bwd_reverse_slices_ms", "bwd_fold_ms"]
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


def conv_scan_detail(hip, lib, to_dev, dev):
    """The convolution fused into the scan's load stage (ss_fwd_conv) at the
    c1 bf16 forward shape with a width-4 SiLU convolution, against the two
    separate calls it replaces (ss_conv1d_fwd, then ss_fwd on its output).
    Inputs rotated over two sets; HIP events around each kernel."""
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin
    w = ssin.WORKLOADS["mamba130m_fwd_bf16_8x1536x2048"]
    a = ssin.make(w)
    ac = ssin.make_conv(ssin.CONV_WORKLOADS["mamba130m_conv_bf16_8x1536x2048"])
    sets = [{k: to_dev(v) for k, v in a.items()} for _ in range(2)]
    cw, cb = to_dev(ac["weight"]), to_dev(ac["bias"])
    del a, ac
    outs = [torch.empty_like(c["u"]) for c in sets]
    us = [torch.empty_like(c["u"]) for c in sets]
    fused = [lambda c=c, o=o: binding.ss_fwd_conv(c["u"], cw, c["delta"], c["A"], c["B"], c["C"],
                                                  c["D"], c["z"], c["delta_bias"], True,
                                                  conv_bias=cb, out=o)
             for c, o in zip(sets, outs)]

    def sep(c, o, u):
        binding.ss_conv1d_fwd(c["u"], cw, cb, True, out=u)
        binding.ss_fwd(u, c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"], c["delta_bias"],
                       True, out=o)
    separate = [lambda c=c, o=o, u=u: sep(c, o, u) for c, o, u in zip(sets, outs, us)]
    (fms,) = timed_calls(hip, lib, fused, 2, 20)
    conv_ms, _, scan_ms = timed_calls(hip, lib, separate, 4, 20)
    out = {"mamba130m_fwd_conv_bf16_8x1536x2048": {
        "fused_kernel_ms": round(fms, 5), "separate_conv_ms": round(conv_ms, 5),
        "separate_scan_ms": round(scan_ms, 5),
        "separate_total_ms": round(conv_ms + scan_ms, 5),
        "elements_per_s": w.batch * w.dim * w.seqlen / (fms * 1e-3)}}
    # a training step of the convolution + scan: fused (ss_fwd_conv saving
    # its record, ss_bwd_conv) against the separate calls (ss_conv1d_fwd,
    # ss_fwd saving its record, ss_bwd, ss_conv1d_bwd on its du)
    wb = ssin.WORKLOADS["mamba130m_bwd_bf16_8x1536x2048"]
    c = {k: to_dev(v) for k, v in ssin.make(wb).items()}
    ck = binding.ss_ckpt_empty(c["u"])
    ws = torch.empty(binding.ss_bwd_workspace_size(wb.batch, wb.dim, 16, wb.seqlen, 1),
                     dtype=torch.uint8, device=dev)
    y, u = torch.empty_like(c["u"]), torch.empty_like(c["u"])

    def fused_step():
        binding.ss_fwd_conv(c["u"], cw, c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"],
                            c["delta_bias"], True, conv_bias=cb, out=y, ckpt=ck)
        binding.ss_bwd_conv(c["u"], cw, c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"],
                            c["delta_bias"], True, c["dout"], conv_bias=cb, workspace=ws, ckpt=ck)

    def separate_step():
        binding.ss_conv1d_fwd(c["u"], cw, cb, True, out=u)
        binding.ss_fwd(u, c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"], c["delta_bias"],
                       True, out=y, ckpt=ck)
        g = binding.ss_bwd(u, c["delta"], c["A"], c["B"], c["C"], c["D"], c["z"],
                           c["delta_bias"], True, c["dout"], workspace=ws, ckpt=ck)
        binding.ss_conv1d_bwd(c["u"], cw, cb, True, None, g["du"])
    res = {}
    for name, fn in (("fused_step_ms", fused_step), ("separate_step_ms", separate_step)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / 10, 5)
    res["elements_per_s"] = wb.batch * wb.dim * wb.seqlen / (res["fused_step_ms"] * 1e-3)
    out["mamba130m_step_conv_bf16_8x1536x2048"] = res
    del sets, outs, us, c, ck, ws, y, u
    return out


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


def _scan_call(name, to_dev, dev):
    """One library call pattern of a named scan workload, with its inputs
    resident on the GPU."""
    import torch

    from selective_state_space_scan_amd import binding
    from selective_state_space_scan_amd import inputs as ssin
    if name == "copy_1GiB":
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        return lambda: dst.copy_(src), (src, dst)
    wname = PROFILE_WORKLOADS[name]
    w = ssin.WORKLOADS[wname]
    d = {k: to_dev(v) for k, v in ssin.make(w).items()}
    io = 1 if w.io == "bf16" else 0
    if w.kind == "decode":
        out = torch.empty_like(d["u"])
        return (lambda: binding.ss_state_update(d["state"], d["u"], d["delta"], d["A"], d["B"],
                                                d["C"], d["D"], d["z"], d["delta_bias"], True,
                                                out=out)), (d, out)
    y = torch.empty_like(d["u"])
    last = (torch.empty(w.batch, w.dim, w.dstate, device=dev) if w.last_state else None)
    if name.startswith("fwdconv"):   # the convolution fused in front of the scan
        ac = ssin.make_conv(ssin.CONV_WORKLOADS["mamba130m_conv_bf16_8x1536x2048"])
        cw, cb = to_dev(ac["weight"]), to_dev(ac["bias"])
        return (lambda: binding.ss_fwd_conv(d["u"], cw, d["delta"], d["A"], d["B"], d["C"],
                                            d["D"], d["z"], d["delta_bias"], True,
                                            conv_bias=cb, out=y)), (d, y, cw, cb)
    if name.startswith("stepconv"):   # fused convolution + scan, forward saving its record and backward
        ac = ssin.make_conv(ssin.CONV_WORKLOADS["mamba130m_conv_bf16_8x1536x2048"])
        cw, cb = to_dev(ac["weight"]), to_dev(ac["bias"])
        ck = binding.ss_ckpt_empty(d["u"], dstate=w.dstate)
        ws = torch.empty(binding.ss_bwd_workspace_size(w.batch, w.dim, w.dstate, w.seqlen, io),
                         dtype=torch.uint8, device=dev)

        def cstep():
            binding.ss_fwd_conv(d["u"], cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                d["delta_bias"], True, conv_bias=cb, out=y, ckpt=ck)
            binding.ss_bwd_conv(d["u"], cw, d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                d["delta_bias"], True, d["dout"], conv_bias=cb, workspace=ws,
                                ckpt=ck)
        return cstep, (d, y, cw, cb, ck, ws)
    if w.kind == "fwd" or name.startswith("fwd"):
        return (lambda: binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       d["delta_bias"], True, out=y, last_state=last)), (d, y, last)
    ws = torch.empty(binding.ss_bwd_workspace_size(w.batch, w.dim, w.dstate, w.seqlen, io),
                     dtype=torch.uint8, device=dev)
    if name.endswith("standalone"):
        return (lambda: binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                       d["delta_bias"], True, d["dout"], workspace=ws)), (d, ws)
    ck = binding.ss_ckpt_empty(d["u"], dstate=w.dstate)

    def step():
        binding.ss_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], True, out=y, ckpt=ck)
        binding.ss_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"],
                       d["delta_bias"], True, d["dout"], workspace=ws, ckpt=ck)
    return step, (d, y, ws, ck)


# --only NAME: the workloads a profiler run can select (scan workload name, or
# the 1 GiB device copy that calibrates the traffic counters)
PROFILE_WORKLOADS = {
    "step_f32_8x1536x2048": "mamba130m_bwd_f32_8x1536x2048",
    "step_bf16_8x1536x2048": "mamba130m_bwd_bf16_8x1536x2048",
    "bwd_f32_8x1536x2048_standalone": "mamba130m_bwd_f32_8x1536x2048",
    "fwd_bf16_8x1536x2048": "mamba130m_fwd_bf16_8x1536x2048",
    "fwdconv_bf16_8x1536x2048": "mamba130m_fwd_bf16_8x1536x2048",
    "stepconv_bf16_8x1536x2048": "mamba130m_bwd_bf16_8x1536x2048",
    "fwd_bf16_4x5120x4096": "mamba2p8b_fwd_bf16_4x5120x4096",
    "decode_bf16_256x5120": "decode_bf16_256x5120",
    "fwd_bf16_1x1536x16384": "mamba130m_long_bf16_1x1536x16384",
    "step_bf16_1x1536x16384": "mamba130m_long_bf16_1x1536x16384",
    "bwd_bf16_1x1536x16384_standalone": "mamba130m_long_bf16_1x1536x16384",
    "fwd_bf16_1x1536x2048": "mamba130m_prefill_bf16_1x1536x2048",
    "step_bf16_1x1536x2048": "mamba130m_prefill_bf16_1x1536x2048",
    "copy_1GiB": None,
}


def prefill_regime_detail(to_dev, dev):
    """One short bf16 sequence (1 x 1536 x 2048), in the automatic regime
    (sequential at this length) and in the segmented one (ss_set_scan_regime).
    Mean call times over several calls, HIP events around each call."""
    from selective_state_space_scan_amd import binding
    out = {}
    for regime, tag in ((binding.SS_SCAN_AUTO, "auto"), (binding.SS_SCAN_SEGMENTED, "segmented")):
        binding.set_scan_regime(regime)
        try:
            for only, key in (("fwd_bf16_1x1536x2048", "fwd_ms"),
                              ("step_bf16_1x1536x2048", "step_ms")):
                out[f"{tag}_{key}"] = round(run_only(only, 20, 3, to_dev, dev)["ms_per_call"], 5)
        finally:
            binding.set_scan_regime(binding.SS_SCAN_AUTO)
    E = 1 * 1536 * 2048
    out["segmented_step_elements_per_s"] = E / (out["segmented_step_ms"] * 1e-3)
    out["speedup_fwd"] = round(out["auto_fwd_ms"] / out["segmented_fwd_ms"], 2)
    out["speedup_step"] = round(out["auto_step_ms"] / out["segmented_step_ms"], 2)
    return {"mamba130m_prefill_bf16_1x1536x2048": out}


def long_sequence_detail(to_dev, dev):
    """One long bf16 sequence (1 x 1536 x 16384): few (row, state) lanes, so
    the scan runs as time segments.  Mean call times over several calls,
    HIP events around each kind of call (each is several kernels)."""
    out = {}
    for only, key in (("fwd_bf16_1x1536x16384", "fwd_ms"),
                      ("bwd_bf16_1x1536x16384_standalone", "bwd_standalone_ms"),
                      ("step_bf16_1x1536x16384", "step_ms")):
        out[key] = round(run_only(only, 20, 3, to_dev, dev)["ms_per_call"], 5)
    E = 1 * 1536 * 16384
    out["step_elements_per_s"] = E / (out["step_ms"] * 1e-3)
    return {"mamba130m_long_bf16_1x1536x16384": out}


def run_only(name, steps, warmup, to_dev, dev):
    import torch
    call, keep = _scan_call(name, to_dev, dev)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    del keep
    return {"only": name, "steps": steps, "ms_per_call": e0.elapsed_time(e1) / max(steps, 1)}


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
    ap.add_argument("--summarize", metavar="DIR",
                    help="print the markdown summary of the rocprofv3 passes in DIR for --kernel "
                         "(with --only naming the workload and --copy-dir the calibration)")
    ap.add_argument("--copy-dir", metavar="DIR")
    ap.add_argument("--kernel")
    ap.add_argument("--only", choices=sorted(PROFILE_WORKLOADS),
                    help="run one workload --steps times after --warmup (for rocprofv3 "
                         "traces and counters) and print its mean call time")
    args = ap.parse_args()
    if args.summarize:
        w = PROFILE_WORKLOADS[args.only]
        key = args.kernel if args.kernel in KERNEL_SOURCES else None
        srcs = KERNEL_SOURCES.get(key, []) if key else []
        print(summarize_profile(args.summarize, args.copy_dir, args.kernel, w,
                                f"{args.only} ({w})", args.only, srcs), end="")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); sharding the selective "
              "scan across GPUs is not built.", file=sys.stderr)
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
    if args.only:
        print(json.dumps(run_only(args.only, args.steps, args.warmup, to_dev, dev)), flush=True)
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
    traffic = profile_value(dom, "step_f32_8x1536x2048", "traffic_bytes_per_launch")
    valu = profile_value(dom, "step_f32_8x1536x2048", "valu_insts_per_launch")
    copy_gbps = copy_ceiling_gbps(dev)
    kernels = {n: {"avg_ms": round(kern_ms[n], 5), "algorithmic_bytes": kb[n],
                   "algorithmic_GBps": round(kb[n] / (kern_ms[n] * 1e-3) / 1e9, 1),
                   "hbm_frac": round(kb[n] / (kern_ms[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
               for n in names}
    issue = None
    if valu:
        floor_ms = valu * VALU_ISSUE_CYCLES / SIMDS / CLOCK_HZ * 1e3
        issue = {"valu_insts_per_launch": int(valu), "cycles_per_valu_inst": VALU_ISSUE_CYCLES,
                 "simds": SIMDS, "clock_GHz": CLOCK_HZ / 1e9,
                 "floor_ms": round(floor_ms, 5), "frac": round(floor_ms / kern_ms[dom], 4)}

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
        # The dominant kernel against the HBM roofline (algorithmic bytes per
        # launch / its average duration, HIP events on its stream), with the
        # measured copy ceiling beside it, and its VALU issue floor (the
        # committed counter summary's VALU instruction count at the measured
        # issue cost) -- the scan kernels are bound by instruction issue.
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": int(traffic) if traffic else None,
                     "algorithmic_bytes": kb[dom], "avg_ms": round(kern_ms[dom], 5),
                     "copy_ceiling_GBps": round(copy_gbps, 1),
                     "frac_of_copy_ceiling": round(ach / copy_gbps, 4),
                     "measured_GBps": (round(traffic / (kern_ms[dom] * 1e-3) / 1e9, 1)
                                       if traffic else None),
                     "valu_issue": issue},
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

        detail.update(long_sequence_detail(to_dev, dev))
        detail.update(prefill_regime_detail(to_dev, dev))
        detail.update(wide_state_detail(hip, lib, to_dev, dev))
        detail.update(conv_detail(hip, lib, to_dev, dev))
        detail.update(conv_scan_detail(hip, lib, to_dev, dev))
        detail.update(ssd_detail(hip, lib, to_dev, dev))
        result["detail"] = detail

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    if not args.no_cpu_baseline:
        from oracle import oracle
        nproc = os.cpu_count() or 1
        threads = max(1, min(16, nproc))   # the host-core share of one GPU

        def oracle_step(nb, nthreads):
            x = {k: (v[:nb] if k in ("u", "delta", "z", "dout", "B", "C") else v).astype(np.float64)
                 for k, v in arr.items()}
            t0 = time.perf_counter()
            oracle.fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                       x["delta_bias"], True, threads=nthreads)
            oracle.bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"],
                       x["delta_bias"], True, x["dout"], threads=nthreads)
            return nb * w.dim * w.seqlen / (time.perf_counter() - t0)
        one = oracle_step(1, 1)                  # one batch entry, one thread
        allc = oracle_step(w.batch, threads)     # the whole workload, all threads
        result["cpu_baseline"] = {
            "value": allc, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "nproc": nproc, "cpu_model": cpu_model(),
            "single_thread_elements_per_s": one, "all_core_elements_per_s": allc,
            "sample": f"f64 oracle fwd+bwd (incl. the dB/dC sums over channels): one batch "
                      f"entry ({w.dim} x {w.seqlen}) on 1 thread, then the whole workload "
                      f"({w.batch} x {w.dim} x {w.seqlen}) on {threads} threads"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
