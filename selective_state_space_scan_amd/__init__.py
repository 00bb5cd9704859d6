"""Selective state-space scan (Mamba S6) for AMD Instinct MI355X (gfx950).

The compute lives in ``libss.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/ss.h``).  ``binding`` marshals PyTorch tensors into
that ABI; ``inputs`` draws the seeded synthetic workloads.
"""
