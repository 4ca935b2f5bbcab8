"""Ulysses 4D all-to-all relayout for AMD Instinct MI355X (gfx950).

The compute path is libulysses.so (hand-written HIP kernels behind a C ABI,
include/ulysses.h); `ulysses` is its thin ctypes binding and `workloads`
draws seeded synthetic inputs.
"""
