"""MACaQ online W4A4 linear layer for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmacaq.so`` (hand-written HIP,
declared in ``include/macaq.h``); ``binding`` marshals torch tensors into it.
``inputs`` holds the seeded synthetic workloads. Submodules are imported on
use so that the input generators load without the HIP library.
"""
