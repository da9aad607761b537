"""Batched-concurrent int4 (W4A16, group-wise) MoE decode step on MI355X.

The product is ``libw4moe.so`` (hand-written HIP for gfx950 behind the C ABI
of ``include/w4moe.h``); ``_lib`` binds it with ctypes under the same names,
``engine`` does device-memory plumbing with torch, ``inputs`` draws seeded
synthetic workloads.  Importing this package loads nothing; the library is
opened on first use and raises if it has not been built.
"""
