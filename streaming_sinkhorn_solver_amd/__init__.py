"""Streaming log-domain Sinkhorn for entropic optimal transport on AMD MI355X.

The solver itself is the HIP library ``libfs_sinkhorn.so`` (C ABI in
``include/fs_sinkhorn.h``); ``binding`` is its ctypes binding and
``workloads`` draws the seeded synthetic inputs.  Import ``binding``
explicitly: importing this package does not load the library.
"""
__all__ = ["binding", "workloads", "build"]
