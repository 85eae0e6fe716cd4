"""MI355X (gfx950) broadcasting binary operators with autograd backward.

The computation lives in ``libzk.so`` (C ABI: include/zk.h, HIP kernels in
``csrc/``); ``zk`` is its ctypes binding and ``workloads`` draws the seeded
synthetic inputs.  Importing the package loads nothing; the first call into
``zk`` loads the library and raises if it is missing.
"""
from . import zk  # noqa: F401

__all__ = ["zk"]
