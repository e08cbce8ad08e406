"""Fused, chunked linear-cross-entropy for AMD Instinct MI355X (gfx950).

The compute lives in liblce.so (HIP kernels behind the C ABI of include/lce.h);
``_lib`` is its ctypes binding and ``functional.linear_cross_entropy`` the
autograd entry point.  Importing the package loads nothing; the library is
loaded on first use and its absence is an error.
"""

__all__ = ["linear_cross_entropy"]


def linear_cross_entropy(*args, **kwargs):
    from .functional import linear_cross_entropy as _f
    return _f(*args, **kwargs)
