"""MI355X-native Mixture-of-Experts layer (forward + backward) behind the libmoe C ABI.

`_lib` is the ctypes binding of include/moe.h; `workloads` draws the seeded synthetic
inputs.  All layer arithmetic runs in the HIP kernels of libmoe.so.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "lib"]


def __getattr__(name):
    if name == "lib":
        from . import _lib
        return _lib
    raise AttributeError(name)
