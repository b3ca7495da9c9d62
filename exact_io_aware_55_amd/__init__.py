"""Exact (FlashAttention) attention forward and backward for AMD gfx950.

The compute runs in hand-written HIP kernels inside ``libfa.so`` behind a C
ABI (``include/fa.h``); :mod:`exact_io_aware_55_amd.binding` marshals torch
tensors into that ABI.  The library is loaded lazily, on first use.
"""

__all__ = ["forward", "backward", "forward_f32"]


def __getattr__(name):
    if name in ("forward", "backward", "forward_f32", "bwd_workspace_size"):
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
