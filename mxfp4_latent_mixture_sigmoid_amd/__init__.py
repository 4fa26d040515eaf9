"""MI355X (gfx950) routed-expert forward of an MXFP4 Stable LatentMoE layer.

The compute path is the HIP library ``libmxmoe.so`` behind the C ABI in ``include/mxmoe.h``;
``abi`` binds it with ctypes and ``MoELayer`` manages device buffers with torch.
"""
from . import abi  # noqa: F401

__all__ = ["abi", "MoELayer"]


def __getattr__(name):
    if name == "MoELayer":
        from .layer import MoELayer
        return MoELayer
    raise AttributeError(name)
