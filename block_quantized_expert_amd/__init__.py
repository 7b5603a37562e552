"""MI355X-native routed MoE FFN with MXFP4 block-quantized experts.

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP
kernels for gfx950, declared in ``include/moe.h``); ``binding`` is a thin
ctypes layer over it that marshals torch tensors and streams.
"""

__all__ = ["binding", "inputs"]
