"""MI355X (gfx950) int4-weight MoE FFN step: HIP kernels behind a C ABI.

The compute path is libmoe_int4.so (include/moe.h); `moe` is its ctypes
binding, and `layer.MoeLayer` a small convenience wrapper that owns a
context and its resident experts.
"""
from . import moe  # noqa: F401
