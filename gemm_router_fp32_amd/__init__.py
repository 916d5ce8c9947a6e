"""libq4moe: routed-MoE 4-bit decode on MI355X (gfx950) behind a C ABI.

`q4moe` is the thin ctypes binding of libq4moe.so (include/q4moe.h); every
step of the computation runs in the library's HIP kernels.  PyTorch tensors
only carry device memory and the current stream.
"""
from . import q4moe  # noqa: F401
from .q4moe import *  # noqa: F401,F403
