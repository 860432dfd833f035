"""MI355X (gfx950) batch-1 fine-grained MoE decode step.

The hot path is the C-ABI library ``libmoedecode.so`` (hand-written HIP, see
``include/moe_decode.h``); ``fine_grained_moe_router_amd.native`` is its thin
ctypes binding. Importing this package loads nothing; the binding loads the
library on first use and raises if it is missing.
"""
__all__ = ["budget", "native"]
