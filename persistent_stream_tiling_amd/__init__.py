"""MI355X-native tiled GEMM with data-parallel, persistent, Stream-K and hybrid schedules.

A thin Python binding over the C ABI of ``libgemmsk.so`` (include/gemm_sk.h).
Every arithmetic step runs in the library's gfx950 kernels; this package only
marshals arguments.  PyTorch supplies device memory and the current stream.
"""
from ._lib import (BF16, DP, DTYPES, F16, F32, I8, FLAG_C_INPUT_DTYPE,
                   FLAG_DEBUG_DROP_SIGNAL, FLAG_FIXUP_TWO_KERNEL, FLAG_STREAM_COPIES,
                   FLAG_PING_PONG, FLAG_HILBERT_ORDER, FLAG_RING_KERNEL, FLAG_TILE_SPLIT,
                   FLAG_FIXUP_HEAD, FLAG_FIXUP_SPLIT, FLAG_NO_XCD_REMAP, FLAG_ONE_TILE, HYBRID,
                   PERSISTENT, ROLE_CONTRIB, ROLE_FULL, ROLE_OWNER, SCHEDULES, STREAMK, load,
                   variants)
from .plan import FixupError, GemmPlan, matmul, plan_for_device

__all__ = ["GemmPlan", "FixupError", "matmul", "plan_for_device", "load", "variants",
           "SCHEDULES", "DTYPES", "DP", "PERSISTENT", "STREAMK", "HYBRID", "F32", "F16", "BF16",
           "I8", "FLAG_ONE_TILE", "FLAG_NO_XCD_REMAP", "FLAG_FIXUP_HEAD", "FLAG_FIXUP_SPLIT",
           "FLAG_C_INPUT_DTYPE", "FLAG_DEBUG_DROP_SIGNAL", "FLAG_FIXUP_TWO_KERNEL",
           "FLAG_STREAM_COPIES", "FLAG_PING_PONG", "FLAG_HILBERT_ORDER", "FLAG_RING_KERNEL",
           "FLAG_TILE_SPLIT", "ROLE_FULL", "ROLE_CONTRIB", "ROLE_OWNER"]
