"""MI355X (gfx950) FP4 mixture-of-experts feed-forward layer.

The layer runs entirely in the HIP kernels of ``libmoe_fp4.so`` behind the C ABI of
``include/moe_fp4.h``; :mod:`.binding` marshals torch tensors into that ABI.
"""
from .binding import *  # noqa: F401,F403
from .binding import load_library, LIB_PATH  # noqa: F401
