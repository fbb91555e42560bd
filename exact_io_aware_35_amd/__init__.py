"""MI355X (gfx950) exact attention: tiled forward with online softmax and LSE,
and the recompute-from-LSE backward, behind a C ABI (include/fa.h).

The Python layer only marshals arguments to libfa_mi355x.so; see binding.py.
"""

from .binding import (  # noqa: F401
    FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FaError, PreparedCall, backward, backward_qkvpacked, forward,
    forward_fp8, forward_qkvpacked, load_library, prepare_forward, prepare_forward_fp8,
    workspace_size,
    backward_noalloc,
)
from .autograd import FlashAttention, flash_attention  # noqa: F401
