"""MI355X (gfx950) chunked gated delta rule with dynamic state/W fake QDQ.

The computation runs in hand-written HIP kernels (csrc/) behind the C ABI in
include/gdn.h; binding.py marshals torch device tensors into that ABI.
"""
from .binding import (GDN_BF16, GDN_F32, QDQ_E4M3, QDQ_INT8, QDQ_OFF, GdnError,  # noqa: F401
                      gdn_chunk_bwd, gdn_chunk_fwd, gdn_qdq_state, load_library, saved_layout,
                      make_fwd_args)
