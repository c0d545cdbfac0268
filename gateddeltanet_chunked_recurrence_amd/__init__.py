"""MI355X (gfx950) chunked gated delta rule with dynamic state/W fake QDQ.

The computation runs in hand-written HIP kernels (csrc/) behind the C ABI in
include/gdn.h; binding.py marshals torch device tensors into that ABI.
"""
from .binding import (GDN_BF16, GDN_F32, QDQ_E4M3, QDQ_INT8, QDQ_OFF, READOUT_AFTER_WRITE,  # noqa: F401
                      READOUT_BEFORE_WRITE, GdnError, gdn_chunk_bwd, gdn_chunk_fwd,
                      gdn_decode_bwd, gdn_decode_fwd, gdn_prefill_decode_bwd,
                      gdn_prefill_decode_fwd, gdn_qdq_state, load_library, make_fwd_args,
                      saved_layout)
