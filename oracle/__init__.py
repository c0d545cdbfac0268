"""CPU float64 oracle for the chunked gated delta rule with state/W fake QDQ.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import anything under oracle/. The product path
(gateddeltanet_chunked_recurrence_amd) never imports it and shares no code
with it.

Modules:
  qdq        FP32 dynamic fake quantize-dequantize (E4M3 / INT8) of a tile
  recurrent  token-by-token recurrence (numpy float64), optional state QDQ
  chunked    chunked WY form with state/W QDQ (torch float64 CPU) and the
             identity straight-through backward (autograd)
  decode     decode continuation: exact chunk prefill of a prefix, then
             token-state writes through the state quantizer, both readouts,
             and the straight-through backward (torch float64 CPU)
"""
from .qdq import FMT_OFF, FMT_E4M3, FMT_INT8, qdq32, round_e4m3, round_int8, e4m3_encode  # noqa: F401
from .recurrent import recurrent_fwd  # noqa: F401
from .chunked import chunked_fwd, chunked_bwd, wy_factor, default_scale  # noqa: F401
from .decode import (READOUT_AFTER_WRITE, READOUT_BEFORE_WRITE, decode_bwd, decode_fwd,  # noqa: F401
                     prefill_decode_bwd, prefill_decode_fwd)
