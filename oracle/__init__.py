"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .qsa_oracle import (attn_fwd, attn_bwd, head_bwd, head_rows, row_weights, decode_bf16, decode_e4m3fn, decode_f32,
                         IDX_FLUSHED, IDX_MASKED, LOG2E)
from . import scalar
