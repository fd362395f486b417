"""fp64 CPU oracle (test infrastructure only; see h3_oracle.py)."""
from .h3_oracle import *  # noqa: F401,F403
from .h3_oracle import (HEAD_DIM, ROTARY_DIM, HALF, FREQS_PER_AXIS, ROPE_THETA,  # noqa: F401
                        RMS_EPS)
from .h3_oracle_backward import (attention_head_backward, attention_backward,  # noqa: F401
                                 log_sum_exp_rows, mm_rope_backward, rms_norm_backward,
                                 qk_prologue_backward, packed_attention_backward)
from .h3_oracle_fp8 import (e4m3_encode, e4m3_decode, e4m3_round, quantized_operands,  # noqa: F401
                            quantized_attention_head, packed_attention_fp8)
