"""fp64 CPU oracle (test infrastructure only; see h3_oracle.py)."""
from .h3_oracle import *  # noqa: F401,F403
from .h3_oracle import (HEAD_DIM, ROTARY_DIM, HALF, FREQS_PER_AXIS, ROPE_THETA,  # noqa: F401
                        RMS_EPS)
