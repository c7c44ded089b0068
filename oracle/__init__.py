"""CPU oracle of the EAGLE-3 draft head (test infrastructure only: the
tests, the smoke check and the bench's CPU-baseline leg use it; the
product path never does)."""
from .eagle3_oracle import (draft_chain, draft_extend, draft_step, greedy_accept, linear,  # noqa: F401
                            relaxed_accept, target_order, decode_e4m3, decode_e2m1, weight_view,
                            QuantWeight,
                            mla_attend_plain, rms_norm, rope_interleaved, rope_inv_freq,
                            rope_rotate_half, silu, softmax_attend, yarn_inv_freq, yarn_mscale)
