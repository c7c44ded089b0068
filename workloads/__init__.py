"""Workload shapes and seeded synthetic inputs shared by the oracle, the tests and the bench."""
from .configs import CONFIGS, MHA, MLA, QUANTIZED, SMALL, Eagle3Config, get_config  # noqa: F401
from .synth import (make_accept_targets, make_d2t, make_extend_inputs, make_inputs, make_weights,  # noqa: F401
                    make_relaxed_inputs, normal_bf16, quant_codes, random_drafts)
from .layout import cache_keys, to_plain, to_tiled  # noqa: F401
