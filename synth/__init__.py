"""Seeded synthetic inputs shared by the tests, the bench and the oracle."""
from .inputs import (CONFIGS, DEFAULT_IGNORE_INDEX, Workload, attach_logprobs,  # noqa: F401
                     bf16_bits_to_f32, config, f32_to_bf16_bits, make_inputs, segment_lengths)
