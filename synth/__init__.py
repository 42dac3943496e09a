"""Seeded synthetic workloads shared by the CPU oracle tests, the GPU parity tests and the benchmark.

Holds configuration data and random draws only; no part of the step's arithmetic lives here.
"""
from .configs import (BF16, BIDIR, CAUSAL, CONFIGS, F32, FP8KV, LMHEAD_CONFIGS, QUAD, QUAD_CONFIGS,  # noqa: F401
                      TWO_STREAM_CONFIGS, lmhead_seed_of, quad_seed_of, seed_of, two_stream_seed_of)
from .gen import (bf16_bits_to_f32, cache_capacity, config_step, f32_to_bf16_bits, f32_to_e4m3_bits,  # noqa: F401
                  fresh_logits, lmhead_step, make_lmhead, make_quad_step, make_step, make_two_stream, params_for,
                  quad_slot_count, quad_step, two_stream_step)
