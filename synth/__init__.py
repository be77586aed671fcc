"""Seeded synthetic inputs (weights, prompts, planted drafts) and workload configurations.

Shared by the CPU oracle and the GPU path; holds none of the decoding method's arithmetic.
"""
from .configs import (B4, B27, CONFIGS, GREEDY, LONG, SMALL, TINY, DecoderCfg, DrafterCfg, RunCfg,  # noqa: F401
                      SamplingCfg, tensor_shapes, with_layers)
