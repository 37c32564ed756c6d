"""Seeded synthetic inputs for the trie-constrained beam step.

Shared by the oracle's tests and by the GPU path's tests and benchmark; it
holds shapes, distributions, seeds and input formats only, and no part of the
beam step itself.
"""
from .configs import BF16, CONFIGS, F32, Config, get  # noqa: F401
from .catalog import Trie, csr_from_codes, make_codes, make_trie, relabel, sid_tokens  # noqa: F401
from .logits import (bf16_bits_to_f32, full_step, iter_step_blocks, prefix_block,  # noqa: F401
                     prefix_row, step_logits, to_bf16_bits, token_bias)
