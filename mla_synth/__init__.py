"""Seeded synthetic MLA-decode workloads shared by the oracle tests and the GPU path.

Holds shapes, random draws, storage rounding, the cache-producing quantiser and
block packing only; no attention arithmetic lives here.
"""
from .configs import BLOCK_TOKENS, CONFIGS, SEEDS, MlaConfig, block_layout  # noqa: F401
from .gen import (MlaInputs, append_rows, append_slots, attended_pairs, make_inputs, pack_codes,  # noqa: F401
                  quantise_rtn, to_bf16_exact, bf16_bits, workload)
