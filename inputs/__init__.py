"""Seeded synthetic workloads (shapes, constants and random tensors only)."""
from .configs import CONFIGS, FRAME, TINY, VIDEO5S, VIDEO10S, VIDEO15S, Config, seed_for  # noqa: F401
from .generate import (box_blocks, make_inputs, random_case, sample_query_blocks,  # noqa: F401
                       smooth_field)
