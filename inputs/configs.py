"""The five synthetic workloads the library is measured and parity-checked on.

Grid sizes follow a MiniMax-H3-class video latent at 1344x768 (or 768x1344), 24 fps, with an
8x spatial VAE factor (mhpq.cn/news/447544, section 2.1: one latent frame is 8x smaller per side than
the picture), a 4x temporal VAE factor and a 2x2 patchifier (assumed; the pages do not state
them). Tokens are flattened as n = (t*H + h)*W + w.

This module holds shapes and constants only; no arithmetic of the method lives here.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    id: int
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]            # (T, H, W) latent tokens after patchify
    sections: Optional[Tuple[int, int, int]]  # RoPE head_dim split (d_t, d_h, d_w)
    theta: float
    eps: float
    sparsities: Tuple[float, ...]
    field: str                            # "normal" | "smooth" | "smooth_boxes"
    stages: Tuple[str, ...]               # which stages the workload lists
    block_size: int = 64

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.block_size)


# head_dim split over (t, h, w) for RoPE: 16/24/24 at D=64, 32/48/48 at D=128.
_SPLIT = {64: (16, 24, 24), 128: (32, 48, 48)}

CONFIGS = {
    1: Config(1, "tiny_4x8x8", 1, 2, 64, (4, 8, 8), _SPLIT[64], 1e4, 1e-6, (0.5,), "normal",
              ("norm_rope", "dense", "select", "sparse")),
    2: Config(2, "frame_1x48x84", 1, 24, 128, (1, 48, 84), _SPLIT[128], 1e4, 1e-6, (0.75,), "normal",
              ("norm_rope", "dense", "select", "sparse")),
    3: Config(3, "video5s_31x48x84", 1, 48, 128, (31, 48, 84), _SPLIT[128], 1e4, 1e-6, (0.75,), "smooth",
              ("dense", "select", "sparse")),
    4: Config(4, "video10s_61x48x84", 1, 12, 128, (61, 48, 84), _SPLIT[128], 1e4, 1e-6, (0.75, 0.80), "smooth",
              ("norm_rope", "dense", "select", "sparse")),
    5: Config(5, "video15s_91x84x48", 1, 12, 128, (91, 84, 48), _SPLIT[128], 1e4, 1e-6, (0.75,), "smooth_boxes",
              ("dense", "select", "sparse")),
}

# the five workloads by name
TINY, FRAME, VIDEO5S, VIDEO10S, VIDEO15S = (CONFIGS[i] for i in (1, 2, 3, 4, 5))

# tensor ids used to derive per-tensor seeds
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "wq": 3, "wk": 4, "boxes": 5}
BASE_SEED = 0

# smooth-field recipe (the three video workloads): Gaussian sigma and truncation radius in tokens, added noise std
FIELD_SIGMA = 2.0
FIELD_RADIUS = 8
FIELD_NOISE_STD = 0.5
# planted subject boxes (the 15 s workload)
BOX_COUNT = 4
BOX_EDGE = 8
BOX_KEY_GAIN = 3.0


def seed_for(cfg_id: int, tensor: str) -> int:
    """Deterministic seed for one tensor of one workload."""
    return BASE_SEED * 1_000_003 + cfg_id * 1000 + TENSOR_IDS[tensor]
