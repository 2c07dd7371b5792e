"""Seeded synthetic inputs, shared by the tests, the bench and the oracle's callers.

Nothing here computes any step of the method: it draws random tensors and shapes them.
Tensors are produced with torch on the requested device (the GPU for the large workloads, where
a host-side smooth field of ~10^9 values would take minutes) and cast to bfloat16 with
round-to-nearest-even. Both sides of a parity check consume the same bf16 bytes.

Recipe (stated again in the design notes):
  * normal:  q, k, v i.i.d. N(0,1).
  * smooth:  q and k are, independently per tensor, head and channel, white N(0,1) noise on the
             T x H x W grid passed through a separable Gaussian filter (sigma 2 tokens, truncated
             at radius 8, mirror boundaries), rescaled to unit empirical std over the tensor, plus
             N(0, 0.5^2) noise; v is N(0,1).
  * smooth_boxes: as smooth, and k is multiplied by 3 inside the union of 4 seeded 8x8x8 boxes
             (all heads, channels), before the bf16 cast.
  * norm weights w_q, w_k ~ U(0.5, 1.5) in float32, shape [head_dim].
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import torch

from .configs import (BOX_COUNT, BOX_EDGE, BOX_KEY_GAIN, CONFIGS, FIELD_NOISE_STD, FIELD_RADIUS,
                      FIELD_SIGMA, Config, seed_for)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gaussian_taps(sigma: float = FIELD_SIGMA, radius: int = FIELD_RADIUS) -> torch.Tensor:
    x = torch.arange(-radius, radius + 1, dtype=torch.float64)
    w = torch.exp(-0.5 * (x / sigma) ** 2)
    return (w / w.sum()).to(torch.float32)


def _mirror_index(length: int, radius: int, device) -> torch.Tensor:
    idx = torch.arange(-radius, length + radius, device=device).abs()
    return torch.where(idx > length - 1, 2 * (length - 1) - idx, idx)


def _filter_axis(x: torch.Tensor, axis: int, taps: torch.Tensor) -> torch.Tensor:
    length = x.shape[axis]
    radius = (taps.numel() - 1) // 2
    if length == 1:
        return x
    if length <= radius:
        raise ValueError("axis too short for the filter radius")
    xp = x.index_select(axis, _mirror_index(length, radius, x.device))
    y = torch.zeros_like(x)
    for i, t in enumerate(taps.tolist()):
        y.add_(xp.narrow(axis, i, length), alpha=t)
    return y


def smooth_field(grid: Tuple[int, int, int], channels: int, gen: torch.Generator, device) -> torch.Tensor:
    """Float32 [T*H*W, channels] field; see the module docstring for the recipe."""
    t, h, w = grid
    x = torch.randn((t, h, w, channels), generator=gen, device=device, dtype=torch.float32)
    taps = gaussian_taps()
    for axis in range(3):
        x = _filter_axis(x, axis, taps)
    x.div_(x.std())
    x.add_(torch.randn(x.shape, generator=gen, device=device, dtype=torch.float32), alpha=FIELD_NOISE_STD)
    return x.reshape(t * h * w, channels)


def plant_boxes(grid: Tuple[int, int, int], gen: torch.Generator) -> List[Tuple[int, int, int]]:
    """Origins of BOX_COUNT boxes of edge BOX_EDGE lying fully inside the grid."""
    t, h, w = grid
    out = []
    for _ in range(BOX_COUNT):
        o = [int(torch.randint(0, n - BOX_EDGE + 1, (1,), generator=gen).item()) for n in (t, h, w)]
        out.append(tuple(o))
    return out


def box_token_mask(grid: Tuple[int, int, int], boxes, device) -> torch.Tensor:
    t, h, w = grid
    m = torch.zeros((t, h, w), dtype=torch.bool, device=device)
    for (a, b, c) in boxes:
        m[a:a + BOX_EDGE, b:b + BOX_EDGE, c:c + BOX_EDGE] = True
    return m.reshape(-1)


def normal_bf16(shape, seed: int, device) -> torch.Tensor:
    g = _gen(device, seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def norm_weight(head_dim: int, seed: int, device) -> torch.Tensor:
    g = _gen(device, seed)
    return (torch.rand((head_dim,), generator=g, device=device, dtype=torch.float32) + 0.5)


def make_inputs(cfg: Config | int, device="cpu") -> Dict[str, object]:
    """q, k, v (bf16, [B, N, heads, D], contiguous), w_q, w_k (fp32 [D]) and, for the planted-box
    workload, the box origins."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    b, n, hd, d = cfg.batch, cfg.n_tokens, cfg.heads, cfg.head_dim
    shape = (b, n, hd, d)
    out: Dict[str, object] = {"cfg": cfg}
    if cfg.field == "normal":
        out["q"] = normal_bf16(shape, seed_for(cfg.id, "q"), device)
        out["k"] = normal_bf16(shape, seed_for(cfg.id, "k"), device)
    else:
        boxes = None
        if cfg.field == "smooth_boxes":
            boxes = plant_boxes(cfg.grid, _gen("cpu", seed_for(cfg.id, "boxes")))
            out["boxes"] = boxes
        for name in ("q", "k"):
            g = _gen(device, seed_for(cfg.id, name))
            parts = []
            for _ in range(b):
                f = smooth_field(cfg.grid, hd * d, g, device)
                if name == "k" and boxes is not None:
                    mask = box_token_mask(cfg.grid, boxes, device)
                    f[mask] *= BOX_KEY_GAIN
                parts.append(f.to(torch.bfloat16).reshape(1, n, hd, d))
                del f
            out[name] = torch.cat(parts, 0) if b > 1 else parts[0]
    out["v"] = normal_bf16(shape, seed_for(cfg.id, "v"), device)
    out["wq"] = norm_weight(d, seed_for(cfg.id, "wq"), device)
    out["wk"] = norm_weight(d, seed_for(cfg.id, "wk"), device)
    return out


def random_case(batch: int, n_tokens: int, heads: int, head_dim: int, seed: int, device="cpu",
                scale: float = 1.0) -> Dict[str, torch.Tensor]:
    """Free-shape N(0, scale^2) q, k, v in bf16 plus U(0.5,1.5) weights, for edge-case tests."""
    shape = (batch, n_tokens, heads, head_dim)
    g = _gen(device, seed)
    mk = lambda: (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale).to(torch.bfloat16)
    q, k, v = mk(), mk(), mk()
    wq = torch.rand((head_dim,), generator=g, device=device, dtype=torch.float32) + 0.5
    wk = torch.rand((head_dim,), generator=g, device=device, dtype=torch.float32) + 0.5
    return {"q": q, "k": k, "v": v, "wq": wq, "wk": wk}


def sample_query_blocks(n_blocks: int, count: int, seed: int, extra=()) -> List[int]:
    """Seeded sample of query-block indices, always containing the first and last block."""
    g = _gen("cpu", seed)
    chosen = {0, n_blocks - 1}
    chosen.update(int(e) for e in extra if 0 <= int(e) < n_blocks)
    if n_blocks > len(chosen):
        perm = torch.randperm(n_blocks, generator=g).tolist()
        for p in perm:
            if len(chosen) >= max(count, 2):
                break
            chosen.add(p)
    return sorted(chosen)


def box_blocks(grid, boxes, block_size: int = 64) -> List[int]:
    """Indices of the 64-token blocks that contain at least one token of a planted box."""
    m = box_token_mask(grid, boxes, "cpu")
    tok = torch.nonzero(m).flatten()
    return sorted(set((tok // block_size).tolist()))


def bytes_of(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


__all__ = ["make_inputs", "random_case", "smooth_field", "gaussian_taps", "plant_boxes",
           "box_token_mask", "sample_query_blocks", "box_blocks", "normal_bf16", "norm_weight",
           "bytes_of"]
