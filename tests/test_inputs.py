"""The seeded input generators: determinism, shapes, recipe statistics (CPU)."""
import numpy as np
import torch

from inputs import FRAME, TINY, VIDEO5S, VIDEO10S, VIDEO15S, make_inputs, random_case, sample_query_blocks
from inputs.generate import box_blocks, box_token_mask, gaussian_taps, plant_boxes, smooth_field


def test_config_table_shapes():
    expect = [(TINY, 256, 4), (FRAME, 4032, 63), (VIDEO5S, 124992, 1953), (VIDEO10S, 245952, 3843),
              (VIDEO15S, 366912, 5733)]
    for cfg, n, nb in expect:
        assert cfg.n_tokens == n and cfg.n_blocks == nb
        if cfg.sections is not None:
            assert sum(cfg.sections) == cfg.head_dim


def test_make_inputs_deterministic_and_typed():
    a = make_inputs(1)
    b = make_inputs(1)
    for name in ("q", "k", "v"):
        assert a[name].dtype == torch.bfloat16 and a[name].shape == (1, 256, 2, 64)
        assert a[name].is_contiguous()
        assert torch.equal(a[name], b[name])
    assert not torch.equal(a["q"], a["k"])
    assert a["wq"].dtype == torch.float32 and (a["wq"] >= 0.5).all() and (a["wq"] < 1.5).all()
    x = a["q"].float()
    assert abs(x.mean().item()) < 0.1 and abs(x.std().item() - 1) < 0.1


def test_smooth_field_statistics():
    g = torch.Generator().manual_seed(3)
    f = smooth_field((12, 16, 20), 8, g, "cpu").reshape(12, 16, 20, 8)
    # unit-std field plus std-0.5 noise
    assert abs(f.std().item() - np.sqrt(1.25)) < 0.1
    # neighbours along w are strongly correlated (sigma 2), far tokens are not
    a = f[:, :, :-1].flatten().numpy()
    b = f[:, :, 1:].flatten().numpy()
    c = f[:, :, :-10].flatten().numpy()
    d = f[:, :, 10:].flatten().numpy()
    assert np.corrcoef(a, b)[0, 1] > 0.6
    assert abs(np.corrcoef(c, d)[0, 1]) < 0.2
    taps = gaussian_taps()
    assert taps.numel() == 17 and abs(taps.sum().item() - 1) < 1e-6


def test_boxes_inside_grid_and_blocks():
    grid = VIDEO15S.grid
    boxes = plant_boxes(grid, torch.Generator().manual_seed(7))
    assert len(boxes) == 4
    for o in boxes:
        for x, n in zip(o, grid):
            assert 0 <= x <= n - 8
    m = box_token_mask(grid, boxes, "cpu")
    assert m.sum().item() <= 4 * 512 and m.sum().item() >= 512
    bl = box_blocks(grid, boxes)
    assert all(0 <= b < VIDEO15S.n_blocks for b in bl)


def test_sample_query_blocks():
    s = sample_query_blocks(1953, 32, 0)
    assert s[0] == 0 and s[-1] == 1952 and len(s) == 32 and s == sorted(set(s))
    assert sample_query_blocks(1953, 32, 0) == s
    assert sample_query_blocks(3, 32, 0) == [0, 1, 2]


def test_random_case():
    c = random_case(2, 100, 3, 64, seed=5)
    assert c["q"].shape == (2, 100, 3, 64) and c["q"].dtype == torch.bfloat16
