"""Host-side model of the cross-lane row maxima of the bf16 attention tile
(video_diffusion_transformer_qk_amd/csrc/attention.hip, rows_tile): a query's scores sit in lanes
l, l^16, l^32, l^48 of a 64-lane wave, and both query tiles are combined in one pass. The two
gfx950 swap instructions are modelled as the ISA describes them (v_permlane16_swap exchanges the
odd 16-lane rows of its first operand with the even rows of its second; v_permlane32_swap the upper
32 lanes of its first with the lower 32 of its second); the test checks the lane bookkeeping the
kernel builds on them: which lane ends up with which query tile's maximum, the ballot masks that
split the rescale decision by query tile, and the threshold each lane compares against."""
import numpy as np


def permlane16_swap(x, y):
    x, y = x.copy(), y.copy()
    for row_x, row_y in ((1, 0), (3, 2)):
        sx, sy = slice(16 * row_x, 16 * row_x + 16), slice(16 * row_y, 16 * row_y + 16)
        x[sx], y[sy] = y[sy].copy(), x[sx].copy()
    return x, y


def permlane32_swap(x, y):
    x, y = x.copy(), y.copy()
    x[32:], y[:32] = y[:32].copy(), x[32:].copy()
    return x, y


def pair_max(v):
    a, b = permlane32_swap(v, v)
    return np.maximum(a, b)


def test_merged_row_maxima_lane_map():
    rng = np.random.default_rng(7)
    lane = np.arange(64)
    for _ in range(200):
        ml = rng.standard_normal((2, 64))  # per-lane partial maxima of query tiles 0 and 1
        # the exact four-lane maximum of query q = lane % 16 in each query tile
        want = np.array([[ml[qt, (l % 16)::16].max() for l in lane] for qt in range(2)])
        r0, r1 = permlane16_swap(ml[0], ml[1])
        z = pair_max(np.maximum(r0, r1))
        qt_of_row = (lane >> 4) & 1
        assert np.array_equal(z, want[qt_of_row, lane])
        # the rescale path: one more swap gives every lane both tiles' maxima
        zz0, zz1 = permlane16_swap(z, z)
        assert np.array_equal(zz0, want[0]) and np.array_equal(zz1, want[1])
        # ballot split: query tile 0's lanes are rows 0 and 2, query tile 1's rows 1 and 3
        thr = rng.standard_normal((2, 16))[:, lane % 16] + 0.5
        thr_mix = np.where(qt_of_row == 1, thr[1], thr[0])
        over = sum(1 << int(l) for l in lane if z[l] > thr_mix[l])
        for qt, mask in ((0, 0x0000FFFF0000FFFF), (1, 0xFFFF0000FFFF0000)):
            assert bool(over & mask) == bool((want[qt] > thr[qt]).any())
