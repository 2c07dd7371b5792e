"""Pins for the float64 oracle: closed forms, invariants, library special cases, brute force and
hand-worked fixtures. Each pin is chosen so that a plausible slip in the oracle (a dropped term,
a wrong axis, sign or index, a transposed operand) fails at least one of them. CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ----------------------------------------------------------------------------------- rms_norm

def test_rms_norm_matches_torch_library_routine():
    x = rnd(2, 5, 3, 16)
    w = RNG.uniform(0.5, 1.5, 16)
    for eps in (1e-6, 0.3):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (16,), torch.from_numpy(w), eps).numpy()
        np.testing.assert_allclose(O.rms_norm(x, w, eps), ref, rtol=1e-14, atol=1e-14)


def test_rms_norm_closed_form_rms_and_eps_inside_sqrt():
    x = rnd(4, 7, 2, 32)
    w = RNG.uniform(0.5, 1.5, 32)
    eps = 0.5  # large, so eps placement matters
    y = O.rms_norm(x, w, eps)
    ms = np.mean(x * x, axis=-1)
    rms_unweighted = np.sqrt(np.mean((y / w) ** 2, axis=-1))
    np.testing.assert_allclose(rms_unweighted, np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # a constant weight c gives output rms c * sqrt(ms/(ms+eps)): "output rms equals its weight"
    c = 1.7
    y2 = O.rms_norm(x, np.full(32, c), 1e-300)
    np.testing.assert_allclose(np.sqrt(np.mean(y2 ** 2, axis=-1)), c, rtol=1e-13)


def test_rms_norm_special_cases():
    w = RNG.uniform(0.5, 1.5, 8)
    for c, eps in ((2.0, 1e-6), (-0.25, 0.1), (3.0, 0.0)):
        x = np.full((1, 1, 1, 8), c)
        np.testing.assert_allclose(O.rms_norm(x, w, eps)[0, 0, 0], w * c / math.sqrt(c * c + eps), rtol=1e-14)
    x = rnd(3, 4, 2, 16)
    w = RNG.uniform(0.5, 1.5, 16)
    # eps = 0: scale invariant, odd
    np.testing.assert_allclose(O.rms_norm(3.5 * x, w, 0.0), O.rms_norm(x, w, 0.0), rtol=1e-13)
    np.testing.assert_allclose(O.rms_norm(-x, w, 0.0), -O.rms_norm(x, w, 0.0), rtol=1e-14)


def test_rms_norm_is_per_head():
    x = rnd(1, 3, 4, 16)
    w = RNG.uniform(0.5, 1.5, 16)
    y = O.rms_norm(x, w, 1e-6)
    x2 = x.copy()
    x2[:, :, 2, :] *= 100.0  # another head changes
    y2 = O.rms_norm(x2, w, 1e-6)
    np.testing.assert_array_equal(y[:, :, [0, 1, 3]], y2[:, :, [0, 1, 3]])


# ----------------------------------------------------------------------------------- rope3d

def _complex_rope_1d(x_section, p, theta):
    """1-D rotary embedding written as complex multiplication z_j * exp(i p theta^(-2j/d))."""
    d = x_section.shape[-1]
    z = x_section[..., 0::2] + 1j * x_section[..., 1::2]
    j = np.arange(d // 2)
    rot = np.exp(1j * np.multiply.outer(p, theta ** (-2.0 * j / d)))  # [N, d/2]
    z = z * rot[None, :, None, :]
    out = np.empty_like(x_section)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def test_rope_worked_example_golden():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "rope_worked_example.txt")) if l.strip() and not l.startswith("#")]
    token = int(lines[0][1])
    expect = np.array([[float(a), float(b)] for _, _, a, b in lines[1:]]).reshape(-1)
    x = np.zeros((1, 24, 1, 8))
    x[..., 0::2] = 1.0
    y = O.rope3d(x, (2, 3, 4), (2, 2, 4), 100.0)
    np.testing.assert_allclose(y[0, token, 0], expect, rtol=0, atol=2e-16)


def test_rope_preserves_norms_and_is_identity_at_origin():
    grid, sec = (3, 4, 5), (16, 24, 24)
    x = rnd(2, 60, 3, 64)
    y = O.rope3d(x, grid, sec, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    pair_x = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    pair_y = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(pair_y, pair_x, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])  # token 0 sits at (0, 0, 0)


def test_rope_single_axis_grids_equal_complex_1d_rope():
    theta = 1e4
    sec = (16, 24, 24)
    for axis, grid in ((0, (9, 1, 1)), (1, (1, 9, 1)), (2, (1, 1, 9))):
        x = rnd(1, 9, 2, 64)
        y = O.rope3d(x, grid, sec, theta)
        offs = (0, 16, 40, 64)
        for a in range(3):
            sl = slice(offs[a], offs[a + 1])
            if a == axis:
                np.testing.assert_allclose(y[..., sl], _complex_rope_1d(x[..., sl], np.arange(9.0), theta), atol=1e-13)
            else:
                np.testing.assert_array_equal(y[..., sl], x[..., sl])


def test_rope_token_flattening_matches_per_axis_coordinates():
    grid, sec, theta = (3, 4, 5), (16, 24, 24), 1e4
    x = rnd(1, 60, 2, 64)
    y = O.rope3d(x, grid, sec, theta)
    n = np.arange(60)
    coords = (n // 20, (n // 5) % 4, n % 5)
    offs = (0, 16, 40, 64)
    for a in range(3):
        sl = slice(offs[a], offs[a + 1])
        np.testing.assert_allclose(y[..., sl], _complex_rope_1d(x[..., sl], coords[a].astype(float), theta), atol=1e-13)


def test_rope_relative_position_property():
    """q.k after RoPE depends only on the (t, h, w) offset between the two tokens."""
    grid, sec, theta = (4, 5, 6), (16, 24, 24), 1e4
    t_, h_, w_ = grid
    tok = lambda t, h, w: (t * h_ + h) * w_ + w
    q = rnd(64)
    k = rnd(64)
    x = np.zeros((1, t_ * h_ * w_, 2, 64))
    x[0, :, 0, :] = q
    x[0, :, 1, :] = k
    y = O.rope3d(x, grid, sec, theta)
    dot = lambda a, b: float(y[0, a, 0] @ y[0, b, 1])
    base = dot(tok(0, 1, 2), tok(2, 3, 1))
    shifted = dot(tok(1, 2, 5 - 1), tok(3, 4, 3))  # both tokens moved by (+1, +1, +2)
    assert abs(base - shifted) < 1e-12 * (1 + abs(base))
    other = dot(tok(0, 1, 2), tok(2, 3, 2))  # different offset: differs
    assert abs(base - other) > 1e-6


def test_rope_group_law_double_application():
    """R(p) R(p) = R(2p): rope twice on a 1x1xW grid equals rope once at even positions of 1x1x2W."""
    theta, sec = 1e4, (16, 24, 24)
    x = rnd(1, 7, 2, 64)
    twice = O.rope3d(O.rope3d(x, (1, 1, 7), sec, theta), (1, 1, 7), sec, theta)
    x2 = np.zeros((1, 14, 2, 64))
    x2[:, 0::2] = x
    once = O.rope3d(x2, (1, 1, 14), sec, theta)[:, 0::2]
    np.testing.assert_allclose(twice, once, atol=1e-12)


def test_rope_frequency_closed_form():
    # section of width 4, theta 100: pair 1 turns at 100^(-1/2) = 0.1 rad per position
    x = np.zeros((1, 6, 1, 8))
    x[..., 0::2] = 1.0
    y = O.rope3d(x, (1, 1, 6), (2, 2, 4), 100.0)
    p = np.arange(6.0)
    np.testing.assert_allclose(y[0, :, 0, 6], np.cos(0.1 * p), atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, 7], np.sin(0.1 * p), atol=1e-15)
    np.testing.assert_allclose(y[0, :, 0, 4], np.cos(p), atol=1e-15)


def test_fused_norm_rope_is_the_composition():
    grid, sec = (2, 3, 4), (16, 24, 24)
    q, k = rnd(1, 24, 3, 64), rnd(1, 24, 3, 64)
    wq, wk = RNG.uniform(0.5, 1.5, 64), RNG.uniform(0.5, 1.5, 64)
    qo, ko = O.qk_norm_rope(q, k, wq, wk, grid, sec, 1e4, 1e-6)
    np.testing.assert_array_equal(qo, O.rope3d(O.rms_norm(q, wq, 1e-6), grid, sec, 1e4))
    np.testing.assert_array_equal(ko, O.rope3d(O.rms_norm(k, wk, 1e-6), grid, sec, 1e4))
    # norm preserved by RoPE => rms of output over head_dim equals rms of the normed input
    n = O.rms_norm(q, wq, 1e-6)
    np.testing.assert_allclose(np.linalg.norm(qo, axis=-1), np.linalg.norm(n, axis=-1), rtol=1e-13)


# ----------------------------------------------------------------------------------- attention

def test_attention_matches_torch_sdpa_float64():
    q, k, v = rnd(2, 37, 3, 16), rnd(2, 37, 3, 16), rnd(2, 37, 3, 16)
    out, lse = O.attention(q, k, v)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v)).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    s = torch.einsum("bhqd,bhkd->bhqk", t(q), t(k)) / 4.0
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13)


def test_attention_brute_force_loops():
    q, k, v = rnd(5, 8), rnd(6, 8), rnd(6, 8)
    out, lse = O.attention_head(q, k, v)
    for i in range(5):
        s = [sum(q[i, d] * k[j, d] for d in range(8)) / math.sqrt(8) for j in range(6)]
        e = [math.exp(x) for x in s]
        z = sum(e)
        for d in range(8):
            assert abs(out[i, d] - sum(e[j] * v[j, d] for j in range(6)) / z) < 1e-13
        assert abs(lse[i] - math.log(z)) < 1e-13


def test_attention_invariants():
    q, k, v = rnd(9, 16), rnd(11, 16), rnd(11, 16)
    out, _ = O.attention_head(q, k, v)
    # constant V -> constant output
    c = np.tile(rnd(16), (11, 1))
    np.testing.assert_allclose(O.attention_head(q, k, c)[0], np.tile(c[0], (9, 1)), atol=1e-13)
    # q = 0 -> uniform weights -> mean of V
    np.testing.assert_allclose(O.attention_head(np.zeros((2, 16)), k, v)[0], np.tile(v.mean(0), (2, 1)), atol=1e-13)
    # single key -> its value
    np.testing.assert_allclose(O.attention_head(q, k[:1], v[:1])[0], np.tile(v[0], (9, 1)), atol=1e-14)
    # shifting every key by the same vector leaves O unchanged
    u = rnd(16)
    np.testing.assert_allclose(O.attention_head(q, k + u, v)[0], out, atol=1e-12)
    # jointly permuting keys and values leaves O unchanged
    perm = RNG.permutation(11)
    np.testing.assert_allclose(O.attention_head(q, k[perm], v[perm])[0], out, atol=1e-13)
    # with V = identity the output is the probability matrix: rows sum to 1, entries >= 0
    p, _ = O.attention_head(q, k, np.eye(11))
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)


def test_attention_two_key_closed_form():
    q = np.array([[2.0, 0.0, 0.0, 0.0]])
    k = np.array([[1.0, 0.0, 0.0, 0.0], [-1.0, 0.0, 0.0, 0.0]])
    v = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0]])
    out, lse = O.attention_head(q, k, v)
    s1, s2 = 1.0, -1.0  # (2 * +-1) / sqrt(4)
    a = math.exp(s1) / (math.exp(s1) + math.exp(s2))
    np.testing.assert_allclose(out[0], a * v[0] + (1 - a) * v[1], rtol=1e-15)
    assert abs(lse[0] - math.log(math.exp(s1) + math.exp(s2))) < 1e-15


def test_attention_large_logits_are_stable():
    q = rnd(3, 16) * 40
    k = rnd(20, 16) * 40
    out, lse = O.attention_head(q, k, rnd(20, 16))
    assert np.isfinite(out).all() and np.isfinite(lse).all()


# ----------------------------------------------------------------------------------- selection

def _golden_keep_counts():
    rows = []
    for line in open(os.path.join(GOLDEN, "keep_counts.txt")):
        line = line.split("#")[0].strip()
        if line:
            n, s, k = line.split()
            rows.append((int(n), float(s), int(k)))
    return rows


def test_keep_count_golden():
    rows = _golden_keep_counts()
    assert len(rows) >= 8
    for n, s, k in rows:
        assert O.keep_count(n, s) == k, (n, s)


def test_keep_count_monotone_and_bounds():
    for n in (1, 2, 5, 63, 1953):
        prev = n + 1
        for s in np.linspace(0, 0.999, 200):
            k = O.keep_count(n, float(s))
            assert 1 <= k <= n and k <= prev
            prev = k
        assert O.keep_count(n, 0.0) == n
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            O.keep_count(10, bad)


def test_block_means_partial_block_and_closed_form():
    n = 150  # blocks of 64: [0,64), [64,128), [128,150)
    x = np.zeros((1, n, 2, 3))
    x[0, :, 0, 0] = np.arange(n)
    x[0, :, 1, 2] = 1.0
    m = O.block_means(x, 64)
    assert m.shape == (1, 2, 3, 3)
    np.testing.assert_allclose(m[0, 0, :, 0], [31.5, 95.5, (128 + 149) / 2.0])
    np.testing.assert_allclose(m[0, 1, :, 2], [1.0, 1.0, 1.0])


def test_block_scores_equal_block_mean_of_dense_logits():
    n, d = 200, 16
    q, k = rnd(1, n, 2, d), rnd(1, n, 2, d)
    s = O.block_scores(q, k, 64)
    nb = 4
    for h in range(2):
        logits = q[0, :, h, :] @ k[0, :, h, :].T / math.sqrt(d)
        for i in range(nb):
            for j in range(nb):
                blk = logits[i * 64:min(n, (i + 1) * 64), j * 64:min(n, (j + 1) * 64)]
                assert abs(s[0, h, i, j] - blk.mean()) < 1e-12


def _brute_topk(row, keep):
    idx = list(range(len(row)))
    idx.sort(key=lambda j: (-row[j], j))
    return sorted(idx[:keep])


def test_topk_brute_force_with_ties():
    for trial in range(200):
        n = int(RNG.integers(1, 30))
        keep = int(RNG.integers(1, n + 1))
        row = RNG.integers(-3, 4, n).astype(float)  # many exact ties
        got = O.topk_blocks(row[None, :], keep)[0].tolist()
        assert got == _brute_topk(row, keep)


def test_topk_invariants_and_planted_duplicate_blocks():
    n, d = 8 * 64, 16
    q, k = rnd(1, n, 1, d), rnd(1, n, 1, d)
    k[0, 5 * 64:6 * 64] = k[0, 2 * 64:3 * 64]  # key block 5 duplicates block 2
    s = O.block_scores(q, k, 64)
    assert (s[..., 5] == s[..., 2]).all()
    for keep in range(1, 9):
        idx = O.topk_blocks(s, keep)
        assert idx.shape == (1, 1, 8, keep) and idx.dtype == np.int32
        for row, sc in zip(idx[0, 0], s[0, 0]):
            assert len(set(row.tolist())) == keep and (np.diff(row) > 0).all()
            assert row.min() >= 0 and row.max() < 8
            if 5 in row.tolist():
                assert 2 in row.tolist()  # tie resolves to the lower index first
            kept_min = sc[row].min()
            dropped = np.setdiff1d(np.arange(8), row)
            if dropped.size:
                assert sc[dropped].max() <= kept_min
    full = O.subblock_select(q, k, 64, 0.0)
    assert (full == np.arange(8)).all()


def test_near_tie_rows():
    s = np.array([[5.0, 4.0, 3.0, 2.0],
                  [1.0, 1.0 + 5e-6, 0.0, 0.0],
                  [1.0, 1.0 + 2e-5, 0.0, 0.0],
                  [0.0, 0.0, 0.0, 0.0]])
    np.testing.assert_array_equal(O.near_tie_rows(s, 1), [False, True, False, True])
    assert not O.near_tie_rows(s, 4).any()


def test_near_threshold_entries_hand_built_rows():
    """Entries at, just inside and just outside the threshold max - tau, for a window of 1e-9 times
    the row's largest magnitude. Each row is built so that one plausible slip flips an entry:
    comparing with the maximum instead of max - tau (row a, first entry), a wider or narrower
    window (row a, entries 3 and 7), and scaling
    by the row maximum instead of the largest magnitude (rows b and c)."""
    # row a: threshold 0.5, largest magnitude 1.0 -> window 1e-9
    a = np.array([[1.0, 0.5, 0.5 + 4e-10, 0.5 + 2e-9, 0.5 - 9e-10, 0.5 - 1.1e-9, 0.5 + 1e-6, -1.0]])
    np.testing.assert_array_equal(O.near_threshold_entries(a, 0.5),
                                  [[False, True, True, False, True, False, False, False]])
    # row b: the threshold -0.3 is negative while the maximum 0.2 is positive; largest magnitude
    # 0.3 -> window 3e-10 (a window from the maximum, 2e-10, would miss entries 4 and 8)
    b = np.array([[0.2, -0.3, 0.1, -0.3 + 2.5e-10, -0.3 + 4e-10, 0.15, 0.0, -0.3 - 2.5e-10]])
    np.testing.assert_array_equal(O.near_threshold_entries(b, 0.5),
                                  [[False, True, False, True, False, False, False, True]])
    # row c: a large negative entry sets the scale (5.0 -> window 5e-9), far wider than the
    # maximum 0.01 would give
    c = np.array([[0.01, -5.0, -0.01 + 4e-9, -0.01 + 6e-9, -0.01, 0.0, 0.005, -0.01 - 4.9e-9]])
    np.testing.assert_array_equal(O.near_threshold_entries(c, 0.02),
                                  [[False, False, True, False, True, False, False, True]])
    # the rows are independent: stacked, each keeps its own maximum and scale
    both = np.concatenate([a, a * 4.0], axis=0)
    np.testing.assert_array_equal(O.near_threshold_entries(both, 0.5)[0], O.near_threshold_entries(a, 0.5)[0])
    np.testing.assert_array_equal(O.near_threshold_entries(both, 0.5)[1],
                                  [False, False, False, False, False, False, False, False])
    # tau = 0: the window sits on the maximum itself
    np.testing.assert_array_equal(O.near_threshold_entries(np.array([[2.0, 2.0 - 1e-9, 1.0]]), 0.0),
                                  [[True, True, False]])


# ----------------------------------------------------------------------------------- sparse attention

def test_sparse_keep_all_equals_dense():
    n, d = 3 * 64 + 17, 16
    q, k, v = rnd(1, n, 2, d), rnd(1, n, 2, d), rnd(1, n, 2, d)
    nb = 4
    idx = np.tile(np.arange(nb, dtype=np.int32), (1, 2, nb, 1))
    so, sl = O.sparse_attention(q, k, v, idx, 64)
    do, dl = O.attention(q, k, v)
    np.testing.assert_allclose(so, do, atol=1e-12)
    np.testing.assert_allclose(sl, dl, atol=1e-12)


def test_sparse_single_block_and_masked_formulation():
    n, d, nb = 4 * 64, 16, 4
    q, k, v = rnd(1, n, 1, d), rnd(1, n, 1, d), rnd(1, n, 1, d)
    # keep = 1 with block j: plain attention over that block's tokens only
    idx = np.full((1, 1, nb, 1), 2, dtype=np.int32)
    so, _ = O.sparse_attention(q, k, v, idx, 64)
    ref, _ = O.attention_head(q[0, :, 0], k[0, 128:192, 0], v[0, 128:192, 0])
    np.testing.assert_allclose(so[0, :, 0], ref, atol=1e-13)
    # general keep: equal to dense logits with dropped blocks masked to -inf (independent form)
    idx = O.subblock_select(q, k, 64, 0.5)
    so, _ = O.sparse_attention(q, k, v, idx, 64)
    logits = q[0, :, 0] @ k[0, :, 0].T / math.sqrt(d)
    for i in range(nb):
        mask = np.full(nb, -np.inf)
        mask[idx[0, 0, i]] = 0.0
        lg = logits[i * 64:(i + 1) * 64] + np.repeat(mask, 64)[None, :]
        p = np.exp(lg - lg.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(so[0, i * 64:(i + 1) * 64, 0], p @ v[0, :, 0], atol=1e-13)


def test_sparse_index_order_does_not_matter():
    n, d, nb = 5 * 64, 16, 5
    q, k, v = rnd(1, n, 1, d), rnd(1, n, 1, d), rnd(1, n, 1, d)
    idx = O.subblock_select(q, k, 64, 0.4)
    shuffled = idx[..., ::-1].copy()
    a, _ = O.sparse_attention(q, k, v, idx, 64)
    b, _ = O.sparse_attention(q, k, v, shuffled, 64)
    np.testing.assert_allclose(a, b, atol=1e-13)


# ----------------------------------------------------------------------------------- threshold mode

def _brute_threshold(row, tau):
    m = max(row)
    return [j for j in range(len(row)) if row[j] >= m - tau]


def test_threshold_blocks_brute_force_and_csr_layout():
    for trial in range(100):
        r, n = int(RNG.integers(1, 6)), int(RNG.integers(1, 20))
        s = RNG.integers(-4, 5, (r, n)).astype(float) * 0.5   # exact ties and exact threshold hits
        tau = float(RNG.choice([0.0, 0.5, 1.0, 2.5, np.inf]))
        rp, ci = O.threshold_blocks(s, tau)
        assert rp.dtype == np.int64 and ci.dtype == np.int32 and rp[0] == 0 and rp[-1] == len(ci)
        for i in range(r):
            assert ci[rp[i]:rp[i + 1]].tolist() == _brute_threshold(s[i].tolist(), tau)


def test_threshold_special_cases_and_monotonicity():
    n, d = 6 * 64, 16
    q, k = rnd(1, n, 2, d), rnd(1, n, 2, d)
    s = O.block_scores(q, k, 64)
    rp0, ci0 = O.threshold_blocks(s, 0.0)
    assert (np.diff(rp0) == 1).all()                       # tau = 0: only the row maximum (no ties here)
    assert (ci0 == s.reshape(-1, 6).argmax(1)).all()
    rpi, cii = O.threshold_blocks(s, np.inf)
    assert (np.diff(rpi) == 6).all() and (cii.reshape(-1, 6) == np.arange(6)).all()
    prev = np.diff(rp0)
    for tau in (0.01, 0.05, 0.1, 0.5, 2.0):
        rp, ci = O.threshold_blocks(s, tau)
        cnt = np.diff(rp)
        assert (cnt >= prev).all()
        prev = cnt
        # a threshold set is the top-c set of that row for its own count c
        for row in range(rp.size - 1):
            c = cnt[row]
            top = O.topk_blocks(s.reshape(-1, 6)[row:row + 1], int(c))[0]
            assert sorted(ci[rp[row]:rp[row + 1]].tolist()) == top.tolist()
    with pytest.raises(ValueError):
        O.threshold_blocks(s, -1.0)


def test_sparse_csr_matches_fixed_keep_form():
    n, d, nb = 5 * 64, 16, 5
    q, k, v = rnd(1, n, 2, d), rnd(1, n, 2, d), rnd(1, n, 2, d)
    idx = O.subblock_select(q, k, 64, 0.6)
    keep = idx.shape[-1]
    rp = np.arange(0, 2 * nb * keep + 1, keep, dtype=np.int64)
    a, la = O.sparse_attention(q, k, v, idx, 64)
    b, lb = O.sparse_attention_csr(q, k, v, rp, idx.reshape(-1), 64)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    # variable rows: keep-all rows reproduce dense attention
    rpi, cii = O.subblock_select_threshold(q, k, 64, np.inf)
    c, _ = O.sparse_attention_csr(q, k, v, rpi, cii, 64)
    dense, _ = O.attention(q, k, v)
    np.testing.assert_allclose(c, dense, atol=1e-12)


# ----------------------------------------------------------------------------------- AdaLN, SwiGLU

def test_adaln_matches_torch_layer_norm_and_closed_forms():
    x = rnd(2, 7, 48, scale=3.0) + 5.0                    # large mean: the centring must be exact
    shift, scale = rnd(2, 48), rnd(2, 48)
    for eps in (1e-6, 0.25):
        ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), eps=eps).numpy()
        ref = ln * (1.0 + scale[:, None, :]) + shift[:, None, :]
        np.testing.assert_allclose(O.adaln_modulate(x, shift, scale, eps), ref, rtol=1e-13, atol=1e-13)
    # zero scale and shift: every row has mean 0 and variance var/(var+eps)
    y = O.adaln_modulate(x, np.zeros((2, 48)), np.zeros((2, 48)), 0.25)
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-13)
    v = x.var(-1)
    np.testing.assert_allclose(y.var(-1), v / (v + 0.25), rtol=1e-12)
    # constant rows normalise to zero, leaving the shift; scale = -1 removes the normalised part
    c = np.full((2, 3, 48), 4.0)
    np.testing.assert_allclose(O.adaln_modulate(c, shift, scale, 1e-6), np.broadcast_to(shift[:, None, :], c.shape), atol=1e-12)
    np.testing.assert_allclose(O.adaln_modulate(x, shift, -np.ones((2, 48)), 1e-6), np.broadcast_to(shift[:, None, :], x.shape), atol=1e-12)
    # invariant to adding a constant to a row, covariant in batch: scale/shift of batch 1 never touch batch 0
    np.testing.assert_allclose(O.adaln_modulate(x + 7.5, shift, scale, 0.0), O.adaln_modulate(x, shift, scale, 0.0), atol=1e-11)
    s2 = shift.copy(); s2[1] += 100
    np.testing.assert_array_equal(O.adaln_modulate(x, s2, scale, 1e-6)[0], O.adaln_modulate(x, shift, scale, 1e-6)[0])


def test_swiglu_matches_torch_silu_and_special_values():
    a, b = rnd(5, 33, scale=4.0), rnd(5, 33)
    ref = (torch.nn.functional.silu(torch.from_numpy(a)) * torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(O.swiglu(a, b), ref, rtol=1e-14, atol=1e-15)
    assert O.swiglu(np.array([0.0]), np.array([3.0]))[0] == 0.0
    np.testing.assert_allclose(O.swiglu(np.array([40.0]), np.array([2.0])), [80.0], rtol=1e-15)
    np.testing.assert_allclose(O.swiglu(np.array([-40.0]), np.array([2.0])), [0.0], atol=1e-15)
    np.testing.assert_allclose(O.swiglu(np.array([1.0]), np.array([1.0])), [1.0 / (1.0 + math.exp(-1.0))], rtol=1e-15)


# ----------------------------------------------------------------------------------- Cache-DiT gate

def test_residual_change_closed_forms():
    a = rnd(1000)
    d, n = O.residual_change(a, a)
    assert d == 0.0 and n == pytest.approx(np.abs(a).sum(), rel=1e-15)
    d, n = O.residual_change(2 * a, a)              # |2a - a| = |a|: relative change exactly 1
    assert d == pytest.approx(n, rel=1e-14)
    d, n = O.residual_change(a + 0.5, np.zeros(1000))
    assert n == 0.0 and d == pytest.approx(np.abs(a + 0.5).sum(), rel=1e-15)
    x = np.array([1.0, -2.0, 3.0]); y = np.array([1.5, -2.0, 2.0])
    assert O.residual_change(x, y) == (1.5, 5.5)


def test_cache_gate_rule():
    # conservative-style: at most one cached step in a row
    g = O.CacheGate(0.1, 1)
    seq = [0.0, 0.01, 0.01, 0.01, 0.5, 0.01, 0.01]
    assert [g.decide(r) for r in seq] == [False, True, False, True, False, True, False]
    # stride-style: up to three in a row, reset by a large change
    g = O.CacheGate(0.2, 3)
    seq = [0.9, 0.1, 0.1, 0.1, 0.1, 0.1, 0.3, 0.1]
    assert [g.decide(r) for r in seq] == [False, True, True, True, False, True, False, True]
    # threshold is strict and 0 consecutive never reuses
    g = O.CacheGate(0.1, 5)
    assert [g.decide(r) for r in [0.0, 0.1, 0.0999]] == [False, False, True]
    g = O.CacheGate(1.0, 0)
    assert not any(g.decide(0.0) for _ in range(4))
    with pytest.raises(ValueError):
        O.CacheGate(-1.0, 1)


# ----------------------------------------------------------------------------------- FP8 (e4m3)

def _nearest_e4m3_by_search(x: float) -> float:
    """Independent rounding: the nearest finite e4m3 value by exhaustive search over the code
    table, ties to the even code (even mantissa), NaN above the largest value's rounding range."""
    vals = O.e4m3_values()
    codes = [c for c in range(256) if np.isfinite(vals[c]) and not (vals[c] == 0 and c == 0x80)]
    best, best_d, best_c = None, None, None
    for c in codes:
        dist = abs(vals[c] - x)
        if best_d is None or dist < best_d or (dist == best_d and (c & 1) == 0 and (best_c & 1) == 1):
            best, best_d, best_c = vals[c], dist, c
    if abs(x) > 464.0:            # nearer to the missing 480 than to 448: no e4m3 value
        return float("nan")
    return math.copysign(abs(best), x) if best == 0 else best


def test_e4m3_table_from_the_format_definition():
    t = O.e4m3_values()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(t).sum() == 254
    # hand-decoded codes: sign | eeee | mmm with bias 7, subnormals m/8 * 2^-6
    hand = {0x00: 0.0, 0x38: 1.0, 0x30: 0.5, 0x3A: 1.25, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6,
            0x08: 2.0 ** -6, 0xB8: -1.0, 0x44: 3.0, 0x79: 288.0, 0x1D: 0.1015625, 0xFE: -448.0}
    for c, v in hand.items():
        assert t[c] == v, hex(c)
    pos = np.sort(t[(t > 0) & np.isfinite(t)])
    assert len(pos) == 126 and pos[0] == 2.0 ** -9 and pos[-1] == O.E4M3_MAX


def test_e4m3_round_against_table_search_and_torch():
    t = O.e4m3_values()
    fin = t[np.isfinite(t)]
    np.testing.assert_array_equal(O.e4m3_round(fin), fin)              # every value is a fixed point
    pos = np.sort(np.unique(fin[fin >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2                                     # exact ties
    probes = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), [464.0, 465.0, 479.0, 480.0]])
    probes = np.concatenate([probes, -probes])
    got = O.e4m3_round(probes)
    want = np.array([_nearest_e4m3_by_search(float(x)) for x in probes])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    # library routine: torch's float8_e4m3fn cast (round to nearest even) inside the finite range
    x = RNG.uniform(-448, 448, 20000) * np.exp2(RNG.integers(-14, 1, 20000))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_round(x.astype(np.float32).astype(np.float64)), ref)


def test_pow2_scale_is_the_smallest_fitting_power_of_two():
    amax = np.concatenate([[0.0, 448.0, 449.0, 1.0, 224.0, 896.0, 897.0], RNG.uniform(1e-6, 1e6, 500)])
    s = O.pow2_scale(amax)
    # the floor: tiny maxima get 2^-60, which still fits them
    np.testing.assert_array_equal(O.pow2_scale(np.array([1e-30, 448 * 2.0 ** -60, 449 * 2.0 ** -60])),
                                  [2.0 ** -60, 2.0 ** -60, 2.0 ** -59])
    for a, sc in zip(amax, s):
        if a == 0:
            assert sc == 1.0
            continue
        e = math.log2(sc)
        assert e == int(e), "power of two"
        assert a <= 448.0 * sc and a > 448.0 * sc / 2, (a, sc)        # fits, and half would not


def test_quantize_blocks_and_channels_error_bounds_and_scale_invariance():
    x = rnd(2, 200, 3, 16, scale=3.0)
    x8, s = O.quantize_blocks(x, 64)
    assert s.shape == (2, 3, 4)
    sfull = np.repeat(s.transpose(0, 2, 1), 64, axis=1)[:, :200][:, :, :, None]     # [B, N, Hd, 1]
    y = x / sfull
    assert np.abs(y).max() <= 448.0
    err = np.abs(x8 - y)
    assert (err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-300).all()    # half an ulp
    assert np.isin(x8, O.e4m3_values()).all()
    x8b, sb = O.quantize_blocks(x * 2.0 ** 5, 64)                                    # exact rescaling
    np.testing.assert_array_equal(x8b, x8)
    np.testing.assert_array_equal(sb, s * 2.0 ** 5)
    v = rnd(1, 150, 2, 8)
    v8, sv = O.quantize_channels(v)
    assert sv.shape == (1, 2, 8)
    assert np.abs(v8 - v / sv[:, None]).max() <= 448 * 2.0 ** -4


def _fp8_brute(q, k, v):
    """The definition with explicit loops over rows and keys, rounding by table search."""
    q8, sq = O.quantize_blocks(q, 64)
    k8, sk = O.quantize_blocks(k, 64)
    v8, sv = O.quantize_channels(v)
    n, d = q.shape[1], q.shape[3]
    out = np.zeros((n, v.shape[3]))
    lse = np.zeros(n)
    for i in range(n):
        xs = []
        for j in range(n):
            dot = sum(q8[0, i, 0, c] * k8[0, j, 0, c] for c in range(d))
            xs.append(dot * sq[0, 0, i // 64] * sk[0, 0, j // 64] * math.log2(math.e) / math.sqrt(d))
        m = math.ceil(max(xs))
        ps = [_nearest_e4m3_by_search(2.0 ** (8.0 + xv - m)) for xv in xs]
        l = sum(ps)
        for c in range(v.shape[3]):
            out[i, c] = sum(ps[j] * v8[0, j, 0, c] for j in range(n)) * sv[0, 0, c] / l
        lse[i] = math.log(2.0) * (m - 8 + math.log2(l))
    return out, lse


def test_attention_fp8_brute_force_and_closed_forms():
    q, k, v = rnd(1, 70, 1, 8), rnd(1, 70, 1, 8), rnd(1, 70, 1, 4)
    o, lse = O.attention_fp8(q, k, v)
    bo, bl = _fp8_brute(q, k, v)
    np.testing.assert_allclose(o[0, :, 0], bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], bl, rtol=1e-12, atol=1e-12)
    # constant value rows (representable after scaling): output equals that value exactly
    vc = np.broadcast_to(np.array([0.75, -1.5, 3.0, 0.0]), (1, 70, 1, 4)).copy()
    oc, _ = O.attention_fp8(q, k, vc)
    np.testing.assert_allclose(oc[0, :, 0], np.broadcast_to(vc[0, 0, 0], (70, 4)), rtol=1e-15)
    # identical keys: equal weights, the output is the mean of the quantised values
    kc = np.broadcast_to(k[:, :1], k.shape).copy()
    oi, li = O.attention_fp8(q, kc, v)
    v8, sv = O.quantize_channels(v)
    np.testing.assert_allclose(oi[0, :, 0], np.broadcast_to((v8[0, :, 0] * sv[0, 0]).mean(0), (70, 4)), rtol=1e-12)
    # the quantised path stays close to exact attention on these inputs
    ex, _ = O.attention(q, k, v)
    assert np.abs(o - ex).max() < 0.15


def test_sparse_attention_fp8_special_cases():
    q, k, v = rnd(1, 192, 2, 16), rnd(1, 192, 2, 16), rnd(1, 192, 2, 8)
    idx_all = np.broadcast_to(np.arange(3), (1, 2, 3, 3)).copy()
    so, sl = O.sparse_attention_fp8(q, k, v, idx_all)
    do, dl = O.attention_fp8(q, k, v)
    np.testing.assert_allclose(so, do, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sl, dl, rtol=1e-12, atol=1e-13)
    # one kept block == dense fp8 attention of that query block over that key block's tokens,
    # with the quantisation (scales) of the full tensors
    idx1 = np.full((1, 2, 3, 1), 2)
    o1, _ = O.sparse_attention_fp8(q, k, v, idx1)
    q8, sq = O.quantize_blocks(q); k8, sk = O.quantize_blocks(k); v8, sv = O.quantize_channels(v)
    x = (q8[0, 64:128, 1] @ k8[0, 128:192, 1].T) * sq[0, 1, 1] * sk[0, 1, 2] * math.log2(math.e) / 4.0
    p = O.e4m3_round(np.exp2(8 + x - np.ceil(x.max(1, keepdims=True))))
    ref = (p @ v8[0, 128:192, 1]) * sv[0, 1] / p.sum(1, keepdims=True)
    np.testing.assert_allclose(o1[0, 64:128, 1], ref, rtol=1e-12)
    # sampled-row helper agrees with the full computation
    r, rl = O.attention_fp8_rows(q, k, v, 0, 1, 2, block_idx=idx_all[0, 1, 2])
    np.testing.assert_allclose(r, do[0, 128:192, 1], rtol=1e-12, atol=1e-13)
    # detail: same outputs; one probability moved to a neighbouring e4m3 code (relative change at
    # most 2^-3 of its value) moves the output by no more than 2^-3 * wmax * dev
    od, ld, wmax, dev = O.attention_fp8_detail(q, k, v)
    np.testing.assert_array_equal(od, do)
    np.testing.assert_array_equal(ld, dl)
    q8, sq = O.quantize_blocks(q); k8, sk = O.quantize_blocks(k); v8, sv = O.quantize_channels(v)
    x = (q8[0, :, 0] @ k8[0, :, 0].T) * np.repeat(sq[0, 0], 64)[:, None] * np.repeat(sk[0, 0], 64)[None, :] \
        * math.log2(math.e) / 4.0
    p = O.e4m3_round(np.exp2(8 + x - np.ceil(x.max(1, keepdims=True))))
    vals = v8[0, :, 0] * sv[0, 0]
    for row in (0, 77, 191):
        j = int(np.argmax(p[row]))
        for factor in (1 - 2.0 ** -4, 1 + 2.0 ** -3):                 # the neighbouring codes of a value
            p2 = p[row].copy(); p2[j] *= factor
            o2 = p2 @ vals / p2.sum()
            assert (np.abs(o2 - od[0, row, 0]) <= 2.0 ** -3 * wmax[0, 0, row] * dev[0, row, 0] + 1e-12).all()
