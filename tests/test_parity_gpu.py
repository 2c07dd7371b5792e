"""GPU parity: every kernel, called through the C ABI (ctypes binding), against the float64
oracle on the same seeded bf16 inputs. Small and ragged cases are compared in full; the three
long-video workloads are compared on every head for a seeded sample of query blocks (each
sampled row's oracle value is exact: a row depends on all keys but on no other row), while
block selection and norm+RoPE are compared on the full tensors."""
import math

import numpy as np
import pytest
import torch

import oracle
from inputs import FRAME, TINY, VIDEO5S, VIDEO10S, VIDEO15S, make_inputs, random_case, sample_query_blocks
from inputs.generate import box_blocks
from tests.parity_util import (ATTN_MAX_ABS, ATTN_MEAN_ABS, FP8_EXACT_MAX_ABS, FP8_EXACT_MAX_REL_RMS,
                               FP8_EXACT_MEAN_ABS, FP8_EXACT_MEAN_REL_RMS, LSE_MAX_ABS, check_attention,
                               check_block_sets, check_norm_rope, f64, log, record)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def h3():
    import video_diffusion_transformer_qk_amd as h3
    h3.load_library()
    return h3


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ full comparisons (small)

def _full_norm_rope(h3, q, k, wq, wk, grid, sections, theta=1e4, eps=1e-6, what="", wl=None):
    qo, ko = h3.qk_norm_rope(q, k, wq, wk, grid, sections, theta, eps)
    _sync()
    rq, rk = oracle.qk_norm_rope(f64(q), f64(k), f64(wq), f64(wk), tuple(grid), tuple(sections), theta,
                                 float(np.float32(eps)))
    for g, r, nm in ((qo, rq, "q"), (ko, rk, "k")):
        worst, exact = check_norm_rope(f64(g), r)
        log(f"{what} norm+rope {nm}: worst {worst:.3f} ulp, exact-RNE fraction {exact:.5f}")
        record(wl or what, "norm+rope", worst_ulp=worst, exact_rne_min=exact)
        assert worst <= 1.0, f"{what} {nm}: {worst} ulp"
        assert exact > 0.99
    return qo, ko


def _full_dense(h3, q, k, v, what="", wl=None):
    o, lse = h3.dense_fwd(q, k, v, return_lse=True)
    _sync()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v))
    mx, mean = check_attention(f64(o), ro, f"{what} dense")
    lerr = float(np.abs(f64(lse) - rl).max())
    record(wl or what, "dense (full)", max_abs=mx, mean_abs=mean, lse_max_abs=lerr)
    assert lerr <= LSE_MAX_ABS
    return o


def _full_select_sparse(h3, q, k, v, sparsity, what="", wl=None):
    idx = h3.subblock_select(q, k, sparsity)
    _sync()
    qd, kd = f64(q), f64(k)
    scores = oracle.block_scores(qd, kd, 64)
    keep = oracle.keep_count(scores.shape[-1], sparsity)
    ref_idx = oracle.topk_blocks(scores, keep)
    assert tuple(idx.shape) == ref_idx.shape
    mism, near = check_block_sets(idx.cpu().numpy(), ref_idx, scores, keep, f"{what} select s={sparsity}")
    record(wl or what, f"select s={sparsity}", rows=int(np.prod(scores.shape[:-1])), mismatched=mism, near_tie_rows=near)
    o, lse = h3.block_sparse_fwd(q, k, v, idx, return_lse=True)
    _sync()
    ro, rl = oracle.sparse_attention(qd, kd, f64(v), idx.cpu().numpy(), 64)
    mx, mean = check_attention(f64(o), ro, f"{what} sparse s={sparsity}")
    lerr = float(np.abs(f64(lse) - rl).max())
    record(wl or what, f"sparse s={sparsity} (full)", max_abs=mx, mean_abs=mean, lse_max_abs=lerr)
    assert lerr <= LSE_MAX_ABS
    return idx, o


def test_tiny_workload_all_stages(h3):
    cfg = TINY
    x = make_inputs(cfg, DEV)
    qo, ko = _full_norm_rope(h3, x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, cfg.theta, cfg.eps, "tiny")
    _full_dense(h3, qo, ko, x["v"], "tiny")
    idx, _ = _full_select_sparse(h3, qo, ko, x["v"], 0.5, "tiny")
    assert idx.shape[-1] == 2


def test_frame_workload_norm_rope(h3):
    cfg = FRAME
    x = make_inputs(cfg, DEV)
    _full_norm_rope(h3, x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, cfg.theta, cfg.eps, "frame")


def test_frame_workload_dense_select_sparse(h3):
    cfg = FRAME
    x = make_inputs(cfg, DEV)
    qo, ko = h3.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, cfg.theta, cfg.eps)
    _full_dense(h3, qo, ko, x["v"], "frame")
    idx, _ = _full_select_sparse(h3, qo, ko, x["v"], 0.75, "frame")
    assert idx.shape[-1] == 16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 63, 200, 333])
def test_ragged_shapes_full(h3, n, d):
    c = random_case(2, n, 3, d, seed=100 + n + d, device=DEV)
    _full_dense(h3, c["q"], c["k"], c["v"], f"ragged n={n} d={d}", wl="ragged")
    for s in (0.0, 0.5, 0.9):
        _full_select_sparse(h3, c["q"], c["k"], c["v"], s, f"ragged n={n} d={d}", wl="ragged")


def test_ragged_norm_rope_grids(h3):
    for grid, d, sec in (((3, 5, 7), 64, (16, 24, 24)), ((2, 3, 11), 128, (32, 48, 48)),
                         ((1, 1, 9), 128, (0, 64, 64)), ((5, 2, 3), 64, (64, 0, 0))):
        n = grid[0] * grid[1] * grid[2]
        c = random_case(2, n, 5, d, seed=7 + n, device=DEV, scale=3.0)
        _full_norm_rope(h3, c["q"], c["k"], c["wq"], c["wk"], grid, sec, 1e4, 1e-6, f"grid {grid}", wl="ragged grids")


def _pooled_matches_separate(h3, q, k, wq, wk, grid, sections, sparsity, what, inplace=False):
    """qk_norm_rope_pool + subblock_select_pooled against qk_norm_rope + subblock_select: the same
    q', k' and the same kept sets, bit for bit (the pooled path sums the same rounded outputs)."""
    qa, ka = h3.qk_norm_rope(q, k, wq, wk, grid, sections)
    ia = h3.subblock_select(qa, ka, sparsity)
    if inplace:
        q2, k2 = q.clone(), k.clone()
        qb, kb, pooled = h3.qk_norm_rope_pool(q2, k2, wq, wk, grid, sections, inplace=True)
        assert qb.data_ptr() == q2.data_ptr() and kb.data_ptr() == k2.data_ptr()
    else:
        qb, kb, pooled = h3.qk_norm_rope_pool(q, k, wq, wk, grid, sections)
    ib = h3.subblock_select_pooled(pooled, sparsity)
    _sync()
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16)), f"{what}: q' differs"
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16)), f"{what}: k' differs"
    assert torch.equal(ia, ib), f"{what}: kept sets differ ({int((ia != ib).sum())} entries)"
    log(f"{what}: pooled norm+rope and selection identical to the separate calls ({tuple(ib.shape)})")


def test_norm_rope_pool_matches_separate_calls(h3):
    cfg = TINY
    x = make_inputs(cfg, DEV)
    _pooled_matches_separate(h3, x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, 0.5, "tiny")
    for grid, d, sec in (((3, 5, 7), 64, (16, 24, 24)), ((2, 3, 11), 128, (32, 48, 48)),
                         ((1, 1, 9), 128, (0, 64, 64)), ((5, 2, 3), 64, (64, 0, 0)), ((4, 8, 9), 128, (32, 48, 48))):
        n = grid[0] * grid[1] * grid[2]
        c = random_case(2, n, 5, d, seed=7 + n, device=DEV, scale=3.0)
        for s in (0.0, 0.5):
            _pooled_matches_separate(h3, c["q"], c["k"], c["wq"], c["wk"], grid, sec, s, f"grid {grid} d={d} s={s}")
    c = random_case(1, 288, 17, 128, seed=5, device=DEV)
    _pooled_matches_separate(h3, c["q"], c["k"], c["wq"], c["wk"], (2, 12, 12), (32, 48, 48), 0.75,
                             "17 heads, in place", inplace=True)
    cfg = FRAME
    x = make_inputs(cfg, DEV)
    _pooled_matches_separate(h3, x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, 0.75, "frame")


@pytest.mark.timeout(600)
def test_norm_rope_pool_matches_separate_calls_video10s(h3):
    cfg = VIDEO10S
    x = make_inputs(cfg, DEV)
    _pooled_matches_separate(h3, x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, 0.75, "10s")


def test_norm_rope_inplace_matches_out_of_place(h3):
    c = random_case(1, 96, 4, 128, seed=3, device=DEV)
    a, b = h3.qk_norm_rope(c["q"], c["k"], c["wq"], c["wk"], (2, 6, 8), (32, 48, 48))
    q2, k2 = c["q"].clone(), c["k"].clone()
    h3.qk_norm_rope(q2, k2, c["wq"], c["wk"], (2, 6, 8), (32, 48, 48), inplace=True)
    _sync()
    assert torch.equal(a, q2) and torch.equal(b, k2)


def test_keep_all_sparse_is_bitwise_dense(h3):
    c = random_case(1, 64 * 9, 2, 128, seed=11, device=DEV)
    nb = 9
    idx = torch.arange(nb, dtype=torch.int32, device=DEV).repeat(1, 2, nb, 1).contiguous()
    dense = h3.dense_fwd(c["q"], c["k"], c["v"])
    sparse = h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx)
    sel = h3.subblock_select(c["q"], c["k"], 0.0)
    _sync()
    assert torch.equal(sel.cpu(), idx.cpu())
    assert torch.equal(dense, sparse)


def test_sparse_index_order_irrelevant(h3):
    c = random_case(1, 64 * 8, 2, 64, seed=12, device=DEV)
    idx = h3.subblock_select(c["q"], c["k"], 0.5)
    rev = idx.flip(-1).contiguous()
    a = h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx)
    b = h3.block_sparse_fwd(c["q"], c["k"], c["v"], rev)
    _sync()
    # kept blocks are visited in ascending key order whatever their order in the row
    assert torch.equal(a, b), "reversed index order changed the result"


@pytest.mark.parametrize("b,n,d,strides", [(1, 64 * 37 - 5, 64, (2, 3, 9, 36, 37)), (1, 64 * 37 - 5, 128, (4, 10, 37)),
                                           (1, 64 * 9, 128, (2, 9)), (1, 64 * 4098 - 3, 64, (63, 4000)),
                                           (2, 64 * 37 - 5, 128, (9, 37))])
def test_group_stride_is_bitwise_neutral(h3, b, n, d, strides):
    """Which four query blocks share a sparse workgroup (i..i+3, or i, i+S, i+2S, i+3S) changes
    the schedule only: top-k, CSR (with empty rows) and fp8 outputs and lse are bit-identical for
    every stride, including strides that do not divide the block count and S = nB."""
    c = random_case(b, n, 2, d, seed=5000 + n + d + b, device=DEV)
    nb = -(-n // 64)
    idx = h3.subblock_select(c["q"], c["k"], 0.5 if nb < 100 else 0.99)
    keep = idx.shape[-1]
    rows = b * 2 * nb
    counts = (torch.arange(rows) * 7) % (keep + 1)             # 0..keep kept blocks per row
    rp = torch.zeros(rows + 1, dtype=torch.int64)
    rp[1:] = torch.cumsum(counts, 0)
    ih = idx.cpu().reshape(rows, keep)
    ci = torch.cat([ih[r, :counts[r]] for r in range(rows)]).to(torch.int32)
    rp, ci = rp.to(DEV), ci.contiguous().to(DEV)
    fq = h3.fp8_quantize(c["q"], c["k"], c["v"])

    def run(stride):
        return (h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx, return_lse=True, group_stride=stride),
                h3.block_sparse_csr_fwd(c["q"], c["k"], c["v"], rp, ci, return_lse=True, group_stride=stride),
                h3.fp8_block_sparse_fwd(fq, idx, return_lse=True, group_stride=stride))

    base = run(1)
    _sync()
    assert bool((base[1][1][0, 0, :64] == -math.inf).all()), "row 0 of the CSR case keeps no block"
    for stride in strides:
        got = run(stride)
        _sync()
        for (o, lse), (o1, lse1), nm in zip(got, base, ("top-k", "csr", "fp8")):
            assert torch.equal(o, o1) and torch.equal(lse, lse1), f"{nm} b={b} n={n} d={d}: stride {stride} changed the result"


def test_sparse_union_across_windows_and_ragged_groups(h3):
    """More key blocks than one union window (4096) and a block count that is not a multiple of
    the 4 query blocks a workgroup takes: sampled query blocks against the oracle, the CSR form
    and a shuffled index order bit for bit."""
    nb = 4098                                   # two union windows, last group of 2 blocks
    n = nb * 64 - 17                            # partial last key block
    c = random_case(1, n, 1, 64, seed=4242, device=DEV)
    idx = h3.subblock_select(c["q"], c["k"], 0.99)
    keep = idx.shape[-1]
    o, lse = h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx, return_lse=True)
    perm = torch.argsort(torch.rand(idx.shape, generator=torch.Generator(device=DEV).manual_seed(7), device=DEV), dim=-1)
    shuffled = torch.gather(idx, -1, perm).contiguous()
    o2 = h3.block_sparse_fwd(c["q"], c["k"], c["v"], shuffled)
    rp = torch.arange(0, nb + 1, dtype=torch.int64, device=DEV) * keep
    o3 = h3.block_sparse_csr_fwd(c["q"], c["k"], c["v"], rp, shuffled.reshape(-1).contiguous())
    _sync()
    assert torch.equal(o, o2) and torch.equal(o, o3)
    ih = idx.cpu().numpy()
    assert (ih < 4096).any() and (ih >= 4096).any(), "kept sets should span both windows"
    qh, kh, vh, oh, lh = c["q"].cpu(), c["k"].cpu(), c["v"].cpu(), o.cpu(), lse.cpu()
    for i in sample_query_blocks(nb, 12, seed=99, extra=(nb - 2, nb - 3, 4095, 4096)):
        rows = np.arange(i * 64, min((i + 1) * 64, n))
        keys = oracle.block_token_ids(ih[0, 0, i], 64, n)
        ref, rl = oracle.attention_head(f64(qh[0, rows, 0]), f64(kh[0, keys, 0]), f64(vh[0, keys, 0]))
        check_attention(f64(oh[0, rows, 0]), ref, f"two-window sparse block {i}")
        assert np.abs(f64(lh[0, 0, rows]) - rl).max() <= LSE_MAX_ABS


def test_select_ties_resolve_to_lower_index(h3):
    # all-zero queries: every score is 0 -> the kept set is the lowest `keep` indices
    c = random_case(1, 64 * 10, 2, 128, seed=13, device=DEV)
    q0 = torch.zeros_like(c["q"])
    idx = h3.subblock_select(q0, c["k"], 0.7)
    _sync()
    keep = oracle.keep_count(10, 0.7)
    assert keep == 3
    assert (idx.cpu().numpy() == np.arange(keep)).all()
    # duplicated key blocks: block 7 equals block 2, so whenever 7 is kept, 2 is kept too
    k = c["k"].clone()
    k[:, 7 * 64:8 * 64] = k[:, 2 * 64:3 * 64]
    idx = h3.subblock_select(c["q"], k, 0.6)
    _sync()
    for row in idx.reshape(-1, idx.shape[-1]).cpu().numpy().tolist():
        if 7 in row:
            assert 2 in row


@pytest.mark.parametrize("nb", [100, 300])
def test_select_rows_of_equal_scores(h3, nb):
    """Every key block equal: every score of a row ties, so the kept set is the lowest `keep`
    indices. With 100 blocks the row's entries all fall in one bracket and are decided on their
    float64 scores; with 300 the bracket cannot be narrowed and the row goes to the exact radix
    fallback. Both must give the same answer as the oracle's stable sort."""
    c = random_case(1, 64 * nb, 3, 128, seed=31 + nb, device=DEV)
    k = c["k"][:, :64].repeat(1, nb, 1, 1).contiguous()
    idx = h3.subblock_select(c["q"], k, 0.5)
    _sync()
    keep = oracle.keep_count(nb, 0.5)
    got = idx.cpu().numpy().reshape(-1, keep)
    assert (got == np.arange(keep)).all(), f"{nb} equal blocks: first bad row {np.nonzero((got != np.arange(keep)).any(1))[0][:3]}"
    scores = oracle.block_scores(f64(c["q"]), f64(k), 64)
    np.testing.assert_array_equal(got, oracle.topk_blocks(scores, keep).reshape(-1, keep))
    record("equal scores", f"select nB={nb}", rows=got.shape[0], mismatched=0)


def test_select_scores_apart_by_far_less_than_the_bound(h3):
    """Key blocks that differ only in one channel of one token, by (j + 1) 2^-20: the block scores
    of a row differ by about 1e-8 of their size, far inside the error bound of the integer-digit
    scores and far above float64 rounding, so every entry is decided on its float64 score. The
    kept sets must equal the oracle's bit for bit (no near-tie allowance is used here)."""
    nb, d = 40, 128
    c = random_case(1, 64 * nb, 4, d, seed=77, device=DEV)
    k = c["k"][:, :64].repeat(1, nb, 1, 1).float()
    for j in range(nb):
        k[:, 64 * j, :, 0] = (j + 1) * 2.0 ** -20
    k = k.to(torch.bfloat16).contiguous()
    for s in (0.5, 0.8):
        idx = h3.subblock_select(c["q"], k, s)
        _sync()
        keep = oracle.keep_count(nb, s)
        scores = oracle.block_scores(f64(c["q"]), f64(k), 64)
        ref = oracle.topk_blocks(scores, keep)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref)
        # the construction really is ordered by j: the kept blocks are the highest or the lowest
        q0 = oracle.block_means(f64(c["q"]), 64)[..., 0].reshape(-1)
        rows = ref.reshape(-1, keep)
        assert all((r == np.arange(nb - keep, nb)).all() if q > 0 else (r == np.arange(keep)).all()
                   for r, q in zip(rows, q0) if q != 0)
        record("near-equal scores", f"select s={s}", rows=rows.shape[0], mismatched=0)


def test_python_layer_rejects_bad_inputs(h3):
    c = random_case(1, 64, 2, 64, seed=1, device=DEV)
    with pytest.raises(TypeError):
        h3.dense_fwd(c["q"].float(), c["k"], c["v"])
    with pytest.raises(ValueError):
        h3.dense_fwd(c["q"].transpose(1, 2), c["k"], c["v"])
    with pytest.raises(h3.H3AttnError):
        c2 = random_case(1, 64, 2, 96, seed=1, device=DEV)
        h3.dense_fwd(c2["q"], c2["k"], c2["v"])
    with pytest.raises(ValueError):
        h3.qk_norm_rope(c["q"], c["k"], c["wq"], c["wk"], (2, 2, 2), (16, 24, 24))
    # outputs and weights of the wrong size or on the host are refused before any launch (the
    # kernels would write or read past them)
    grid, sec = (1, 8, 8), (16, 24, 24)
    with pytest.raises(ValueError):
        h3.qk_norm_rope(c["q"], c["k"], c["wq"][:32].contiguous(), c["wk"], grid, sec)
    with pytest.raises(ValueError):
        h3.qk_norm_rope(c["q"], c["k"], c["wq"], c["wk"], grid, sec, out=(torch.empty_like(c["q"][:, :32]),
                                                                           torch.empty_like(c["k"])))
    with pytest.raises(ValueError):
        h3.dense_fwd(c["q"], c["k"], c["v"], out=torch.empty_like(c["q"][:, :32]))
    with pytest.raises(ValueError):
        h3.dense_fwd(c["q"], c["k"], c["v"], out=torch.empty(tuple(c["q"].shape), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        h3.subblock_select(c["q"], c["k"], 0.5, out=torch.empty((1, 2, 1, 2), dtype=torch.int32, device=DEV))
    idx = h3.subblock_select(c["q"], c["k"], 0.0)
    with pytest.raises(ValueError):
        h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx, out=torch.empty_like(c["q"][:, :, :1]))
    with pytest.raises((ValueError, TypeError)):
        h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx.cpu())
    x = torch.randn((1, 4, 64), device=DEV).to(torch.bfloat16)
    sh = torch.zeros((1, 64), device=DEV)
    with pytest.raises(ValueError):
        h3.adaln_modulate(x, sh, sh, out=torch.empty_like(x[:, :2]))
    with pytest.raises(ValueError):
        h3.swiglu(x, x, out=torch.empty_like(x[:, :2]))
    with pytest.raises(ValueError):
        h3.residual_change(x, x, out=torch.empty((3,), dtype=torch.float64, device=DEV))
    _sync()


# ------------------------------------------------------------------ long-video workloads (sampled)

def _sampled_dense(h3, q, k, v, qblocks_per_head, what):
    """Dense output and LSE of every sampled query block against the oracle (each sampled row is
    exact: it depends on all keys and on no other row)."""
    o, lse = h3.dense_fwd(q, k, v, return_lse=True)
    _sync()
    qh, kh, vh, oh, lh = q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu()
    worst, lworst, means = 0.0, 0.0, []
    for h, blocks in qblocks_per_head.items():
        rows = np.concatenate([np.arange(i * 64, min((i + 1) * 64, q.shape[1])) for i in blocks])
        ref, rl = oracle.attention_head(f64(qh[0, rows, h]), f64(kh[0, :, h]), f64(vh[0, :, h]))
        mx, mean = check_attention(f64(oh[0, rows, h]), ref, f"{what} dense head {h} ({len(blocks)} blocks)")
        lerr = float(np.abs(f64(lh[0, h, rows]) - rl).max())
        assert lerr <= LSE_MAX_ABS, f"{what} dense head {h}: lse error {lerr}"
        worst, lworst = max(worst, mx), max(lworst, lerr)
        means.append(mean)
    nblk = sum(len(b) for b in qblocks_per_head.values())
    record(what, "dense (sampled)", blocks=nblk, max_abs=worst, mean_abs=float(np.mean(means)), lse_max_abs=lworst)
    return worst


def _full_select_sampled_sparse(h3, q, k, v, sparsity, qblocks_per_head, what, head_chunk=4, group_stride=1):
    """Kept sets of every row against the oracle, then block-sparse output and LSE of the sampled
    query blocks over their kept key blocks."""
    idx = h3.subblock_select(q, k, sparsity)
    o, lse = h3.block_sparse_fwd(q, k, v, idx, group_stride=group_stride, return_lse=True)
    if group_stride != 1:
        o1 = h3.block_sparse_fwd(q, k, v, idx)
        _sync()
        assert torch.equal(o, o1), f"{what}: group stride {group_stride} changed the result"
        del o1
    _sync()
    qh, kh, vh, oh, lh, ih = q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu(), idx.cpu().numpy()
    heads = q.shape[2]
    nb = idx.shape[2]
    keep = idx.shape[3]
    assert keep == oracle.keep_count(nb, sparsity)
    for h0 in range(0, heads, head_chunk):
        sl = slice(h0, min(heads, h0 + head_chunk))
        scores = oracle.block_scores(f64(qh[:, :, sl]), f64(kh[:, :, sl]), 64)
        ref_idx = oracle.topk_blocks(scores, keep)
        mism, near = check_block_sets(ih[:, sl], ref_idx, scores, keep, f"{what} select s={sparsity} heads {h0}..")
        record(what, f"select s={sparsity}", rows=int(np.prod(scores.shape[:-1])), mismatched=mism,
               near_tie_rows=near)
    worst, lworst, means, nblk = 0.0, 0.0, [], 0
    for h, blocks in qblocks_per_head.items():
        for i in blocks:
            rows = np.arange(i * 64, min((i + 1) * 64, q.shape[1]))
            keys = oracle.block_token_ids(ih[0, h, i], 64, q.shape[1])
            ref, rl = oracle.attention_head(f64(qh[0, rows, h]), f64(kh[0, keys, h]), f64(vh[0, keys, h]))
            mx, mean = check_attention(f64(oh[0, rows, h]), ref, f"{what} sparse s={sparsity} head {h} block {i}")
            lerr = float(np.abs(f64(lh[0, h, rows]) - rl).max())
            assert lerr <= LSE_MAX_ABS, f"{what} sparse head {h} block {i}: lse error {lerr}"
            worst, lworst = max(worst, mx), max(lworst, lerr)
            means.append(mean)
            nblk += 1
    record(what, f"sparse s={sparsity} (sampled)", blocks=nblk, max_abs=worst, mean_abs=float(np.mean(means)),
           lse_max_abs=lworst)


def _samples(cfg, per_head, extra=()):
    return {h: sample_query_blocks(cfg.n_blocks, per_head, seed=1000 * cfg.id + h, extra=extra)
            for h in range(cfg.heads)}


@pytest.mark.timeout(900)
def test_video5s_dense_sampled(h3):
    cfg = VIDEO5S
    x = make_inputs(cfg, DEV)
    _sampled_dense(h3, x["q"], x["k"], x["v"], _samples(cfg, 32), "5s")


@pytest.mark.timeout(900)
def test_video5s_select_and_sparse(h3):
    cfg = VIDEO5S
    x = make_inputs(cfg, DEV)
    _full_select_sampled_sparse(h3, x["q"], x["k"], x["v"], 0.75, _samples(cfg, 32), "5s", head_chunk=8,
                                group_stride=h3.frame_group_stride(cfg.grid))


@pytest.mark.timeout(900)
def test_video10s_norm_rope_full(h3):
    cfg = VIDEO10S
    x = make_inputs(cfg, DEV)
    qo, ko = h3.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, cfg.theta, cfg.eps)
    _sync()
    qh, kh, qoh, koh = x["q"].cpu(), x["k"].cpu(), qo.cpu(), ko.cpu()
    wq, wk = f64(x["wq"]), f64(x["wk"])
    eps = float(np.float32(cfg.eps))
    for h0 in range(0, cfg.heads, 2):
        sl = slice(h0, h0 + 2)
        rq, rk = oracle.qk_norm_rope(f64(qh[:, :, sl]), f64(kh[:, :, sl]), wq, wk, cfg.grid, cfg.sections, cfg.theta, eps)
        for g, r, nm in ((qoh[:, :, sl], rq, "q"), (koh[:, :, sl], rk, "k")):
            worst, exact = check_norm_rope(f64(g), r)
            log(f"10s norm+rope {nm} heads {h0}..{h0 + 1}: worst {worst:.3f} ulp, exact {exact:.5f}")
            record("10s", "norm+rope", worst_ulp=worst, exact_rne_min=exact)
            assert worst <= 1.0 and exact > 0.99


@pytest.mark.timeout(900)
def test_video10s_dense_select_sparse(h3):
    cfg = VIDEO10S
    x = make_inputs(cfg, DEV)
    qo, ko = h3.qk_norm_rope(x["q"], x["k"], x["wq"], x["wk"], cfg.grid, cfg.sections, cfg.theta, cfg.eps)
    _sampled_dense(h3, qo, ko, x["v"], _samples(cfg, 32), "10s")
    for s in cfg.sparsities:
        _full_select_sampled_sparse(h3, qo, ko, x["v"], s, _samples(cfg, 32), "10s",
                                    group_stride=h3.frame_group_stride(cfg.grid))


@pytest.mark.timeout(900)
def test_video15s_boxes_select_sparse_dense(h3):
    cfg = VIDEO15S
    x = make_inputs(cfg, DEV)
    bb = box_blocks(cfg.grid, x["boxes"])
    extra = [bb[0], bb[len(bb) // 2], bb[-1]]
    smp = _samples(cfg, 32, extra=extra)
    _full_select_sampled_sparse(h3, x["q"], x["k"], x["v"], 0.75, smp, "15s",
                                group_stride=h3.frame_group_stride(cfg.grid))
    _sampled_dense(h3, x["q"], x["k"], x["v"], smp, "15s")


# ------------------------------------------------------------------ threshold mode (CSR)

def _tau_for(scores, keep_frac=0.25):
    """A tau that keeps roughly keep_frac of the blocks (median over rows of the gap between the
    row maximum and the row's keep_frac quantile), computed from the oracle's scores."""
    flat = scores.reshape(-1, scores.shape[-1])
    gap = flat.max(1) - np.quantile(flat, 1.0 - keep_frac, axis=1)
    return float(np.median(gap))


def _check_threshold_sets(rp, ci, scores, tau, what):
    flat = scores.reshape(-1, scores.shape[-1])
    r, nb = flat.shape
    rp = rp.cpu().numpy()
    ci = ci.cpu().numpy()
    assert rp.shape == (r + 1,) and rp[0] == 0 and rp[-1] == ci.size
    g = np.zeros((r, nb), dtype=bool)
    for i in range(r):
        row = ci[rp[i]:rp[i + 1]]
        assert (row >= 0).all() and (row < nb).all()
        if row.size > 1:
            assert (np.diff(row) > 0).all(), f"{what}: row {i} not ascending"
        g[i, row] = True
    rrp, rci = oracle.threshold_blocks(scores, tau)
    ref = np.zeros((r, nb), dtype=bool)
    for i in range(r):
        ref[i, rci[rrp[i]:rrp[i + 1]]] = True
    diff = g != ref
    near = oracle.near_threshold_entries(flat, tau)
    log(f"{what}: tau {tau:.4g}, kept {g.sum()} of {g.size} ({g.mean():.3f}), differing {int(diff.sum())} "
        f"(near-threshold {int((diff & near).sum())})")
    record(what.split()[0], "threshold select", entries=int(g.size), kept=int(g.sum()), differing=int(diff.sum()),
           near_threshold_entries=int(near.sum()))
    assert not (diff & ~near).any(), f"{what}: {int((diff & ~near).sum())} entries differ away from the threshold"


@pytest.mark.parametrize("n,d", [(256, 64), (333, 128), (64 * 20, 128)])
def test_threshold_select_and_csr_attention_full(h3, n, d):
    c = random_case(2, n, 3, d, seed=500 + n, device=DEV)
    qd, kd, vd = f64(c["q"]), f64(c["k"]), f64(c["v"])
    scores = oracle.block_scores(qd, kd, 64)
    for tau in (0.0, _tau_for(scores), float("inf")):
        rp, ci = h3.subblock_select_threshold(c["q"], c["k"], tau)
        _sync()
        _check_threshold_sets(rp, ci, scores, tau, f"threshold n={n} d={d}")
        o, lse = h3.block_sparse_csr_fwd(c["q"], c["k"], c["v"], rp, ci, return_lse=True)
        _sync()
        ro, rl = oracle.sparse_attention_csr(qd, kd, vd, rp.cpu().numpy(), ci.cpu().numpy(), 64)
        check_attention(f64(o), ro, f"csr sparse n={n} d={d} tau={tau:.3g}")
        assert np.abs(f64(lse) - rl).max() <= LSE_MAX_ABS


def test_kept_set_check_flags_exactly_the_bad_rows(h3):
    """Top-k and CSR kept sets from the selection kernels are valid; planted bad rows (an index out
    of range, a repeated index, a decreasing or overlong CSR range) are flagged with their reason
    and nothing else is. With validate=True the attention calls raise before any launch."""
    b, n, h, d = 1, 64 * 10, 2, 64
    nb = 10
    c = random_case(b, n, h, d, seed=77, device=DEV)
    idx = h3.subblock_select(c["q"], c["k"], 0.5)
    fl = h3.check_block_idx(idx)
    _sync()
    assert fl.shape == (b, h, nb) and int(fl.count_nonzero()) == 0
    bad = idx.clone()
    bad[0, 1, 3, 0] = nb          # out of range
    bad[0, 0, 2, 1] = bad[0, 0, 2, 0]  # repeated
    bad[0, 1, 7, 2] = -1          # out of range
    bad[0, 0, 9, 0] = nb + 5
    bad[0, 0, 9, 1] = bad[0, 0, 9, 2]  # both reasons in one row
    fl = h3.check_block_idx(bad).cpu()
    want = torch.zeros((b, h, nb), dtype=torch.uint8)
    want[0, 1, 3] = 1
    want[0, 0, 2] = 2
    want[0, 1, 7] = 1
    want[0, 0, 9] = 3
    assert torch.equal(fl, want), fl
    with pytest.raises(h3.H3AttnError):
        h3.block_sparse_fwd(c["q"], c["k"], c["v"], bad, validate=True)
    h3.block_sparse_fwd(c["q"], c["k"], c["v"], idx, validate=True)  # valid: runs
    fq = h3.fp8_quantize(c["q"], c["k"], c["v"])
    with pytest.raises(h3.H3AttnError):
        h3.fp8_block_sparse_fwd(fq, bad, validate=True)
    h3.fp8_block_sparse_fwd(fq, idx, validate=True)
    # CSR: threshold-mode rows are valid
    rp, ci = h3.subblock_select_threshold(c["q"], c["k"], 0.3)
    assert int(h3.check_csr(rp, ci, b, h, nb).count_nonzero()) == 0
    # hand-built rows over b = 1, h = 2, nB = 4 (8 rows), col_idx capacity 9
    rows = [[1, 3], [], [0, 0, 2], [3], [0, 4], [2, 1, 0], [], [1]]
    ptr = [0]
    for r in rows:
        ptr.append(ptr[-1] + len(r))
    rp2 = torch.tensor(ptr, dtype=torch.int64)
    ci2 = torch.tensor([x for r in rows for x in r], dtype=torch.int32)
    rp2[7] = 20                   # row 6 runs past col_idx (capacity 9), row 7 ends below its start
    fl = h3.check_csr(rp2.to(DEV), ci2.to(DEV), 1, 2, 4).cpu()
    assert fl.tolist() == [0, 0, 2, 0, 1, 0, 4, 4], fl.tolist()
    x = random_case(1, 256, 2, 64, seed=78, device=DEV)
    with pytest.raises(h3.H3AttnError):
        h3.block_sparse_csr_fwd(x["q"], x["k"], x["v"], rp2.to(DEV), ci2.to(DEV), validate=True)
    log("kept-set checks: valid sets pass, every planted bad row flagged with its reason")


@pytest.mark.timeout(600)
def test_select_threshold_and_sparse_at_the_row_limit(h3):
    """nB = 19968 (1,277,952 tokens, one head): the longest row of float64 scores that the top-k and
    threshold-fill kernels hold in one CU's LDS, the largest nB the selection accepts. The oracle's
    scores for sampled query blocks: kept sets bit-exact (near ties excepted), threshold rows, and
    block-sparse attention over the kept set."""
    nb = 19968
    n = nb * 64
    c = random_case(1, n, 1, 64, seed=905, device=DEV)
    q, k, v = c["q"], c["k"], c["v"]
    keep = oracle.keep_count(nb, 0.75)
    idx = h3.subblock_select(q, k, 0.75)
    o = h3.block_sparse_fwd(q, k, v, idx)
    _sync()
    assert int(h3.check_block_idx(idx).count_nonzero()) == 0
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    rows = sample_query_blocks(nb, 24, seed=906, extra=(0, nb - 1))
    scores = oracle.block_scores(f64(qh), f64(kh), 64)[:, :, rows]   # [1, 1, R, nB]
    ih = idx.cpu().numpy()
    check_block_sets(ih[:, :, rows], oracle.topk_blocks(scores, keep), scores, keep, "row-limit select s=0.75")
    oh = o.cpu()
    for i in rows[:6]:
        rr = np.arange(i * 64, (i + 1) * 64)
        keys = oracle.block_token_ids(ih[0, 0, i], 64, n)
        ref, _ = oracle.attention_head(f64(qh[0, rr, 0]), f64(kh[0, keys, 0]), f64(vh[0, keys, 0]))
        check_attention(f64(oh[0, rr, 0]), ref, f"row-limit sparse block {i}")
    del o, idx
    tau = _tau_for(scores, 0.05)
    rp, ci = h3.subblock_select_threshold(q, k, tau)
    _sync()
    assert int(h3.check_csr(rp, ci, 1, 1, nb).count_nonzero()) == 0
    rpn, cin = rp.cpu().numpy(), ci.cpu().numpy()
    sub_rp, sub_ci = [0], []
    for r in rows:
        seg = cin[rpn[r]:rpn[r + 1]]
        sub_ci.append(seg)
        sub_rp.append(sub_rp[-1] + seg.size)
    _check_threshold_sets(torch.tensor(sub_rp, dtype=torch.int64), torch.from_numpy(np.concatenate(sub_ci)), scores,
                          tau, "row-limit threshold")


def test_csr_keep_all_is_bitwise_dense_and_empty_rows(h3):
    c = random_case(1, 64 * 6, 2, 128, seed=21, device=DEV)
    rp, ci = h3.subblock_select_threshold(c["q"], c["k"], float("inf"))
    dense = h3.dense_fwd(c["q"], c["k"], c["v"])
    csr = h3.block_sparse_csr_fwd(c["q"], c["k"], c["v"], rp, ci)
    _sync()
    assert torch.equal(dense, csr)
    # an empty kept set yields zeros and lse = -inf; the other rows are unaffected
    rp2 = rp.clone()
    rp2[1:] -= 6          # row 0 empty; rows 1.. shifted onto col_idx[0..]
    rp2[0] = 0
    ci2 = ci[6:].contiguous()
    o, lse = h3.block_sparse_csr_fwd(c["q"], c["k"], c["v"], rp2, ci2, return_lse=True)
    _sync()
    assert (o[0, :64, 0].float() == 0).all() and torch.isinf(lse[0, 0, :64]).all()
    assert torch.equal(o[0, 64:, 0], dense[0, 64:, 0]) and torch.equal(o[0, :, 1], dense[0, :, 1])


@pytest.mark.timeout(900)
def test_video5s_threshold_select_and_csr_sparse(h3):
    cfg = VIDEO5S
    x = make_inputs(cfg, DEV)
    q, k, v = x["q"], x["k"], x["v"]
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    scores = np.concatenate([oracle.block_scores(f64(qh[:, :, h0:h0 + 8]), f64(kh[:, :, h0:h0 + 8]), 64)
                             for h0 in range(0, cfg.heads, 8)], axis=1)
    tau = _tau_for(scores)
    rp, ci = h3.subblock_select_threshold(q, k, tau)
    o = h3.block_sparse_csr_fwd(q, k, v, rp, ci, group_stride=h3.frame_group_stride(cfg.grid))
    o1 = h3.block_sparse_csr_fwd(q, k, v, rp, ci)
    _sync()
    assert torch.equal(o, o1), "5s csr: frame group stride changed the result"
    del o1
    _check_threshold_sets(rp, ci, scores, tau, "5s threshold")
    rpn, cin, oh = rp.cpu().numpy(), ci.cpu().numpy(), o.cpu()
    nb = cfg.n_blocks
    for h, blocks in _samples(cfg, 2).items():
        for i in blocks:
            r = h * nb + i
            rows = np.arange(i * 64, (i + 1) * 64)
            keys = oracle.block_token_ids(cin[rpn[r]:rpn[r + 1]], 64, cfg.n_tokens)
            ref, _ = oracle.attention_head(f64(qh[0, rows, h]), f64(kh[0, keys, h]), f64(vh[0, keys, h]))
            check_attention(f64(oh[0, rows, h]), ref, f"5s csr sparse head {h} block {i}")


# ------------------------------------------------------------------ AdaLN and SwiGLU

def _check_elementwise(gpu, ref, floor, what):
    from tests.parity_util import bf16_ulp
    tol = np.maximum(bf16_ulp(ref), floor)
    worst = float(np.max(np.abs(gpu - ref) / tol))
    rne = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    exact = float(np.mean(gpu == rne))
    log(f"{what}: worst {worst:.3f} ulp, exact-RNE fraction {exact:.5f}")
    assert worst <= 1.0 and exact > 0.99, what


@pytest.mark.parametrize("b,n,c", [(2, 333, 6144), (1, 64, 96), (3, 17, 16384), (1, 1, 8), (1, 5, 8192), (2, 3, 12000)])
def test_adaln_modulate_full(h3, b, n, c):
    g = torch.Generator(device=DEV).manual_seed(b * 1000 + n + c)
    x = (torch.randn((b, n, c), generator=g, device=DEV) * 2.0 + 3.0).to(torch.bfloat16)
    shift = torch.randn((b, c), generator=g, device=DEV)
    scale = torch.randn((b, c), generator=g, device=DEV) * 0.5
    y = h3.adaln_modulate(x, shift, scale, 1e-6)
    _sync()
    xd, sh, scd = f64(x), f64(shift), f64(scale)
    ref = oracle.adaln_modulate(xd, sh, scd, float(np.float32(1e-6)))
    xn = oracle.adaln_modulate(xd, np.zeros_like(sh), np.zeros_like(scd), float(np.float32(1e-6)))
    floor = 2.0 ** -14 * (np.abs(xn * (1 + scd[:, None, :])) + np.abs(sh[:, None, :]))
    _check_elementwise(f64(y), ref, floor, f"adaln {b}x{n}x{c}")
    y2 = x.clone()
    h3.adaln_modulate(y2, shift, scale, 1e-6, out=y2)
    _sync()
    assert torch.equal(y2, y)


def test_swiglu_full_separate_and_fused_layout(h3):
    g = torch.Generator(device=DEV).manual_seed(77)
    a = (torch.randn((3, 129, 4096), generator=g, device=DEV) * 3).to(torch.bfloat16)
    u = torch.randn((3, 129, 4096), generator=g, device=DEV).to(torch.bfloat16)
    y = h3.swiglu(a, u)
    _sync()
    ref = oracle.swiglu(f64(a), f64(u))
    _check_elementwise(f64(y), ref, 1e-30, "swiglu separate")
    both = torch.cat([a, u], dim=-1).contiguous()         # one [.., 2F] tensor: gate half, up half
    y2 = h3.swiglu(both[..., :4096], both[..., 4096:])
    _sync()
    assert torch.equal(y2, y)
    tiny = h3.swiglu(a[0, :1, :8].contiguous(), u[0, :1, :8].contiguous())
    _sync()
    _check_elementwise(f64(tiny), oracle.swiglu(f64(a[0, :1, :8]), f64(u[0, :1, :8])), 1e-30, "swiglu 8")


# ------------------------------------------------------------------ Cache-DiT residual gate

@pytest.mark.parametrize("n", [1, 7, 8, 1000, 65536 + 3, 2 * 8192 * 8 * 5 + 11])
def test_residual_change_matches_oracle(h3, n):
    g = torch.Generator(device=DEV).manual_seed(n)
    prev = torch.randn((n,), generator=g, device=DEV).to(torch.bfloat16)
    cur = (prev.float() + 0.05 * torch.randn((n,), generator=g, device=DEV)).to(torch.bfloat16)
    res = h3.residual_change(cur, prev)
    _sync()
    d, p = res.tolist()
    rd, rp = oracle.residual_change(f64(cur), f64(prev))
    assert abs(d - rd) <= 1e-6 * max(rd, 1e-30) + 1e-12 and abs(p - rp) <= 1e-6 * rp
    res2 = h3.residual_change(cur, prev)
    _sync()
    assert res2.tolist() == [d, p]        # fixed reduction order: bitwise repeatable
    same = h3.residual_change(prev, prev)
    _sync()
    assert same[0].item() == 0.0


def test_cache_gate_drives_a_step_sequence(h3):
    """The library gate on GPU-measured changes makes the same decisions as the oracle rule on
    oracle-measured changes (sequence built so no change sits near the threshold)."""
    g = torch.Generator(device=DEV).manual_seed(3)
    base = torch.randn((4, 256, 512), generator=g, device=DEV)
    scales = [0.0, 0.01, 0.01, 0.3, 0.01, 0.01, 0.01, 0.01, 0.5, 0.02]
    states, prev = [], base
    for s in scales:
        cur = prev + s * torch.randn(prev.shape, generator=g, device=DEV)
        states.append(cur.to(torch.bfloat16))
        prev = cur
    for mc in (1, 3):
        gate = h3.CacheGate(0.1, mc)
        ref = oracle.CacheGate(0.1, mc)
        for i, st in enumerate(states):
            got = gate.step(st, states[i - 1] if i > 0 else None)
            if i == 0:
                want = ref.decide(float("inf"))
            else:
                d, p = oracle.residual_change(f64(st), f64(states[i - 1]))
                want = ref.decide(d / p)
            assert got == want, (mc, i)


# ----------------------------------------------------------------- fp8 (e4m3) attention

def _e4m3(t):
    """Decode uint8 e4m3 codes through the oracle's code table (from the format definition)."""
    return oracle.e4m3_values()[t.cpu().numpy()]


# byte slot of key kappa inside a 64-key block of v8t, as the ABI documents it
_V8T_SLOT = np.array([32 * ((kk >> 2) & 1) + 16 * (kk >> 5) + 4 * ((kk >> 3) & 3) + (kk & 3) for kk in range(64)])


def _v8t_to_tokens(v8t_vals, n):
    """[B, H, D, nB*64] (slot order) -> [B, N, H, D] values, and the padding slots."""
    b, h, d, np_ = v8t_vals.shape
    blocks = v8t_vals.reshape(b, h, d, np_ // 64, 64)[..., _V8T_SLOT]          # key order
    tok = blocks.reshape(b, h, d, np_).transpose(0, 3, 1, 2)
    return tok[:, :n], tok[:, n:]


def _scaled_case(b, n, h, d, seed):
    """N(0,1) inputs whose tokens (q, k: factors 2^-3 .. 2^1, so scores stay in the range of
    real attention) and channels (v: 2^-4 .. 2^4) differ in magnitude, so that the power-of-two
    scales differ between blocks and channels."""
    c = random_case(b, n, h, d, seed=seed, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    tok = torch.exp2(torch.randint(-3, 2, (1, n, 1, 1), generator=g, device=DEV).float())
    ch = torch.exp2(torch.randint(-4, 5, (1, 1, 1, d), generator=g, device=DEV).float())
    for nm in ("q", "k"):
        c[nm] = (c[nm].float() * tok).to(torch.bfloat16)
    c["v"] = (c["v"].float() * ch).to(torch.bfloat16)
    return c


@pytest.mark.parametrize("b,n,h,d", [(1, 256, 2, 64), (2, 333, 3, 128), (1, 1, 1, 64), (1, 4100, 1, 128)])
def test_fp8_quantize_bit_exact(h3, b, n, h, d):
    c = _scaled_case(b, n, h, d, 700 + n)
    fq = h3.fp8_quantize(c["q"], c["k"], c["v"])
    _sync()
    for nm, t8, ts in (("q", fq.q8, fq.q_scale), ("k", fq.k8, fq.k_scale)):
        ref8, refs = oracle.quantize_blocks(f64(c[nm]), 64)
        np.testing.assert_array_equal(ts.cpu().numpy().astype(np.float64), refs, err_msg=f"{nm} scales")
        np.testing.assert_array_equal(_e4m3(t8), ref8, err_msg=f"{nm} codes")
    v8, sv = oracle.quantize_channels(f64(c["v"]))
    np.testing.assert_array_equal(fq.v_scale.cpu().numpy().astype(np.float64), sv)
    tok, pad = _v8t_to_tokens(_e4m3(fq.v8t), n)
    np.testing.assert_array_equal(tok, v8)
    assert (pad == 0).all()
    log(f"fp8 quantize {b}x{n}x{h}x{d}: codes and scales bit-exact")


def _fp8_vs_exact(g, exact, what, wl, v=None):
    """fp8 output against exact float64 attention: absolute for the workloads' N(0,1) values, or,
    with v given, relative to the RMS of each value channel over the keys of its (batch, head)."""
    err = np.abs(g - exact)
    if v is None:
        mx, mean = float(err.max()), float(err.mean())
        lim = (FP8_EXACT_MAX_ABS, FP8_EXACT_MEAN_ABS)
    else:
        rms = np.sqrt(np.mean(v * v, axis=1, keepdims=True))          # [B, 1, Hd, D]
        rel = err / np.maximum(rms, 1e-30)
        mx, mean = float(rel.max()), float(rel.mean())
        lim = (FP8_EXACT_MAX_REL_RMS, FP8_EXACT_MEAN_REL_RMS)
    log(f"{what}: fp8 path vs exact attention max {mx:.3g} mean {mean:.3g} (limits {lim[0]}, {lim[1]}"
        f"{', per value-channel RMS' if v is not None else ''})")
    record(wl, "fp8 vs exact" + (" (rel rms)" if v is not None else ""), max_abs=mx, mean_abs=mean)
    assert mx <= lim[0] and mean <= lim[1], f"{what}: fp8 vs exact attention max {mx} mean {mean}"


def _fp8_compare(o, lse, ref, rl, wmax, dev, what, exact=None, wl="fp8", v=None):
    """fp8 path vs its oracle. Where the fp32 score decides an e4m3 probability code next to a
    rounding boundary, the GPU and the float64 oracle may pick neighbouring codes; one such
    choice moves a row by at most 2^-3 * wmax * dev (oracle quantities of that row). The bound
    per element is therefore ATTN_MAX_ABS + 2^-8 |ref| (bf16 output rounding of larger values)
    + 2^-3 * wmax * dev; the mean error must stay within the bf16 path's bound and at most 2% of
    the rows may exceed ATTN_MAX_ABS + 2^-8 |ref|. With `exact` given, the output is also held to
    the fp8 bar against exact attention (_fp8_vs_exact)."""
    g = f64(o)
    err = np.abs(g - ref)
    w = np.transpose(wmax, (0, 2, 1))[..., None]                       # [B, N, Hd, 1]
    base = ATTN_MAX_ABS + 2.0 ** -8 * np.abs(ref)
    bound = base + 2.0 ** -3 * w * dev
    over = (err > base).any(axis=-1)
    lerr = np.abs(f64(lse) - rl)
    lbound = LSE_MAX_ABS + math.log(2.0) * np.log2(1.0 + 2.0 ** -3 * wmax)
    log(f"{what}: max-abs {err.max():.3g} mean-abs {err.mean():.3g}, rows over base: {int(over.sum())} "
        f"of {over.size}, worst err/bound {(err / bound).max():.3f}, lse max-abs {lerr.max():.3g}")
    record(wl, "fp8 vs fp8 oracle", max_abs=float(err.max()), mean_abs=float(err.mean()),
           err_over_bound=float((err / bound).max()), rows_over_base=int(over.sum()), rows=int(over.size))
    assert err.mean() <= ATTN_MEAN_ABS + 2.0 ** -9 * np.abs(ref).mean(), what
    assert (err <= bound).all(), what
    assert over.mean() <= 0.02, what
    assert (lerr <= lbound).all(), what
    if exact is not None:
        _fp8_vs_exact(g, exact, what, wl, v)


@pytest.mark.parametrize("b,n,d", [(1, 1, 64), (1, 63, 128), (2, 200, 64), (1, 333, 128), (1, 64 * 20, 128),
                                   (2, 64 * 9 + 7, 128)])
def test_fp8_dense_and_sparse_full(h3, b, n, d):
    c = _scaled_case(b, n, 3, d, 800 + n + b)
    qd, kd, vd = f64(c["q"]), f64(c["k"]), f64(c["v"])
    fq = h3.fp8_quantize(c["q"], c["k"], c["v"])
    o, lse = h3.fp8_dense_fwd(fq, return_lse=True)
    _sync()
    ref, rl, wm, dv = oracle.attention_fp8_detail(qd, kd, vd)
    _fp8_compare(o, lse, ref, rl, wm, dv, f"fp8 dense n={n} d={d}", exact=oracle.attention(qd, kd, vd)[0],
                 wl="fp8 ragged", v=vd)
    for s in (0.0, 0.5, 0.9):
        idx = h3.subblock_select(c["q"], c["k"], s)
        os_, ls = h3.fp8_block_sparse_fwd(fq, idx, return_lse=True)
        _sync()
        ih = idx.cpu().numpy()
        rs, rls, wms, dvs = oracle.attention_fp8_detail(qd, kd, vd, ih)
        _fp8_compare(os_, ls, rs, rls, wms, dvs, f"fp8 sparse n={n} d={d} s={s}",
                     exact=oracle.sparse_attention(qd, kd, vd, ih, 64)[0], wl="fp8 ragged", v=vd)
        if s == 0.0:
            assert torch.equal(os_, o), "keep-all fp8 sparse must equal fp8 dense bit for bit"


def test_fp8_frame_workload(h3):
    x = make_inputs(FRAME, DEV)
    qd, kd, vd = f64(x["q"]), f64(x["k"]), f64(x["v"])
    fq = h3.fp8_quantize(x["q"], x["k"], x["v"])
    o, lse = h3.fp8_dense_fwd(fq, return_lse=True)
    idx = h3.subblock_select(x["q"], x["k"], 0.75)
    os_, ls = h3.fp8_block_sparse_fwd(fq, idx, return_lse=True)
    _sync()
    ref, rl, wm, dv = oracle.attention_fp8_detail(qd, kd, vd)
    _fp8_compare(o, lse, ref, rl, wm, dv, "fp8 dense frame", exact=oracle.attention(qd, kd, vd)[0], wl="frame")
    ih = idx.cpu().numpy()
    rs, rls, wms, dvs = oracle.attention_fp8_detail(qd, kd, vd, ih)
    _fp8_compare(os_, ls, rs, rls, wms, dvs, "fp8 sparse frame s=0.75",
                 exact=oracle.sparse_attention(qd, kd, vd, ih, 64)[0], wl="frame")


@pytest.mark.timeout(900)
def test_fp8_video5s_sampled(h3):
    cfg = VIDEO5S
    x = make_inputs(cfg, DEV)
    fq = h3.fp8_quantize(x["q"], x["k"], x["v"])
    o = h3.fp8_dense_fwd(fq)
    idx = h3.subblock_select(x["q"], x["k"], 0.75)
    os_ = h3.fp8_block_sparse_fwd(fq, idx, group_stride=h3.frame_group_stride(cfg.grid))
    os1 = h3.fp8_block_sparse_fwd(fq, idx)
    _sync()
    assert torch.equal(os_, os1), "fp8 5s: frame group stride changed the result"
    del os1
    qh, kh, vh, oh, osh, ih = x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), o.cpu(), os_.cpu(), idx.cpu().numpy()
    for h in (0, 17, 47):
        qd, kd, vd = f64(qh[:, :, h:h + 1]), f64(kh[:, :, h:h + 1]), f64(vh[:, :, h:h + 1])
        for i in sample_query_blocks(cfg.n_blocks, 4, seed=3000 + h):
            rows = np.arange(i * 64, (i + 1) * 64)
            for what, got, bidx in (("dense", oh, None), ("sparse", osh, ih[0, h, i])):
                ref, rl, wm, dv = oracle.attention_fp8_rows(qd, kd, vd, 0, 0, i, block_idx=bidx, detail=True)
                g = f64(got[0, rows, h])
                err = np.abs(g - ref)
                bound = ATTN_MAX_ABS + 2.0 ** -8 * np.abs(ref) + 2.0 ** -3 * wm[:, None] * dv
                log(f"fp8 {what} 5s head {h} block {i}: max-abs {err.max():.3g} mean-abs {err.mean():.3g}")
                record("5s", f"fp8 {what} vs fp8 oracle", blocks=1, max_abs=float(err.max()),
                       mean_abs=float(err.mean()))
                assert (err <= bound).all() and err.mean() <= ATTN_MEAN_ABS, f"fp8 {what} 5s head {h} block {i}"
                keys = slice(None) if bidx is None else oracle.block_token_ids(bidx, 64, cfg.n_tokens)
                exact, _ = oracle.attention_head(qd[0, rows, 0], kd[0, keys, 0], vd[0, keys, 0])
                _fp8_vs_exact(g, exact, f"fp8 {what} 5s head {h} block {i}", "5s")


@pytest.mark.timeout(900)
def test_offsets_past_two_to_the_31_elements(h3):
    """q, k, v of 1 x 366,912 x 48 x 128 (2.25e9 elements, 4.5 GB each): element and byte offsets
    past 2^31 in every kernel of the path and of the fp8 path. The last head holds the largest
    offsets; its norm+RoPE rows, sampled dense and block-sparse rows, kept sets, e4m3 codes and
    sampled fp8 dense and block-sparse rows are checked against the oracle."""
    b, n, h, d = 1, 366912, 48, 128
    grid, sections = (91, 84, 48), (32, 48, 48)
    assert b * n * h * d > 2 ** 31
    c = random_case(b, n, h, d, seed=907, device=DEV)
    qo, ko = h3.qk_norm_rope(c["q"], c["k"], c["wq"], c["wk"], grid, sections, 1e4, 1e-6)
    _sync()
    last = slice(h - 1, h)
    rq, rk = oracle.qk_norm_rope(f64(c["q"][:, :, last]), f64(c["k"][:, :, last]), f64(c["wq"]), f64(c["wk"]),
                                 grid, sections, 1e4, float(np.float32(1e-6)))
    for g, r, nm in ((qo[:, :, last], rq, "q"), (ko[:, :, last], rk, "k")):
        worst, exact = check_norm_rope(f64(g), r)
        log(f"2^31+ norm+rope {nm} last head: worst {worst:.3f} ulp, exact {exact:.5f}")
        assert worst <= 1.0 and exact > 0.99
    del c["q"], c["k"]
    nb = n // 64
    blocks = sample_query_blocks(nb, 3, seed=908, extra=(nb - 1,))
    _sampled_dense(h3, qo, ko, c["v"], {h - 1: blocks}, "2^31+")
    keep = oracle.keep_count(nb, 0.75)
    idx = h3.subblock_select(qo, ko, 0.75)
    o = h3.block_sparse_fwd(qo, ko, c["v"], idx, group_stride=h3.frame_group_stride(grid))
    _sync()
    qh, kh, vh = qo[:, :, last].cpu(), ko[:, :, last].cpu(), c["v"][:, :, last].cpu()
    scores = oracle.block_scores(f64(qh), f64(kh), 64)
    ih = idx[:, last].cpu().numpy()
    check_block_sets(ih, oracle.topk_blocks(scores, keep), scores, keep, "2^31+ select last head")
    oh = o[:, :, last].cpu()
    for i in blocks:
        rr = np.arange(i * 64, (i + 1) * 64)
        keys = oracle.block_token_ids(ih[0, 0, i], 64, n)
        ref, _ = oracle.attention_head(f64(qh[0, rr, 0]), f64(kh[0, keys, 0]), f64(vh[0, keys, 0]))
        check_attention(f64(oh[0, rr, 0]), ref, f"2^31+ sparse last head block {i}")
    del o
    fq = h3.fp8_quantize(qo, ko, c["v"])
    _sync()
    for nm, src, t8, ts in (("q", qh, fq.q8, fq.q_scale), ("k", kh, fq.k8, fq.k_scale)):
        ref8, refs = oracle.quantize_blocks(f64(src), 64)
        np.testing.assert_array_equal(ts[:, last].cpu().numpy().astype(np.float64), refs, err_msg=f"{nm} scales")
        np.testing.assert_array_equal(_e4m3(t8[:, :, last]), ref8, err_msg=f"{nm} codes")
    v8, sv = oracle.quantize_channels(f64(vh))
    np.testing.assert_array_equal(fq.v_scale[:, last].cpu().numpy().astype(np.float64), sv)
    tok, pad = _v8t_to_tokens(_e4m3(fq.v8t[:, last]), n)
    np.testing.assert_array_equal(tok, v8)
    del qo, ko
    o8 = h3.fp8_dense_fwd(fq)
    os8 = h3.fp8_block_sparse_fwd(fq, idx, group_stride=h3.frame_group_stride(grid))
    _sync()
    qd, kd, vd = f64(qh), f64(kh), f64(vh)
    o8h, os8h = o8[:, :, last].cpu(), os8[:, :, last].cpu()
    for i in blocks:
        rr = np.arange(i * 64, (i + 1) * 64)
        for what, got, bidx in (("dense", o8h, None), ("sparse", os8h, ih[0, 0, i])):
            ref, _, wm, dv = oracle.attention_fp8_rows(qd, kd, vd, 0, 0, i, block_idx=bidx, detail=True)
            err = np.abs(f64(got[0, rr, 0]) - ref)
            bound = ATTN_MAX_ABS + 2.0 ** -8 * np.abs(ref) + 2.0 ** -3 * wm[:, None] * dv
            log(f"2^31+ fp8 {what} last head block {i}: max-abs {err.max():.3g} mean-abs {err.mean():.3g}")
            assert (err <= bound).all() and err.mean() <= ATTN_MEAN_ABS, f"2^31+ fp8 {what} block {i}"
    log("2^31+ offsets: norm+rope, dense, select, sparse, fp8 codes and fp8 attention of the last head match the oracle")


def test_c_program_drives_the_path_through_the_c_abi(h3, tmp_path):
    """tests/c_abi_consumer.cpp (built by __graft_entry__.build()) is a host program with no Python
    or torch: it allocates its own device buffers and stream and runs norm+RoPE -> dense -> select ->
    block-sparse through the four entry points. Its outputs on a ragged two-batch case (N = 240,
    a partial last block) are checked against the oracle. It also runs the selection with the
    pooling inside the norm+RoPE pass and exits nonzero unless q', k' and the kept sets are the
    same bits as the stand-alone calls'."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "c_abi_consumer")
    assert os.path.exists(exe), "tests/_build/c_abi_consumer is missing: run __graft_entry__.build()"
    b, grid, heads, d, sections, theta, eps, sparsity = 2, (3, 8, 10), 3, 128, (32, 48, 48), 1e4, 1e-6, 0.5
    n = grid[0] * grid[1] * grid[2]
    x = random_case(b, n, heads, d, seed=931)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().astype("<i2").tobytes()
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(np.array([b, *grid, heads, d, *sections], dtype="<i4").tobytes())
        f.write(np.array([theta, eps], dtype="<f4").tobytes())
        f.write(np.array([sparsity], dtype="<f8").tobytes())
        for nm in ("q", "k", "v"):
            f.write(bits(x[nm]))
        f.write(x["wq"].numpy().astype("<f4").tobytes())
        f.write(x["wk"].numpy().astype("<f4").tobytes())
    r = subprocess.run([exe, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    log(r.stdout.strip())
    raw = open(tmp_path / "out.bin", "rb").read()
    elems = b * n * heads * d
    nb = -(-n // 64)
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    def bf16_array(a):
        return torch.from_numpy(a.copy()).view(torch.bfloat16).reshape(b, n, heads, d)

    qo, ko, od = (bf16_array(take("<i2", elems)) for _ in range(3))
    lse = take("<f4", b * heads * n).reshape(b, heads, n)
    keep = int(take("<i4", 1)[0])
    idx = take("<i4", b * heads * nb * keep).reshape(b, heads, nb, keep)
    osp = bf16_array(take("<i2", elems))
    assert off == len(raw) and keep == oracle.keep_count(nb, sparsity)
    rq, rk = oracle.qk_norm_rope(f64(x["q"]), f64(x["k"]), f64(x["wq"]), f64(x["wk"]), grid, sections, theta,
                                 float(np.float32(eps)))
    for got, ref, nm in ((qo, rq, "q"), (ko, rk, "k")):
        worst, exact = check_norm_rope(f64(got), ref)
        assert worst <= 1.0 and exact > 0.99, f"C consumer norm+rope {nm}: {worst} ulp"
    qd, kd, vd = f64(qo), f64(ko), f64(x["v"])
    ro, rl = oracle.attention(qd, kd, vd)
    check_attention(f64(od), ro, "C consumer dense")
    assert np.abs(lse.astype(np.float64) - rl).max() <= LSE_MAX_ABS
    scores = oracle.block_scores(qd, kd, 64)
    check_block_sets(idx, oracle.topk_blocks(scores, keep), scores, keep, "C consumer select")
    rs, _ = oracle.sparse_attention(qd, kd, vd, idx, 64)
    check_attention(f64(osp), rs, "C consumer block-sparse")
