"""C ABI checks that need no GPU: the library loads, exports every declared symbol, and host-side
validation rejects bad arguments before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")
LIB = os.path.join(ROOT, "video_diffusion_transformer_qk_amd", "libh3attn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libh3attn.so not built")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(h3attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from video_diffusion_transformer_qk_amd import _lib
    return _lib.load_library()


def test_every_declared_symbol_is_exported_and_bound(lib):
    from video_diffusion_transformer_qk_amd import _lib
    syms = declared_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(lib, s), s
        assert s in _lib.SIGNATURES, f"{s} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(syms)


def test_version_and_error_string(lib):
    assert b"gfx950" in lib.h3attn_version()
    assert lib.h3attn_last_error() is not None


def test_keep_count_matches_oracle_and_golden(lib):
    golden = os.path.join(ROOT, "tests", "golden", "keep_counts.txt")
    for line in open(golden):
        line = line.split("#")[0].strip()
        if not line:
            continue
        n, s, k = line.split()
        assert lib.h3attn_keep_count(int(n), float(s)) == int(k)
    for n in (1, 7, 63, 1953, 5733):
        for s in (0.0, 0.1, 0.5, 0.75, 0.8, 0.95):
            assert lib.h3attn_keep_count(n, s) == oracle.keep_count(n, s)
    assert lib.h3attn_keep_count(0, 0.5) == -1
    assert lib.h3attn_keep_count(10, 1.0) == -1
    assert lib.h3attn_keep_count(10, -0.1) == -1


def test_workspace_bytes(lib):
    """The select workspace is O(B * heads * nB * D): float64 means, 3 digit bytes per mean, an
    exponent and two norms per block (blocks padded to 32), per-head key maxima, the fallback list.
    No nB x nB score matrix."""
    r = lambda x: (x + 255) // 256 * 256
    for (bh, nb, d) in ((48, 1953, 128), (12, 5733, 128), (2, 10, 64)):
        nbp = (nb + 31) // 32 * 32
        want = 2 * (r(bh * nb * d * 8) + r(bh * nbp * d * 3) + r(bh * nbp * 4) + r(bh * nbp * 8)) \
            + r(bh * 16) + r((1 + bh * nb) * 4)
        assert lib.h3attn_select_workspace_bytes(1, bh, nb * 64, d, 64) == want
        assert want <= bh * nbp * (22 * d + 28) + bh * 16 + 4 + 10 * 256   # linear in nB, far below nB^2
    # 5 s workload: 0.27 GB (the float64 score matrix alone would have been 1.46 GB)
    assert lib.h3attn_select_workspace_bytes(1, 48, 124992, 128, 64) < 0.28e9
    assert lib.h3attn_select_workspace_bytes(0, 48, 124992, 128, 64) == 0


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def _err(lib):
    return lib.h3attn_last_error().decode()


def test_dense_validation(lib):
    f = lib.h3attn_dense_fwd
    assert f(None, FAKE, FAKE, FAKE, None, 1, 2, 64, 64, None) == 1 and "q is NULL" in _err(lib)
    assert f(FAKE + 2, FAKE, FAKE, FAKE, None, 1, 2, 64, 64, None) == 1 and "aligned" in _err(lib)
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 64, 96, None) == 2 and "head_dim" in _err(lib)
    assert f(FAKE, FAKE, FAKE, FAKE, None, 0, 2, 64, 64, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 0, 64, 64, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, None, 1, 2, 0, 64, None) == 1
    assert f(FAKE, 0x20000, 0x30000, FAKE, None, 1, 2, 64, 64, None) == 1 and "alias" in _err(lib)
    assert f(FAKE, 0x20000, 0x30000, 0x40000, FAKE + 1, 1, 2, 64, 64, None) == 1 and "lse" in _err(lib)


def test_norm_rope_validation(lib):
    from video_diffusion_transformer_qk_amd._lib import Grid
    f = lib.h3attn_qk_norm_rope
    P = [0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000]
    g = Grid(2, 3, 4)
    assert f(*P, 1, 2, 64, Grid(0, 3, 4), 16, 24, 24, 1e4, 1e-6, None) == 1
    assert f(*P, 1, 2, 64, g, 16, 24, 26, 1e4, 1e-6, None) == 1 and "add up" in _err(lib)
    assert f(*P, 1, 2, 64, g, 15, 25, 24, 1e4, 1e-6, None) == 1 and "even" in _err(lib)
    assert f(*P, 1, 2, 80, g, 16, 32, 32, 1e4, 1e-6, None) == 2
    assert f(*P, 1, 2, 64, g, 16, 24, 24, 0.0, 1e-6, None) == 1 and "theta" in _err(lib)
    assert f(*P, 1, 2, 64, g, 16, 24, 24, 1e4, -1.0, None) == 1 and "eps" in _err(lib)
    assert f(P[0], P[1], P[2], P[2], P[4], P[5], 1, 2, 64, g, 16, 24, 24, 1e4, 1e-6, None) == 1


def test_select_and_sparse_validation(lib):
    f = lib.h3attn_subblock_select
    nbytes = lib.h3attn_select_workspace_bytes(1, 2, 640, 64, 64)
    ws = 0x100000
    ok_args = dict(q=0x10000, k=0x20000, b=1, h=2, n=640, d=64, bs=64, s=0.5, keep=5, idx=0x30000, ws=ws, wsb=nbytes)

    def call(**kw):
        a = dict(ok_args, **kw)
        return f(a["q"], a["k"], a["b"], a["h"], a["n"], a["d"], a["bs"], a["s"], a["keep"], a["idx"], a["ws"], a["wsb"], None)

    assert call(bs=32) == 2 and "block_size" in _err(lib)
    assert call(s=1.0) == 1 and "sparsity" in _err(lib)
    assert call(s=-0.5) == 1
    assert call(keep=4) == 1 and "keep" in _err(lib)
    assert call(wsb=nbytes - 1) == 1 and "workspace" in _err(lib)
    assert call(ws=ws + 16) == 1 and "256-byte" in _err(lib)
    assert call(idx=None) == 1
    assert call(d=72) == 2
    # a row of nB float64 scores must fit in one CU's LDS: nB <= (160 KiB - 4 KiB) / 8 = 19968
    assert call(n=19969 * 64) == 2 and "LDS" in _err(lib)
    assert call(n=19968 * 64) == 1 and "LDS" not in _err(lib)  # passes the row check, fails on keep
    g = lib.h3attn_block_sparse_fwd
    P = (0x10000, 0x20000, 0x30000)
    assert g(*P, 0x40000, 0, 0x50000, None, 1, 2, 640, 64, 64, None) == 1 and "keep" in _err(lib)
    assert g(*P, 0x40000, 11, 0x50000, None, 1, 2, 640, 64, 64, None) == 1
    assert g(*P, None, 3, 0x50000, None, 1, 2, 640, 64, 64, None) == 1
    assert g(*P, 0x40000, 3, 0x50000, None, 1, 2, 640, 64, 32, None) == 2
    gg = lib.h3attn_block_sparse_grouped_fwd
    assert gg(*P, 0x40000, 3, 0x50000, None, 1, 2, 640, 64, 64, 0, None) == 1 and "group_stride" in _err(lib)
    assert gg(*P, 0x40000, 3, 0x50000, None, 1, 2, 640, 64, 64, 11, None) == 1 and "group_stride" in _err(lib)
    assert gg(*P, 0x40000, 0, 0x50000, None, 1, 2, 640, 64, 64, 2, None) == 1 and "keep" in _err(lib)


def test_threshold_validation(lib):
    ws = 0x100000
    nbytes = lib.h3attn_threshold_workspace_bytes(1, 2, 640, 64, 64)
    assert nbytes == lib.h3attn_select_workspace_bytes(1, 2, 640, 64, 64) + 2 * 256
    f = lib.h3attn_subblock_threshold_count
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 64, -1.0, 0x30000, ws, nbytes, None) == 1 and "tau" in _err(lib)
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 64, float("nan"), 0x30000, ws, nbytes, None) == 1
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 64, 0.5, None, ws, nbytes, None) == 1 and "row_ptr" in _err(lib)
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 64, 0.5, 0x30004, ws, nbytes, None) == 1
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 64, 0.5, 0x30000, ws, nbytes - 8, None) == 1 and "workspace" in _err(lib)
    assert f(0x10000, 0x20000, 1, 2, 640, 64, 32, 0.5, 0x30000, ws, nbytes, None) == 2
    assert f(0x10000, 0x20000, 1, 2, 19969 * 64, 64, 64, 0.5, 0x30000, ws, nbytes, None) == 2 and "LDS" in _err(lib)
    g = lib.h3attn_subblock_threshold_fill
    assert g(1, 2, 19969 * 64, 64, 64, 0x30000, 0x40000, 10, ws, nbytes, None) == 2 and "LDS" in _err(lib)
    assert g(1, 2, 640, 64, 64, 0x30000, 0x40000, -1, ws, nbytes, None) == 1
    assert g(1, 2, 640, 64, 64, None, 0x40000, 10, ws, nbytes, None) == 1
    assert g(1, 2, 640, 64, 64, 0x30000, None, 10, ws, nbytes, None) == 1
    h = lib.h3attn_block_sparse_csr_fwd
    P = (0x10000, 0x20000, 0x30000)
    assert h(*P, None, 0x40000, 0x50000, None, 1, 2, 640, 64, 64, None) == 1
    assert h(*P, 0x60000, None, 0x50000, None, 1, 2, 640, 64, 64, None) == 1
    assert h(*P, 0x60000, 0x40000, 0x50000, None, 1, 2, 640, 64, 32, None) == 2
    hg = lib.h3attn_block_sparse_csr_grouped_fwd
    assert hg(*P, 0x60000, 0x40000, 0x50000, None, 1, 2, 640, 64, 64, -1, None) == 1 and "group_stride" in _err(lib)
    assert hg(*P, None, 0x40000, 0x50000, None, 1, 2, 640, 64, 64, 2, None) == 1 and "row_ptr" in _err(lib)


def test_block_ops_validation(lib):
    f = lib.h3attn_adaln_modulate
    P = (0x10000, 0x20000, 0x30000, 0x40000)
    assert f(None, *P[1:], 1, 64, 128, 1e-6, None) == 1
    assert f(*P, 0, 64, 128, 1e-6, None) == 1
    assert f(*P, 1, 64, 100, 1e-6, None) == 2 and "hidden" in _err(lib)
    assert f(*P, 1, 64, 16392, 1e-6, None) == 2
    assert f(*P, 1, 64, 128, -1.0, None) == 1 and "eps" in _err(lib)
    g = lib.h3attn_swiglu
    assert g(0x10000, 0x20000, 0x30000, 0, 128, 128, 128, None) == 1
    assert g(0x10000, 0x20000, 0x30000, 4, 128, 64, 128, None) == 1 and "stride" in _err(lib)
    assert g(0x10000, 0x20000, 0x30000, 4, 100, 104, 104, None) == 2
    assert g(0x10000, 0x20000, 0x10000, 4, 128, 256, 128, None) == 1 and "alias" in _err(lib)
    assert g(0x10002, 0x20000, 0x30000, 4, 128, 128, 128, None) == 1


def test_residual_change_validation(lib):
    f = lib.h3attn_residual_change
    nbytes = lib.h3attn_residual_workspace_bytes(1000)
    assert nbytes >= 16 and nbytes % 256 == 0
    assert lib.h3attn_residual_workspace_bytes(0) == 0
    assert f(None, 0x20000, 1000, 0x30000, 0x100000, nbytes, None) == 1
    assert f(0x10000, 0x20000, 0, 0x30000, 0x100000, nbytes, None) == 1
    assert f(0x10000, 0x20000, 1000, None, 0x100000, nbytes, None) == 1 and "result" in _err(lib)
    assert f(0x10000, 0x20000, 1000, 0x30000, 0x100000, nbytes - 1, None) == 1 and "workspace" in _err(lib)


def test_cache_gate_policy_matches_oracle_rule(lib):
    """The C policy (host code, no GPU) against the oracle's statement of the rule."""
    from video_diffusion_transformer_qk_amd._lib import CacheGateState
    rng = np.random.default_rng(5)
    for trial in range(50):
        thr = float(rng.choice([0.0, 0.05, 0.1, 0.5]))
        mc = int(rng.integers(0, 5))
        st = CacheGateState()
        assert lib.h3attn_cache_gate_init(ctypes.byref(st), thr, mc) == 0
        ref = oracle.CacheGate(thr, mc)
        for r in rng.choice([0.0, 0.01, 0.05, 0.099, 0.1, 0.3, 1.0], size=40):
            assert bool(lib.h3attn_cache_gate_decide(ctypes.byref(st), float(r))) == ref.decide(float(r))
        assert st.steps == 40
    # the ratio of the two device sums is formed inside the library
    for mc in (1, 3):
        st = CacheGateState()
        assert lib.h3attn_cache_gate_init(ctypes.byref(st), 0.1, mc) == 0
        ref = oracle.CacheGate(0.1, mc)
        seq = [None, (0.5, 10.0), (0.5, 10.0), (0.5, 10.0), (3.0, 10.0), (0.0, 0.0), (0.2, 10.0), (0.99, 10.0)]
        for sums in seq:
            arg = None if sums is None else ctypes.cast((ctypes.c_double * 2)(*sums), ctypes.c_void_p)
            want = ref.decide(float("inf") if sums is None or sums[1] <= 0 else sums[0] / sums[1])
            assert bool(lib.h3attn_cache_gate_decide_sums(ctypes.byref(st), arg)) == want
    assert lib.h3attn_cache_gate_decide_sums(None, None) == -1
    st = CacheGateState()
    assert lib.h3attn_cache_gate_init(ctypes.byref(st), -1.0, 1) == 1
    assert lib.h3attn_cache_gate_init(ctypes.byref(st), 0.1, -1) == 1
    assert lib.h3attn_cache_gate_init(None, 0.1, 1) == 1
    assert lib.h3attn_cache_gate_decide(None, 0.0) == -1


def test_fp8_workspace_bytes_and_validation(lib):
    r = lambda x: (x + 255) // 256 * 256
    chunks = (124992 + 1023) // 1024
    assert lib.h3attn_fp8_workspace_bytes(1, 48, 124992, 128, 64) == r(48 * chunks * 128 * 4) + r(48 * 128 * 4)
    assert lib.h3attn_fp8_workspace_bytes(1, 0, 124992, 128, 64) == 0
    q, k, v, q8, k8, v8t, sq, sk, sv, ws = (0x10000 * (i + 1) for i in range(10))
    big = 1 << 20
    f = lib.h3attn_fp8_quantize
    # every call below fails validation before any launch (pointers are never dereferenced)
    assert f(None, k, v, q8, k8, v8t, sq, sk, sv, 1, 2, 64, 64, 64, ws, big, None) == 1 and "q is NULL" in _err(lib)
    assert f(q, k, v, q8 + 8, k8, v8t, sq, sk, sv, 1, 2, 64, 64, 64, ws, big, None) == 1 and "aligned" in _err(lib)
    assert f(q, k, v, q8, k8, v8t, sq, sk, sv, 1, 2, 64, 96, 64, ws, big, None) == 2 and "head_dim" in _err(lib)
    assert f(q, k, v, q8, k8, v8t, sq, sk, sv, 1, 2, 64, 64, 32, ws, big, None) == 2 and "block_size" in _err(lib)
    assert f(q, k, v, q8, k8, v8t, sq, sk, sv, 1, 2, 64, 64, 64, ws, 16, None) == 1 and "workspace" in _err(lib)
    assert f(q, k, v, q, k8, v8t, sq, sk, sv, 1, 2, 64, 64, 64, ws, big, None) == 1 and "alias" in _err(lib)
    g = lib.h3attn_fp8_dense_fwd
    out = 0x200000
    assert g(None, k8, v8t, sq, sk, sv, out, None, 1, 2, 64, 64, 64, None) == 1 and "q8 is NULL" in _err(lib)
    assert g(q8, k8, v8t, sq, sk, sv, out, out + 2, 1, 2, 64, 64, 64, None) == 1 and "lse" in _err(lib)
    assert g(q8, k8, v8t, sq, sk, sv, q8, None, 1, 2, 64, 64, 64, None) == 1 and "alias" in _err(lib)
    assert g(q8, k8, v8t, sq, sk, sv, out, None, 1, 2, 64, 128, 16, None) == 2 and "block_size" in _err(lib)
    h = lib.h3attn_fp8_block_sparse_fwd
    idx = 0x300000
    assert h(q8, k8, v8t, sq, sk, sv, None, 1, out, None, 1, 2, 128, 64, 64, 1, None) == 1 and "block_idx" in _err(lib)
    assert h(q8, k8, v8t, sq, sk, sv, idx, 0, out, None, 1, 2, 128, 64, 64, 1, None) == 1 and "keep" in _err(lib)
    assert h(q8, k8, v8t, sq, sk, sv, idx, 3, out, None, 1, 2, 128, 64, 64, 1, None) == 1 and "keep" in _err(lib)
    assert h(q8, k8, v8t, sq, sk, sv, idx + 2, 1, out, None, 1, 2, 128, 64, 64, 1, None) == 1 and "aligned" in _err(lib)
    assert h(q8, k8, v8t, sq, sk, sv, idx, 1, out, None, 1, 2, 128, 64, 64, 3, None) == 1 and "group_stride" in _err(lib)


def test_kept_set_check_validation(lib):
    f = lib.h3attn_check_block_idx
    assert f(None, 1, 2, 10, 3, 0x2000, None) == 1 and "block_idx" in _err(lib)
    assert f(0x1002, 1, 2, 10, 3, 0x2000, None) == 1 and "aligned" in _err(lib)
    assert f(0x1000, 1, 2, 10, 3, None, None) == 1 and "row_flags" in _err(lib)
    assert f(0x1000, 1, 2, 10, 0, 0x2000, None) == 1 and "keep" in _err(lib)
    assert f(0x1000, 1, 2, 10, 11, 0x2000, None) == 1 and "keep" in _err(lib)
    assert f(0x1000, 0, 2, 10, 3, 0x2000, None) == 1
    assert f(0x1000, 1, 2, (1 << 20) + 1, 3, 0x2000, None) == 2 and "n_blocks" in _err(lib)
    g = lib.h3attn_check_csr
    assert g(None, 0x1000, 5, 1, 2, 10, 0x2000, None) == 1 and "row_ptr" in _err(lib)
    assert g(0x1004, 0x1000, 5, 1, 2, 10, 0x2000, None) == 1 and "8-byte" in _err(lib)
    assert g(0x1000, None, 5, 1, 2, 10, 0x2000, None) == 1 and "col_idx" in _err(lib)
    assert g(0x1000, 0x1000, -1, 1, 2, 10, 0x2000, None) == 1 and "col_capacity" in _err(lib)
    assert g(0x1000, 0x1000, 5, 1, 2, 10, None, None) == 1 and "row_flags" in _err(lib)
    assert g(0x1000, 0x1000, 5, 1, 2, (1 << 20) + 1, 0x2000, None) == 2


def test_frame_group_stride_rule():
    import video_diffusion_transformer_qk_amd as h3
    assert h3.frame_group_stride((31, 48, 84)) == 63      # 5 s: 63 blocks per frame
    assert h3.frame_group_stride((91, 84, 48)) == 63      # 15 s vertical
    assert h3.frame_group_stride((4, 8, 8)) == 1          # frames of 64 tokens: one block each
    assert h3.frame_group_stride((4, 16, 16)) == 4
    assert h3.frame_group_stride((1, 48, 84)) == 1        # one frame
    assert h3.frame_group_stride((3, 48, 84)) == 1        # fewer than four frames
    assert h3.frame_group_stride((5, 10, 10)) == 1        # frames are not whole blocks
