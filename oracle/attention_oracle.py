"""Plain float64 CPU oracle for the video-DiT attention hot path.

TEST INFRASTRUCTURE. Only the tests, the package entry's smoke check and the benchmark's CPU
baseline leg may import this module. The product path never calls it, and it shares no code,
tables or constants with the HIP kernels.

Each function is the plain definition of one step, written in numpy float64, slow and direct.
Inputs are the bf16 tensors the GPU consumed, converted exactly to float64; weights are float32
converted to float64; theta, eps and sparsity are the values passed through the C ABI.

Sources (web pages on MiniMax-H3 video generation; cited by page title and section):
  [P3] "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai/posts/minimax-h3-speed-quality)
       section "先把近两倍的免费收益拿走": the lossless runtime fuses QK RMSNorm and 3D RoPE into
       one kernel; fusion does not change the math.
       section "6.24 倍里，真正有损的部分大约是三倍": SubBlock cuts queries and keys into
       64-token blocks, estimates which key blocks contribute little, keeps only high-score key
       blocks for a block-sparse attention kernel; sparsity is the fraction of key blocks dropped.
  [P4] "MiniMax-H3 在 8×H200 上基准测试：无损加速 1.95×，最高 6.24×" (chat-gpts.plus/?p=43161)
       section "为什么重要": attention over very long latent sequences is one of the two costs.

Where the pages leave a step open, the reading taken is stated at the function. Parity pins
for every function live in the CPU tests; the numeric conventions of RoPE (pair layout,
frequencies, positions) are self-consistent readings and, for the absolute convention,
parity unpinned by the pages.

Layout: q, k, v are [B, N, Hd, D] (tokens, then heads, then channels), token n of a T x H x W
latent grid sits at n = (t*H + h)*W + w.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------------------------
# (1) QK RMSNorm + 3D RoPE   [P3, section 先把近两倍的免费收益拿走]
# --------------------------------------------------------------------------------------------


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x * w / sqrt(mean(x^2) + eps), over the last axis (one head's D channels).

    Reading: the norm is per head over D with one weight vector shared by all heads; eps is
    added inside the square root."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * w


def token_positions(grid: Tuple[int, int, int]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Integer (t, h, w) coordinates of every token of a T x H x W grid, flattened t-major."""
    t_len, h_len, w_len = grid
    n = np.arange(t_len * h_len * w_len, dtype=np.int64)
    return n // (h_len * w_len), (n // w_len) % h_len, n % w_len


def rope_frequencies(d_section: int, theta: float) -> np.ndarray:
    """theta^(-2j/d) for j < d/2: the rotation rate of pair j inside one axis section."""
    j = np.arange(d_section // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / d_section)


def rope3d(x: np.ndarray, grid: Tuple[int, int, int], sections: Sequence[int], theta: float) -> np.ndarray:
    """3-axis rotary embedding.

    Reading: the head dimension is cut into contiguous [t | h | w] sections of sizes
    (d_t, d_h, d_w). Inside section a, channels (2j, 2j+1) form a pair rotated by the angle
    p_a * theta^(-2j/d_a), where p_a is the token's integer coordinate on axis a."""
    x = np.asarray(x, dtype=np.float64)
    if sum(sections) != x.shape[-1]:
        raise ValueError("sections must add up to head_dim")
    n_tok = x.shape[1]
    pos = token_positions(grid)
    if pos[0].shape[0] != n_tok:
        raise ValueError("grid does not match the token count")
    out = x.copy()
    off = 0
    for p, d_a in zip(pos, sections):
        ang = p[:, None].astype(np.float64) * rope_frequencies(d_a, theta)[None, :]   # [N, d_a/2]
        c = np.cos(ang)[None, :, None, :]
        s = np.sin(ang)[None, :, None, :]
        x0 = x[..., off:off + d_a:2]
        x1 = x[..., off + 1:off + d_a:2]
        out[..., off:off + d_a:2] = x0 * c - x1 * s
        out[..., off + 1:off + d_a:2] = x0 * s + x1 * c
        off += d_a
    return out


def qk_norm_rope(q, k, w_q, w_k, grid, sections, theta, eps):
    """RMSNorm then RoPE, for q and k (the fused kernel computes the same composition)."""
    return (rope3d(rms_norm(q, w_q, eps), grid, sections, theta),
            rope3d(rms_norm(k, w_k, eps), grid, sections, theta))


# --------------------------------------------------------------------------------------------
# (2) Dense self-attention   [P4, section 为什么重要]
# --------------------------------------------------------------------------------------------


def _softmax_rows(s: np.ndarray):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, row_chunk: int = 256):
    """softmax(q k^T / sqrt(D)) v for one head: q [M, D], k [N, D], v [N, D].
    Returns (O [M, D], lse [M]) with lse = ln sum_j exp(s_ij). Rows are independent; they are
    processed in chunks only to bound memory."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty((q.shape[0],), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for r0 in range(0, q.shape[0], row_chunk):
        s = (q[r0:r0 + row_chunk] @ k.T) * scale
        p, lse[r0:r0 + row_chunk] = _softmax_rows(s)
        out[r0:r0 + row_chunk] = p @ v
    return out, lse


def attention(q, k, v):
    """Non-causal, unmasked multi-head attention on [B, N, Hd, D] tensors.
    Returns (O [B, N, Hd, D], lse [B, Hd, N])."""
    b_len, n_len, h_len, d = q.shape
    out = np.empty((b_len, n_len, h_len, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b_len, h_len, n_len), dtype=np.float64)
    for b in range(b_len):
        for h in range(h_len):
            out[b, :, h, :], lse[b, h] = attention_head(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :])
    return out, lse


# --------------------------------------------------------------------------------------------
# (3) SubBlock selection and block-sparse attention   [P3, section 6.24 倍里，真正有损的部分大约是三倍]
# --------------------------------------------------------------------------------------------


def keep_count(n_blocks: int, sparsity: float) -> int:
    """Key blocks kept per query block: ceil((1 - s) * n), at least 1 and at most n.

    Sparsity is the fraction of key blocks dropped. A 1e-9 guard keeps float noise such as
    (1 - 0.7) * 10 = 3.0000000000000004 from rounding up."""
    if not (0.0 <= sparsity < 1.0) or n_blocks <= 0:
        raise ValueError("need 0 <= sparsity < 1 and n_blocks > 0")
    return int(min(n_blocks, max(1, math.ceil((1.0 - sparsity) * n_blocks - 1e-9))))


def n_blocks_of(n_tokens: int, block_size: int) -> int:
    return -(-n_tokens // block_size)


def block_means(x: np.ndarray, block_size: int) -> np.ndarray:
    """Mean of each run of block_size consecutive tokens, per (batch, head): [B, Hd, nB, D].
    A partial last block averages over its valid tokens."""
    x = np.asarray(x, dtype=np.float64)
    b_len, n_len, h_len, d = x.shape
    nb = n_blocks_of(n_len, block_size)
    out = np.empty((b_len, h_len, nb, d), dtype=np.float64)
    for i in range(nb):
        seg = x[:, i * block_size:min((i + 1) * block_size, n_len)]      # [B, len, Hd, D]
        out[:, :, i, :] = seg.mean(axis=1)
    return out


def block_scores(q: np.ndarray, k: np.ndarray, block_size: int) -> np.ndarray:
    """S_bar[b, h, i, j] = mean(q in block i) . mean(k in block j) / sqrt(D).

    The pages leave the importance estimate open; this library fixes it as the scaled dot product
    of mean-pooled query and key blocks."""
    qm = block_means(q, block_size)
    km = block_means(k, block_size)
    d = q.shape[-1]
    return np.matmul(qm, np.swapaxes(km, -1, -2)) / math.sqrt(d)


def topk_blocks(scores: np.ndarray, keep: int) -> np.ndarray:
    """Per row, the keep largest scores; equal scores rank the lower key index first (a stable
    sort on -score). Returned indices are ascending, int32, shape [..., keep]."""
    scores = np.asarray(scores, dtype=np.float64)
    order = np.argsort(-scores, axis=-1, kind="stable")[..., :keep]
    return np.sort(order, axis=-1).astype(np.int32)


def subblock_select(q, k, block_size: int, sparsity: float) -> np.ndarray:
    """Kept key-block indices [B, Hd, nB, keep] for every query block."""
    nb = n_blocks_of(q.shape[1], block_size)
    return topk_blocks(block_scores(q, k, block_size), keep_count(nb, sparsity))


def near_tie_rows(scores: np.ndarray, keep: int, rel: float = 1e-5) -> np.ndarray:
    """Boolean mask of rows whose keep-th and (keep+1)-th largest scores differ by at most
    rel * max(|a|, |b|); only such rows may legitimately select a different set."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[-1]
    if keep >= n:
        return np.zeros(scores.shape[:-1], dtype=bool)
    srt = -np.sort(-scores, axis=-1)
    a = srt[..., keep - 1]
    b = srt[..., keep]
    return np.abs(a - b) <= rel * np.maximum(np.abs(a), np.abs(b))


def block_token_ids(blocks: Sequence[int], block_size: int, n_tokens: int) -> np.ndarray:
    ids = [np.arange(j * block_size, min((j + 1) * block_size, n_tokens)) for j in blocks]
    return np.concatenate(ids) if ids else np.zeros((0,), dtype=np.int64)


def sparse_attention_rows(q, k, v, block_idx, block_size: int, b: int, h: int, qblock: int):
    """Output rows of query block `qblock` of (batch b, head h): attention restricted to the
    tokens of its kept key blocks, softmax renormalised over those tokens."""
    n_len = q.shape[1]
    rows = np.arange(qblock * block_size, min((qblock + 1) * block_size, n_len))
    keys = block_token_ids(block_idx[b, h, qblock], block_size, k.shape[1])
    return attention_head(q[b, rows, h, :], k[b, keys, h, :], v[b, keys, h, :])


def sparse_attention(q, k, v, block_idx, block_size: int):
    """Block-sparse attention on [B, N, Hd, D] tensors; block_idx is [B, Hd, nB, keep].
    Returns (O [B, N, Hd, D], lse [B, Hd, N])."""
    b_len, n_len, h_len, d = q.shape
    nb = n_blocks_of(n_len, block_size)
    out = np.empty((b_len, n_len, h_len, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b_len, h_len, n_len), dtype=np.float64)
    for b in range(b_len):
        for h in range(h_len):
            for i in range(nb):
                r0, r1 = i * block_size, min((i + 1) * block_size, n_len)
                out[b, r0:r1, h, :], lse[b, h, r0:r1] = sparse_attention_rows(q, k, v, block_idx, block_size, b, h, i)
    return out, lse


# --------------------------------------------------------------------------------------------
# (4) Threshold-mode SubBlock selection with a variable number of kept blocks per row
#     ["MiniMax-H3 在 8×H200 上基准测试…", section 事件核心: SubBlock described as skipping the
#     attention blocks that fall below a threshold]
# --------------------------------------------------------------------------------------------


def threshold_blocks(scores: np.ndarray, tau: float):
    """Per row i of scores [..., nB]: keep key block j iff S_ij >= max_j S_ij - tau (tau >= 0, in
    the units of the scaled block score). Reading: the pages give no threshold rule; this keeps
    every block within tau of the row's best block, so tau = 0 keeps only the best block(s) and
    tau = inf keeps all. Returns (row_ptr int64 [R + 1], col_idx int32 [nnz]) in CSR form over
    the flattened rows, each row's indices ascending."""
    if not (tau >= 0.0):
        raise ValueError("tau must be >= 0")
    scores = np.asarray(scores, dtype=np.float64)
    flat = scores.reshape(-1, scores.shape[-1])
    rows = []
    for r in range(flat.shape[0]):
        thr = flat[r].max() - tau
        rows.append(np.nonzero(flat[r] >= thr)[0].astype(np.int32))
    counts = np.array([len(x) for x in rows], dtype=np.int64)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col_idx = np.concatenate(rows) if rows else np.zeros((0,), dtype=np.int32)
    return row_ptr, col_idx.astype(np.int32)


def subblock_select_threshold(q, k, block_size: int, tau: float):
    """Threshold-mode kept sets of every query block, CSR over rows (b, head, query block)."""
    return threshold_blocks(block_scores(q, k, block_size), tau)


def near_threshold_entries(scores: np.ndarray, tau: float, rel: float = 1e-9) -> np.ndarray:
    """Boolean mask of (row, j) entries whose score lies within rel (relative to the row's
    largest magnitude) of that row's threshold: only these may legitimately flip between two
    correct float evaluations."""
    scores = np.asarray(scores, dtype=np.float64)
    mx = scores.max(axis=-1, keepdims=True)
    scale = np.maximum(np.abs(scores).max(axis=-1, keepdims=True), 1e-300)
    return np.abs(scores - (mx - tau)) <= rel * scale


def sparse_attention_csr(q, k, v, row_ptr, col_idx, block_size: int):
    """Block-sparse attention with a variable kept set per query block (CSR over the rows
    (b, head, query block)). Returns (O [B, N, Hd, D], lse [B, Hd, N])."""
    b_len, n_len, h_len, d = q.shape
    nb = n_blocks_of(n_len, block_size)
    out = np.empty((b_len, n_len, h_len, v.shape[-1]), dtype=np.float64)
    lse = np.empty((b_len, h_len, n_len), dtype=np.float64)
    for b in range(b_len):
        for h in range(h_len):
            for i in range(nb):
                r = (b * h_len + h) * nb + i
                blocks = col_idx[row_ptr[r]:row_ptr[r + 1]]
                rows = np.arange(i * block_size, min((i + 1) * block_size, n_len))
                keys = block_token_ids(blocks, block_size, n_len)
                out[b, rows, h, :], lse[b, h, rows] = attention_head(q[b, rows, h, :], k[b, keys, h, :], v[b, keys, h, :])
    return out, lse


# --------------------------------------------------------------------------------------------
# (5) The other fused block ops of the lossless runtime: AdaLN modulation and SwiGLU
#     ["MiniMax-H3 的 6.24 倍…", section 先把近两倍的免费收益拿走: the runtime fuses AdaLN and
#     SwiGLU kernels as well as QK RMSNorm and 3D RoPE]
# --------------------------------------------------------------------------------------------


def adaln_modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float) -> np.ndarray:
    """y = LayerNorm(x) * (1 + scale) + shift over the last (hidden) axis.

    Reading: the pages name the fused AdaLN kernel without a formula; this is the usual DiT
    adaptive LayerNorm: normalisation without its own affine weights (biased variance, eps inside
    the square root), then a per-(batch, channel) scale and shift from the conditioning.
    x is [B, N, C]; shift and scale are [B, C]."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    xn = (x - mean) / np.sqrt(var + float(eps))
    shift = np.asarray(shift, dtype=np.float64)[:, None, :]
    scale = np.asarray(scale, dtype=np.float64)[:, None, :]
    return xn * (1.0 + scale) + shift


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up with silu(a) = a / (1 + exp(-a)) (reading: the usual SwiGLU gating)."""
    a = np.asarray(gate, dtype=np.float64)
    b = np.asarray(up, dtype=np.float64)
    return a / (1.0 + np.exp(-a)) * b


# --------------------------------------------------------------------------------------------
# (6) Cache-DiT residual-change gate  ["MiniMax-H3 的 6.24 倍…", section 6.24 倍里…: Cache-DiT
#     compares the residual change between adjacent denoising steps and, when it is small,
#     reuses the cached middle-block results; the conservative setting has a tighter threshold
#     and caches at most one step in a row, the stride setting a looser one and at most three]
# --------------------------------------------------------------------------------------------


def residual_change(cur: np.ndarray, prev: np.ndarray):
    """(sum |cur - prev|, sum |prev|) over all elements; the relative change is their ratio.
    Reading: the pages say "residual change" without a norm; the L1 relative change is used."""
    cur = np.asarray(cur, dtype=np.float64)
    prev = np.asarray(prev, dtype=np.float64)
    return float(np.abs(cur - prev).sum()), float(np.abs(prev).sum())


class CacheGate:
    """Per-step reuse decision. The first step always computes (nothing to compare with). A step
    reuses the cache iff its relative change is below `threshold` and fewer than
    `max_consecutive` steps in a row have already been reused; a computed step resets the run.
    The thresholds are not on the pages (decision parity unpinned)."""

    def __init__(self, threshold: float, max_consecutive: int):
        if not (threshold >= 0.0) or max_consecutive < 0:
            raise ValueError("threshold >= 0 and max_consecutive >= 0 required")
        self.threshold = float(threshold)
        self.max_consecutive = int(max_consecutive)
        self.consecutive = 0
        self.steps = 0

    def decide(self, rel_change: float) -> bool:
        reuse = (self.steps > 0 and rel_change < self.threshold
                 and self.consecutive < self.max_consecutive)
        self.consecutive = self.consecutive + 1 if reuse else 0
        self.steps += 1
        return reuse


# --------------------------------------------------------------------------------------------
# (7) FP8 (e4m3) attention
#     ["智東西…H3 Lightning" (hao.cnyes.com), section "02. 從50步壓到9步三層最佳化實現12倍提速":
#     SageAttention2 speeds up the attention computation; "VDN-MiniMax-H3：基于MiniMax H3的视频
#     生成加速开源项目" (aipuzi.cn), sections "二、功能特色" and "三、技术细节": FP8 quantized
#     inference]. The pages give no quantization rule; the readings taken are stated below.
# --------------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The 256 values of the OCP fp8 e4m3 format (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the all-ones exponent with
    mantissa 7 is NaN and there is no infinity), indexed by the byte code."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value, ties to the even mantissa. Magnitudes that round above
    448 (from 464 exclusive) have no e4m3 value and become NaN (no saturation)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.empty_like(a)
    normal = a >= 2.0 ** -6
    # normal range: a = f * 2^e with f in [1, 2); mantissa steps of 2^(e-3)
    e = np.floor(np.log2(np.where(normal, a, 1.0)))
    # guard log2 rounding at exact powers of two
    e = np.where(np.where(normal, a, 1.0) < 2.0 ** e, e - 1, e)
    e = np.where(np.where(normal, a, 1.0) >= 2.0 ** (e + 1), e + 1, e)
    step = 2.0 ** (e - 3)
    out[normal] = (np.rint(a / step) * step)[normal]          # np.rint: ties to even
    sub = ~normal
    out[sub] = np.rint(a[sub] / 2.0 ** -9) * 2.0 ** -9        # subnormal grid 2^-9 (2^-6 exact)
    out = np.where(out > E4M3_MAX, np.nan, out)
    return np.copysign(out, x)


POW2_SCALE_MIN_EXP = -60


def pow2_scale(amax: np.ndarray) -> np.ndarray:
    """Smallest power of two s with amax <= 448 * s (1 where amax is 0), but not below 2^-60.
    Reading: power-of-two scales keep the scaling exact, so a quantised value is the e4m3
    rounding of x / s; the floor keeps the product of two scales a normal float32 (it only
    matters for blocks whose largest magnitude is below 448 * 2^-60)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(amax > 0, amax, 1.0))           # amax = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 9 + (m > 0.875), POW2_SCALE_MIN_EXP)   # 448 = 0.875 * 2^9
    return np.where(amax > 0, np.ldexp(1.0, e), 1.0)


def quantize_blocks(x: np.ndarray, block_size: int = 64):
    """Per (batch, head, 64-token block) e4m3 quantisation of q or k [B, N, Hd, D]: returns the
    e4m3 values x8 (same shape, x ~ x8 * s) and the scales s [B, Hd, nB] (reading: one scale per
    block, the granularity SubBlock works at)."""
    x = np.asarray(x, dtype=np.float64)
    b_len, n, h_len, d = x.shape
    nb = n_blocks_of(n, block_size)
    scales = np.empty((b_len, h_len, nb))
    x8 = np.empty_like(x)
    for i in range(nb):
        sl = slice(i * block_size, min((i + 1) * block_size, n))
        amax = np.abs(x[:, sl]).max(axis=(1, 3))                # [B, Hd]
        s = pow2_scale(amax)
        scales[:, :, i] = s
        x8[:, sl] = e4m3_round(x[:, sl] / s[:, None, :, None])
    return x8, scales


def quantize_channels(v: np.ndarray):
    """Per (batch, head, channel) e4m3 quantisation of v [B, N, Hd, D] over all tokens: returns
    v8 (v ~ v8 * s) and s [B, Hd, D] (reading: the P.V product then rescales each output channel
    once)."""
    v = np.asarray(v, dtype=np.float64)
    s = pow2_scale(np.abs(v).max(axis=1))                       # [B, Hd, D]
    return e4m3_round(v / s[:, None]), s


def _fp8_rows(q8, sq, k8, sk, v8, sv, qrows, keys, block_size, detail=False):
    """Quantised attention of query rows qrows over key ids keys for one (batch, head):
    x = (q8 . k8) * s_q * s_k * log2(e) / sqrt(D); m = ceil(max x) per row;
    P = e4m3(2^(8 + x - m)); O = (P @ v8) * s_v / sum(P); LSE = ln2 * (m - 8 + log2 sum(P)).
    With detail, also the two quantities that bound the effect of one probability taking the
    neighbouring e4m3 code: the row's largest weight max P / sum(P), and per channel the largest
    distance max_j |v_j - O| of a value from the output."""
    d = q8.shape[-1]
    s = (q8[qrows] @ k8[keys].T) * sq[qrows // block_size][:, None] * sk[keys // block_size][None, :]
    x = s * (math.log2(math.e) / math.sqrt(d))
    m = np.ceil(x.max(axis=1, keepdims=True))
    p = e4m3_round(np.exp2(8.0 + x - m))
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v8[keys]) * sv[None, :] / l
    lse = math.log(2.0) * (m[:, 0] - 8.0 + np.log2(l[:, 0]))
    if not detail:
        return o, lse
    vals = v8[keys] * sv[None, :]                                       # [keys, D]
    dev = np.maximum(np.abs(vals.max(axis=0)[None, :] - o), np.abs(vals.min(axis=0)[None, :] - o))
    return o, lse, p.max(axis=1) / l[:, 0], dev


def attention_fp8(q, k, v, block_size: int = 64):
    """Dense attention on e4m3-quantised q, k (per 64-token block), v (per channel), with the
    probabilities quantised to e4m3 as 2^(8 + x - m), m the row max rounded up to an integer
    (reading: the probabilities then fill the e4m3 range [2^-9, 256], and a running max that
    only takes integer values moves them by exact powers of two). Returns (O, lse)."""
    q8, sq = quantize_blocks(q, block_size)
    k8, sk = quantize_blocks(k, block_size)
    v8, sv = quantize_channels(v)
    b_len, n, h_len, d = q8.shape
    out = np.empty((b_len, n, h_len, v8.shape[-1]))
    lse = np.empty((b_len, h_len, n))
    allk = np.arange(n)
    for b in range(b_len):
        for h in range(h_len):
            for r0 in range(0, n, 256):
                rows = np.arange(r0, min(r0 + 256, n))
                out[b, rows, h], lse[b, h, rows] = _fp8_rows(q8[b, :, h], sq[b, h], k8[b, :, h], sk[b, h],
                                                           v8[b, :, h], sv[b, h], rows, allk, block_size)
    return out, lse


def sparse_attention_fp8(q, k, v, block_idx, block_size: int = 64):
    """Block-sparse attention on the same quantised tensors: query block i attends to the key
    blocks block_idx[b, h, i, :] only (row max over those keys)."""
    q8, sq = quantize_blocks(q, block_size)
    k8, sk = quantize_blocks(k, block_size)
    v8, sv = quantize_channels(v)
    b_len, n, h_len, d = q8.shape
    nb = n_blocks_of(n, block_size)
    out = np.empty((b_len, n, h_len, v8.shape[-1]))
    lse = np.empty((b_len, h_len, n))
    for b in range(b_len):
        for h in range(h_len):
            for i in range(nb):
                rows = np.arange(i * block_size, min((i + 1) * block_size, n))
                keys = block_token_ids(block_idx[b, h, i], block_size, n)
                out[b, rows, h], lse[b, h, rows] = _fp8_rows(q8[b, :, h], sq[b, h], k8[b, :, h], sk[b, h],
                                                           v8[b, :, h], sv[b, h], rows, keys, block_size)
    return out, lse


def attention_fp8_rows(q, k, v, b: int, h: int, qblock: int, block_idx=None, block_size: int = 64,
                       detail: bool = False):
    """One query block of attention_fp8 (block_idx None) or sparse_attention_fp8, for sampled
    comparisons on long sequences (the quantisation is the same as on the full tensors)."""
    q8, sq = quantize_blocks(q[b:b + 1, :, h:h + 1], block_size)
    k8, sk = quantize_blocks(k[b:b + 1, :, h:h + 1], block_size)
    v8, sv = quantize_channels(v[b:b + 1, :, h:h + 1])
    n = q8.shape[1]
    rows = np.arange(qblock * block_size, min((qblock + 1) * block_size, n))
    keys = np.arange(n) if block_idx is None else block_token_ids(block_idx, block_size, n)
    return _fp8_rows(q8[0, :, 0], sq[0, 0], k8[0, :, 0], sk[0, 0], v8[0, :, 0], sv[0, 0], rows, keys, block_size,
                     detail)


def attention_fp8_detail(q, k, v, block_idx=None, block_size: int = 64):
    """attention_fp8 (block_idx None) or sparse_attention_fp8 with the per-row bound quantities
    of _fp8_rows: returns (O, lse, wmax [B, Hd, N], dev [B, N, Hd, D])."""
    q8, sq = quantize_blocks(q, block_size)
    k8, sk = quantize_blocks(k, block_size)
    v8, sv = quantize_channels(v)
    b_len, n, h_len, d = q8.shape
    nb = n_blocks_of(n, block_size)
    out = np.empty((b_len, n, h_len, v8.shape[-1]))
    dev = np.empty_like(out)
    lse = np.empty((b_len, h_len, n))
    wmax = np.empty((b_len, h_len, n))
    for b in range(b_len):
        for h in range(h_len):
            for i in range(nb):
                rows = np.arange(i * block_size, min((i + 1) * block_size, n))
                keys = np.arange(n) if block_idx is None else block_token_ids(block_idx[b, h, i], block_size, n)
                o, l_, w, dv = _fp8_rows(q8[b, :, h], sq[b, h], k8[b, :, h], sk[b, h], v8[b, :, h], sv[b, h],
                                         rows, keys, block_size, detail=True)
                out[b, rows, h], lse[b, h, rows], wmax[b, h, rows], dev[b, rows, h] = o, l_, w, dv
    return out, lse, wmax, dev
