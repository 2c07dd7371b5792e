/*
 * h3attn — attention hot path of a MiniMax-H3-class video diffusion transformer on AMD MI355X
 * (gfx950 / CDNA4): fused QK RMSNorm + 3D RoPE, dense bf16 self-attention, SubBlock block
 * selection and block-sparse attention.
 *
 * Sources (web pages, cited by title and section):
 *  [P3] "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai/posts/minimax-h3-speed-quality)
 *       section "先把近两倍的免费收益拿走": the lossless runtime's fused QK RMSNorm + 3D RoPE
 *       kernel (fusion leaves the math unchanged);
 *       section "6.24 倍里，真正有损的部分大约是三倍": SubBlock — queries and keys cut into
 *       64-token blocks, low-contribution key blocks estimated and dropped, the rest fed to a
 *       block-sparse attention kernel; sparsity = fraction of key blocks dropped.
 *  [P4] "MiniMax-H3 在 8×H200 上基准测试：无损加速 1.95×，最高 6.24×" (chat-gpts.plus/?p=43161)
 *       section "为什么重要": attention over very long latent sequences is a main cost.
 *  [P2] mhpq.cn/news/447544, section 2.1: a video latent holds one 8x-downsampled latent per
 *       frame, so the token count grows with frame count.
 *
 * Conventions for every call:
 *  - Tensor pointers are caller-owned DEVICE pointers, 16-byte aligned. q, k, v and outputs are
 *    contiguous [batch, n_tokens, heads, head_dim] ("BSHD") bf16 (raw 16-bit patterns).
 *  - Token n of a T x H x W latent grid sits at n = (t*H + h)*W + w.
 *  - Every call validates all arguments on the host first; on error it returns a nonzero
 *    status, writes nothing, launches nothing, and h3attn_last_error() describes the problem.
 *  - Calls are asynchronous on `stream` (NULL = the default stream); none synchronises, none
 *    allocates device memory, none changes the current device. After a launch,
 *    a HIP launch error is reported as H3ATTN_ERR_LAUNCH.
 *  - head_dim must be 64 or 128; block_size must be 64.
 *  - The library keeps no global state except a thread-local error string.
 */
#ifndef H3ATTN_H_
#define H3ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t h3attn_bf16; /* raw bfloat16 bits */

typedef struct {
  int32_t t, h, w; /* latent grid; n_tokens = t*h*w */
} h3attn_grid;

typedef enum {
  H3ATTN_OK = 0,
  H3ATTN_ERR_INVALID_ARGUMENT = 1,
  H3ATTN_ERR_UNSUPPORTED = 2,
  H3ATTN_ERR_LAUNCH = 3
} h3attn_status;

/* Library version string, e.g. "h3attn 0.1.0 gfx950". Never NULL. */
const char* h3attn_version(void);

/* Message for the last failing call on this thread ("" if none). Never NULL. */
const char* h3attn_last_error(void);

/* Key blocks kept per query block at a given sparsity (fraction of key blocks dropped)
 * [P3 "6.24 倍里…"]: min(n, max(1, ceil((1 - s) * n - 1e-9))), computed in double.
 * Returns -1 if n_kblocks <= 0 or sparsity is outside [0, 1). */
int32_t h3attn_keep_count(int32_t n_kblocks, double sparsity);

/* Device workspace bytes that h3attn_subblock_select needs, O(batch * heads * nB * head_dim):
 * the pooled block means of q and k in float64 ([batch, heads, nB, head_dim] each), their
 * base-256 integer digits (3 bytes per channel), a power-of-two exponent and two norms per
 * block, per-head key maxima and a list of rows for the exact fallback, each region 256-byte
 * aligned (22 * head_dim + 28 bytes per (batch, head, block), plus 16 bytes per (batch, head);
 * the digit, exponent and norm regions padded to a multiple of 32 blocks). No score matrix is stored:
 * block scores live on chip. Returns 0 on invalid sizes. */
size_t h3attn_select_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens,
                                     int32_t head_dim, int32_t block_size);

/* Fused per-head RMSNorm then 3D RoPE of q and k [P3 "先把近两倍的免费收益拿走"].
 * For every (b, n, head) row x of q (resp. k):
 *   y = x * w / sqrt(mean(x^2) + eps)          (w = q_weight resp. k_weight, float32 [head_dim])
 *   head_dim is split into contiguous sections [d_t | d_h | d_w] (each even, sum = head_dim);
 *   inside section a, channel pair (2j, 2j+1) is rotated by angle p_a * rope_theta^(-2j/d_a),
 *   p_a being the token's integer t, h or w coordinate.
 * Computed in float32 from the bf16 input, rounded once (nearest-even) to bf16.
 * q_out / k_out may equal q_in / k_in (in place); otherwise the buffers must not overlap.
 * Errors: null or misaligned pointer, batch/heads <= 0, grid sizes <= 0, odd or mismatched
 * sections, eps < 0, theta <= 0 -> INVALID_ARGUMENT; head_dim not 64/128 -> UNSUPPORTED. */
h3attn_status h3attn_qk_norm_rope(const h3attn_bf16* q_in, const h3attn_bf16* k_in,
                                  h3attn_bf16* q_out, h3attn_bf16* k_out,
                                  const float* q_weight, const float* k_weight,
                                  int32_t batch, int32_t heads, int32_t head_dim, h3attn_grid grid,
                                  int32_t d_t, int32_t d_h, int32_t d_w,
                                  float rope_theta, float eps, hipStream_t stream);

/* Dense non-causal self-attention [P4 "为什么重要"]: per (b, head),
 *   out = softmax(q k^T / sqrt(head_dim)) v,   lse = ln sum_j exp(q.k_j / sqrt(head_dim)).
 * bf16 MFMA products, float32 accumulation and softmax; P is rounded to bf16 before P.V.
 * out: bf16 BSHD (must not overlap the inputs). lse: float32 [batch, heads, n_tokens] or NULL.
 * Errors: null/misaligned pointer, sizes <= 0 -> INVALID_ARGUMENT; head_dim not 64/128 ->
 * UNSUPPORTED. */
h3attn_status h3attn_dense_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                               h3attn_bf16* out, float* lse,
                               int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                               hipStream_t stream);

/* SubBlock key-block selection [P3 "6.24 倍里…"]. Blocks are block_size consecutive tokens
 * (the last one may be partial). Block importance is estimated, since the pages leave it open,
 * as the dot product of the mean query of block i and the mean key of block j (over sqrt(D));
 * per query block i the `keep` highest-scoring key blocks are kept, equal scores ranking the
 * lower key index first. The kept sets are those of the float64 scores of the float64 block
 * means: every score is bounded on the int8 matrix cores (exact integer products of the means'
 * base-256 digits, with a rigorous error bound) and only the entries whose bound straddles the
 * keep-th score are decided on their float64 value; no score matrix is written to memory.
 * block_idx: int32 [batch, heads, nB, keep], each row ascending. keep must equal
 * h3attn_keep_count(nB, sparsity). workspace: device buffer of at least
 * h3attn_select_workspace_bytes(...) bytes, 256-byte aligned; its contents are scratch.
 * Errors: bad pointers/sizes, sparsity outside [0,1), keep mismatch, workspace too small ->
 * INVALID_ARGUMENT; head_dim not 64/128, block_size != 64 or nB > 19968 (a row of float64
 * scores must fit in one CU's LDS for the exact fallback) -> UNSUPPORTED. */
h3attn_status h3attn_subblock_select(const h3attn_bf16* q, const h3attn_bf16* k,
                                     int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                     int32_t block_size, double sparsity, int32_t keep,
                                     int32_t* block_idx, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* h3attn_qk_norm_rope and the pooling step of h3attn_subblock_select in one pass [P3 "先把近两倍的
 * 免费收益拿走": a fused pass saves an intermediate tensor's memory traffic; here it also saves the
 * selection's re-read of q' and k']. Writes q_out, k_out exactly as h3attn_qk_norm_rope does (the same bits) and
 * the block means of q_out and k_out (with their digits, exponents and norms) into workspace, which
 * must then be passed, untouched and with the same batch, heads, n_tokens (grid.t * grid.h * grid.w),
 * head_dim and block_size, to h3attn_subblock_select_pooled. workspace: as h3attn_subblock_select
 * (at least h3attn_select_workspace_bytes(...) bytes, 256-byte aligned).
 * Errors: those of h3attn_qk_norm_rope and of h3attn_subblock_select's workspace and size checks. */
h3attn_status h3attn_qk_norm_rope_pool(const h3attn_bf16* q_in, const h3attn_bf16* k_in,
                                       h3attn_bf16* q_out, h3attn_bf16* k_out,
                                       const float* q_weight, const float* k_weight,
                                       int32_t batch, int32_t heads, int32_t head_dim, h3attn_grid grid,
                                       int32_t d_t, int32_t d_h, int32_t d_w,
                                       float rope_theta, float eps, int32_t block_size,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The rest of h3attn_subblock_select [P3 "6.24 倍里…"] on a workspace that h3attn_qk_norm_rope_pool
 * has just filled: the same kept sets, bit for bit, as h3attn_subblock_select on that call's
 * q_out and k_out. Arguments and errors as h3attn_subblock_select without q and k; a workspace not
 * filled that way gives undefined (but in-bounds) results. A filled workspace serves one call: the
 * call rewrites the key blocks' exponents in it in place. */
h3attn_status h3attn_subblock_select_pooled(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                            int32_t block_size, double sparsity, int32_t keep,
                                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* Block-sparse attention [P3 "6.24 倍里…"]: the queries of block i attend only to the tokens of
 * the key blocks block_idx[b, head, i, 0..keep-1], with the softmax renormalised over those
 * tokens (a partial last key block contributes only its valid tokens). Same numerics and
 * outputs as h3attn_dense_fwd. block_idx rows must hold `keep` distinct indices in [0, nB);
 * their order does not matter: each row's kept blocks are visited in ascending key order, so
 * the result is bit-identical for any order (and, with every block kept, to h3attn_dense_fwd).
 * Behaviour for other index values is undefined. One workgroup serves four consecutive query
 * blocks and streams the union of their kept key blocks once.
 * Errors: as h3attn_dense_fwd, plus keep outside [1, nB] -> INVALID_ARGUMENT and
 * block_size != 64 -> UNSUPPORTED. */
h3attn_status h3attn_block_sparse_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                      const int32_t* block_idx, int32_t keep,
                                      h3attn_bf16* out, float* lse,
                                      int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                      int32_t block_size, hipStream_t stream);

/* h3attn_block_sparse_fwd with a choice of which four query blocks share a workgroup (a schedule
 * choice only: the result is bit-identical for every group_stride S). S = 1 is
 * h3attn_block_sparse_fwd (blocks i..i+3); S > 1 takes the blocks i, i+S, i+2S, i+3S. For a video
 * latent of T x H x W tokens whose frames are whole 64-token blocks, S = H*W/64 groups the same
 * spatial position of four consecutive frames, whose kept sets overlap more (79 % against 58 %
 * for neighbouring blocks on the smooth-field workloads), so fewer union tiles are streamed.
 * Errors: as h3attn_block_sparse_fwd, plus group_stride outside [1, nB] -> INVALID_ARGUMENT. */
h3attn_status h3attn_block_sparse_grouped_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                              const int32_t* block_idx, int32_t keep,
                                              h3attn_bf16* out, float* lse,
                                              int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                              int32_t block_size, int32_t group_stride, hipStream_t stream);

/* Validation of a caller-built kept set for h3attn_block_sparse_fwd / _grouped_fwd /
 * h3attn_fp8_block_sparse_fwd, which take it as given (behaviour for bad indices is undefined).
 * For every row r = (b * heads + head) * n_blocks + i of block_idx ([batch, heads, n_blocks,
 * keep] int32) writes row_flags[r] (uint8, device, caller-owned): 0 for a valid row, else bit 0
 * (an index outside [0, n_blocks)) | bit 1 (an index repeated in the row). Asynchronous on
 * `stream`; the caller reads the flags back. Errors: null or misaligned pointers, sizes <= 0,
 * keep outside [1, n_blocks] -> INVALID_ARGUMENT; n_blocks > 2^20 or batch*heads*n_blocks >= 2^31
 * -> UNSUPPORTED. */
h3attn_status h3attn_check_block_idx(const int32_t* block_idx, int32_t batch, int32_t heads, int32_t n_blocks,
                                     int32_t keep, uint8_t* row_flags, hipStream_t stream);

/* ---- Threshold-mode SubBlock selection with a variable number of kept blocks per row ----
 * "MiniMax-H3 在 8×H200 上基准测试…" (chat-gpts.plus), section "事件核心" describes SubBlock as
 * skipping the attention blocks that score below a threshold. The pages give no rule; this mode
 * keeps, for query block i, every key block j whose score (the same pooled estimate as
 * h3attn_subblock_select) is at least max_j score(i, j) - tau, tau >= 0 (tau = +inf keeps all).
 * Kept sets are returned in CSR form over the rows r = (b * heads + head) * nB + i:
 * row_ptr[r] .. row_ptr[r+1] index ascending key-block ids in col_idx. Selection is two calls on
 * the same workspace, so the caller can size col_idx between them. */

/* Workspace bytes for the threshold calls: the select workspace plus a per-row threshold
 * (float64) and count (int64), each region 256-byte aligned. 0 on invalid sizes. */
size_t h3attn_threshold_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens,
                                        int32_t head_dim, int32_t block_size);

/* Pass 1: pools, per-row exact maxima, thresholds and counts (scores recomputed on chip, the
 * entries near the threshold decided on their float64 score); writes row_ptr (int64, B*heads*nB + 1
 * entries, row_ptr[0] = 0, last entry = total kept count). Errors: as h3attn_subblock_select
 * (nB > 19968 -> UNSUPPORTED included), plus tau < 0 or NaN -> INVALID_ARGUMENT. */
h3attn_status h3attn_subblock_threshold_count(const h3attn_bf16* q, const h3attn_bf16* k,
                                              int32_t batch, int32_t heads, int64_t n_tokens,
                                              int32_t head_dim, int32_t block_size, double tau,
                                              int64_t* row_ptr, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/* Pass 2: recomputes the scores and fills col_idx (int32), deciding every entry as pass 1 did,
 * from the workspace left by pass 1 (same sizes, same workspace,
 * same stream, nothing in between that writes the workspace). Entries at positions >=
 * col_capacity are not written: size col_idx from row_ptr's last entry. */
h3attn_status h3attn_subblock_threshold_fill(int32_t batch, int32_t heads, int64_t n_tokens,
                                             int32_t head_dim, int32_t block_size,
                                             const int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Block-sparse attention with a CSR kept set per query block (rows as above; indices distinct
 * and in [0, nB), any order, visited in ascending key order). Same numerics as
 * h3attn_block_sparse_fwd. A row with no kept block yields zeros and lse = -inf. */
h3attn_status h3attn_block_sparse_csr_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                          const int64_t* row_ptr, const int32_t* col_idx,
                                          h3attn_bf16* out, float* lse,
                                          int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                          int32_t block_size, hipStream_t stream);

/* h3attn_block_sparse_csr_fwd with the group_stride of h3attn_block_sparse_grouped_fwd. */
h3attn_status h3attn_block_sparse_csr_grouped_fwd(const h3attn_bf16* q, const h3attn_bf16* k,
                                                  const h3attn_bf16* v, const int64_t* row_ptr,
                                                  const int32_t* col_idx, h3attn_bf16* out, float* lse,
                                                  int32_t batch, int32_t heads, int64_t n_tokens,
                                                  int32_t head_dim, int32_t block_size, int32_t group_stride,
                                                  hipStream_t stream);

/* Validation of caller-built CSR kept sets for the two CSR calls above: for every row r of the
 * batch*heads*n_blocks rows writes row_flags[r] (uint8, device, caller-owned): 0 for a valid row,
 * else bit 0 (an index outside [0, n_blocks)) | bit 1 (an index repeated in the row) | bit 2
 * (row_ptr[r] < 0, row_ptr[r+1] < row_ptr[r] or row_ptr[r+1] > col_capacity, the number of int32
 * entries col_idx holds; the row's indices are then not read). Asynchronous on `stream`.
 * Errors: as h3attn_check_block_idx (col_idx may be NULL only when col_capacity is 0). */
h3attn_status h3attn_check_csr(const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity, int32_t batch,
                               int32_t heads, int32_t n_blocks, uint8_t* row_flags, hipStream_t stream);

/* ---- The other fused per-block ops of the lossless runtime ----
 * "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section "先把近两倍的免费收益拿走":
 * besides QK RMSNorm + 3D RoPE the runtime fuses AdaLN and SwiGLU. The pages give no formulas;
 * these are the usual DiT forms. Both compute in float32 from bf16 and round once to bf16. */

/* AdaLN modulation over the hidden axis of x [batch, n_tokens, hidden] (bf16):
 *   y = (x - mean) / sqrt(var + eps) * (1 + scale[b]) + shift[b]
 * with the biased variance of the row and no affine weights of its own; shift and scale are
 * float32 [batch, hidden]. out may equal x. hidden must be a multiple of 8, at most 16384.
 * Errors: null/misaligned pointers, sizes <= 0, eps < 0 -> INVALID_ARGUMENT; hidden not a
 * multiple of 8 or above 16384 -> UNSUPPORTED. */
h3attn_status h3attn_adaln_modulate(const h3attn_bf16* x, const float* shift, const float* scale,
                                    h3attn_bf16* out, int32_t batch, int64_t n_tokens, int32_t hidden,
                                    float eps, hipStream_t stream);

/* SwiGLU gating: out[r, c] = silu(gate[r, c]) * up[r, c], silu(a) = a / (1 + exp(-a)), for
 * rows x width elements; gate and up rows start every gate_row_stride / up_row_stride elements
 * (so they may be the two halves of one [rows, 2*width] tensor), out is contiguous
 * [rows, width]. out may equal gate or up when that operand's row stride equals width.
 * width and both strides must be multiples of 8. Errors: null/misaligned pointers, sizes <= 0,
 * strides < width -> INVALID_ARGUMENT; width or a stride not a multiple of 8 -> UNSUPPORTED. */
h3attn_status h3attn_swiglu(const h3attn_bf16* gate, const h3attn_bf16* up, h3attn_bf16* out,
                            int64_t rows, int32_t width, int64_t gate_row_stride, int64_t up_row_stride,
                            hipStream_t stream);

/* ---- Cache-DiT residual-change gate ----
 * "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section "6.24 倍里，真正有损的部分大约
 * 是三倍": Cache-DiT measures the residual change between adjacent denoising steps and, when it is
 * small, reuses cached middle-block results; the conservative setting has a tighter threshold and
 * caches at most one step in a row, the stride setting a looser one and at most three. The pages
 * give neither the norm nor the thresholds: the change is the L1 ratio
 * sum|cur - prev| / sum|prev|, and thresholds are the caller's. */

/* Workspace bytes for h3attn_residual_change on n elements (two float64 per partial block). */
size_t h3attn_residual_workspace_bytes(int64_t n);

/* result (DEVICE pointer, 2 doubles) <- { sum |cur - prev|, sum |prev| } over n bf16 elements of
 * two contiguous tensors. Per-thread sums in float32, everything above in float64, combined in a
 * fixed order (deterministic). Errors: null/misaligned pointers, n <= 0, small workspace ->
 * INVALID_ARGUMENT. */
h3attn_status h3attn_residual_change(const h3attn_bf16* cur, const h3attn_bf16* prev, int64_t n,
                                     double* result, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* h3attn_residual_change without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the partial sums live in a file-scope device array of 2^17 pairs (2 MB, held by every GPU the
 * library runs on until the process ends), so n is limited to 2^33 elements; larger n ->
 * INVALID_ARGUMENT. Nothing is allocated and nothing needs clearing (every partial is written
 * before it is read). Calls on one GPU share the array: calls that overlap on one GPU (two
 * streams, two host threads) race. Same results as h3attn_residual_change, bit for bit.
 * Errors: as h3attn_residual_change; a failed lookup of the array -> LAUNCH. */
h3attn_status h3attn_residual_change_noalloc(const h3attn_bf16* cur, const h3attn_bf16* prev, int64_t n,
                                             double* result, hipStream_t stream);

/* Host-side reuse policy (plain C state; no GPU work). */
typedef struct {
  double threshold;        /* reuse only when the relative change is strictly below this */
  int32_t max_consecutive; /* at most this many reused steps in a row (1: conservative, 3: stride) */
  int32_t consecutive;     /* reused steps in the current run */
  int64_t steps;           /* steps decided so far */
} h3attn_cache_gate;

/* Initialise a gate; INVALID_ARGUMENT if threshold < 0 (or NaN), max_consecutive < 0 or gate is NULL. */
h3attn_status h3attn_cache_gate_init(h3attn_cache_gate* gate, double threshold, int32_t max_consecutive);

/* Decide one step: returns 1 to reuse the cached result, 0 to compute (always 0 on the first
 * step, when there is nothing to compare with), -1 if gate is NULL. A computed step resets the
 * run of reused steps. */
int32_t h3attn_cache_gate_decide(h3attn_cache_gate* gate, double rel_change);

/* Decide one step from the two sums h3attn_residual_change wrote (read back by the caller into a
 * HOST array): the relative change is sums[0] / sums[1], or +infinity (compute) when sums[1] is
 * not positive or sums is NULL (the first step, with nothing to compare with). Returns as
 * h3attn_cache_gate_decide. */
int32_t h3attn_cache_gate_decide_sums(h3attn_cache_gate* gate, const double* sums);

/* ---- FP8 (OCP e4m3) attention ----
 * "智東西…H3 Lightning" (hao.cnyes.com), section "02. 從50步壓到9步三層最佳化實現12倍提速":
 * SageAttention2 speeds up the attention computation; "VDN-MiniMax-H3：基于MiniMax H3的视频生成
 * 加速开源项目" (aipuzi.cn), sections "二、功能特色" / "三、技术细节": FP8 quantised inference. The
 * pages give no quantisation rule; this one uses power-of-two scales (so scaling is exact):
 *   q, k: per (batch, head, 64-token block), the smallest power of two s >= 2^-60 with
 *         max|x| <= 448 s; codes are the round-to-nearest-even e4m3 values of x / s;
 *   v:    per (batch, head, channel) over all tokens, the same rule;
 *   attention: x = (q8 . k8) * s_q * s_k * log2(e) / sqrt(D); m = the row max of x rounded up
 *   to an integer; P = e4m3(2^(8 + x - m)); O = (P . v8) * s_v / sum(P) (bf16 output);
 *   lse = ln(2) * (m - 8 + log2 sum(P)).
 * Inputs whose magnitudes exceed 448 * 2^60 are not supported (their codes are NaN).
 *
 * Quantised layouts (all bytes are e4m3 codes; every pointer 16-byte aligned):
 *   q8, k8   [batch, n_tokens, heads, head_dim]
 *   v8t      [batch, heads, head_dim, nB * 64]: v transposed; within each 64-key block, key
 *            kappa = 32a + 8b + 4c + d (a, c in {0,1}; b, d in 0..3) is stored at byte
 *            32c + 16a + 4b + d (the order the P.V product reads it); keys >= n_tokens are 0
 *   q_scale, k_scale float32 [batch, heads, nB]; v_scale float32 [batch, heads, head_dim]. */

/* Workspace bytes for h3attn_fp8_quantize (channel maxima of v per 1024-token chunk and the
 * channel scale exponents). 0 on invalid sizes. */
size_t h3attn_fp8_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                  int32_t block_size);

/* Quantises bf16 q, k, v [batch, n_tokens, heads, head_dim] into the layouts above (four
 * kernels on `stream`). Errors: null or misaligned pointers, bad sizes, block_size != 64,
 * workspace smaller than h3attn_fp8_workspace_bytes -> INVALID_ARGUMENT / UNSUPPORTED. */
h3attn_status h3attn_fp8_quantize(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                  uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                  float* q_scale, float* k_scale, float* v_scale,
                                  int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                  int32_t block_size, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dense attention on the quantised tensors (rule above). out: bf16 [batch, n_tokens, heads,
 * head_dim]; lse: nullable float32 [batch, heads, n_tokens]. Errors as h3attn_dense_fwd. */
h3attn_status h3attn_fp8_dense_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                   const float* q_scale, const float* k_scale, const float* v_scale,
                                   h3attn_bf16* out, float* lse, int32_t batch, int32_t heads, int64_t n_tokens,
                                   int32_t head_dim, int32_t block_size, hipStream_t stream);

/* Block-sparse attention on the quantised tensors: query block i attends to the key blocks
 * block_idx[b, head, i, 0..keep-1] only (same index rules as h3attn_block_sparse_fwd and
 * group_stride as h3attn_block_sparse_grouped_fwd, 1 for consecutive blocks; the row max is
 * taken over the kept keys). */
h3attn_status h3attn_fp8_block_sparse_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                          const float* q_scale, const float* k_scale, const float* v_scale,
                                          const int32_t* block_idx, int32_t keep, h3attn_bf16* out, float* lse,
                                          int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                          int32_t block_size, int32_t group_stride, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H_ */
