// Fused QK RMSNorm + 3D RoPE for gfx950.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section
// "先把近两倍的免费收益拿走": QK RMSNorm and 3D RoPE run as one fused kernel, which removes the
// intermediate tensor and its memory traffic without changing the math.
//
// Design: a pure streaming kernel, bound by HBM bandwidth. Each row (one head of one token of q
// or k) is head_dim bf16 values = D/8 chunks of 16 bytes; D/8 consecutive lanes own one row, one
// 16-byte chunk each, so every row is read and written as whole contiguous 128/256-byte runs.
// A thread keeps its chunk index across kRows rows of the same token, so the four rotation
// angles of its chunk are computed once (in double, reduced to [-pi, pi], then one float sincos)
// and reused kRows times. All kRows loads are issued before any arithmetic to keep many bytes in
// flight. The sum of squares is reduced across the D/8 lanes of a row with cross-lane shuffles.
#include "device_util.h"
#include "kernels.h"
#include "norm_rope_math.h"

namespace h3attn {
namespace {

// Row and token streams are touched once: non-temporal loads and stores keep them out of the
// caches (measured 2-4 % faster than ordinary ones).
template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// kRows rows (heads of q, then of k) per thread, kThreads threads per workgroup.
template <int D, int kRows, int kThreads>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(NormRopeArgs a, RopeTable tab) {
  constexpr int TPR = D / 8;                 // lanes per row
  constexpr int TOK_PER_BLOCK = kThreads / TPR;
  const int c = threadIdx.x % TPR;           // chunk index inside the row: channels 8c .. 8c+7
  // consecutive workgroups take the row groups of the same tokens, so one token's q and k rows
  // are read close together in time
  const int n_rg = (2 * a.heads + kRows - 1) / kRows;
  const int rg = (int)(blockIdx.x % n_rg);
  const int64_t tok = (int64_t)(blockIdx.x / n_rg) * TOK_PER_BLOCK + threadIdx.x / TPR;  // over batch*n_tokens
  const int64_t total_tok = (int64_t)a.batch * a.n_tokens;
  if (tok >= total_tok) return;              // whole row groups exit together (TPR divides 64)

  const int rows_total = 2 * a.heads;
  const int r0 = rg * kRows;

  // Issue all loads first.
  u32x4 x[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = r0 + i;
    if (r < rows_total) {
      const bool is_k = r >= a.heads;
      const int head = is_k ? r - a.heads : r;
      const uint16_t* src = (is_k ? a.k_in : a.q_in) + ((tok * a.heads + head) * D + 8 * c);
      x[i] = load_stream(reinterpret_cast<const u32x4*>(src));
    }
  }

  // Token coordinates on the latent grid (n = (t*H + h)*W + w).
  int64_t pos[3];
  rope_position(tok % a.n_tokens, a.grid_h, a.grid_w, pos);
  float cs[4], sn[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) rope_pair(pos, 4 * c + p, tab, cs[p], sn[p]);

  float wq[8], wk[8];
  {
    const f32x4* wqp = reinterpret_cast<const f32x4*>(a.q_weight + 8 * c);
    const f32x4* wkp = reinterpret_cast<const f32x4*>(a.k_weight + 8 * c);
    f32x4 q0 = wqp[0], q1 = wqp[1], k0 = wkp[0], k1 = wkp[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) { wq[j] = q0[j]; wq[4 + j] = q1[j]; wk[j] = k0[j]; wk[4 + j] = k1[j]; }
  }

  const float inv_d = 1.0f / (float)D;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = r0 + i;
    if (r >= rows_total) break;  // uniform across the row group
    const bool is_k = r >= a.heads;
    const u32x4 o = norm_rope_chunk<TPR>(x[i], is_k ? wk : wq, cs, sn, inv_d, a.eps);
    const int head = is_k ? r - a.heads : r;
    uint16_t* dst = (is_k ? a.k_out : a.q_out) + ((tok * a.heads + head) * D + 8 * c);
    store_stream(reinterpret_cast<u32x4*>(dst), o);
  }
}

}  // namespace

namespace {
template <int D, int kRows, int kThreads>
void launch_norm_rope(const NormRopeArgs& a, const RopeTable& table, hipStream_t stream) {
  const int64_t total_tok = (int64_t)a.batch * a.n_tokens;
  const int64_t row_groups = (2 * a.heads + kRows - 1) / kRows;
  constexpr int tpb = kThreads / (D / 8);  // tokens per workgroup
  const dim3 grid((unsigned)((total_tok + tpb - 1) / tpb * row_groups));
  hipLaunchKernelGGL((qk_norm_rope_kernel<D, kRows, kThreads>), grid, dim3(kThreads), 0, stream, a, table);
}
}  // namespace

// Large launches: 12 rows x 128 threads; below a million head rows (a single frame), where the
// launch is short and its ramp matters, 8 rows x 256 threads (measured best at each size).
void launch_qk_norm_rope(const NormRopeArgs& a, const RopeTable& table, hipStream_t stream) {
  const bool large = (int64_t)a.batch * a.n_tokens * 2 * a.heads >= (int64_t)1 << 20;
  if (a.head_dim == 128) {
    if (large) launch_norm_rope<128, 12, 128>(a, table, stream);
    else launch_norm_rope<128, 8, 256>(a, table, stream);
  } else {
    if (large) launch_norm_rope<64, 12, 128>(a, table, stream);
    else launch_norm_rope<64, 8, 256>(a, table, stream);
  }
}

}  // namespace h3attn
