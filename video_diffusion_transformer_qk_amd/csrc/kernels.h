// Internal launch interface between the C ABI (api.cpp) and the HIP kernels. Arguments are
// already validated by the caller; launchers only compute grid shapes and enqueue kernels.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace h3attn {

// Per-pair RoPE table built on the host: rotation rate (rad per position) and axis (0=t,1=h,2=w)
// of each channel pair. Passed by value as a kernel argument.
struct RopeTable {
  double rate[64];
  int32_t axis[64];
};

struct NormRopeArgs {
  const uint16_t* q_in;
  const uint16_t* k_in;
  uint16_t* q_out;
  uint16_t* k_out;
  const float* q_weight;
  const float* k_weight;
  int64_t n_tokens;     // per batch element
  int32_t batch, heads, head_dim;
  int32_t grid_h, grid_w;
  float eps;
};

void launch_qk_norm_rope(const NormRopeArgs& a, const RopeTable& table, hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_idx;  // null for dense; CSR column indices for the CSR variant
  const int64_t* row_ptr;    // CSR variant only: [B*H*nB + 1]
  uint16_t* out;
  float* lse;                // may be null
  int64_t n_tokens;
  int32_t batch, heads, head_dim;
  int32_t keep;              // sparse only
  int32_t n_blocks;          // sparse only
  int32_t group_stride;      // sparse only: query blocks of a workgroup are i, i+S, i+2S, i+3S (1: consecutive)
};

void launch_dense_fwd(const AttnArgs& a, hipStream_t stream);
void launch_block_sparse_fwd(const AttnArgs& a, hipStream_t stream);
void launch_block_sparse_csr_fwd(const AttnArgs& a, hipStream_t stream);

// Dynamic LDS for one row of nB float64 scores (the selection fallback's row) and for the
// selection kernels' per-row bitmaps: what a CU's 160 KB leaves after the kernels' static LDS;
// longer rows are refused.
constexpr int64_t kSelectRowLdsBytes = 160 * 1024 - 4096;

struct SelectArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t n_tokens;
  int32_t batch, heads, head_dim, block_size, n_blocks, keep;
  int32_t* block_idx;
  // workspace (layout in api.cpp); nBp = nB rounded up to 32
  double* q_mean;      // [B*H, nB, D] float64 block means
  double* k_mean;
  int8_t* q_digits;    // [B*H, nBp/32, D/32, 3, 64 lanes, 16 bytes]: base-256 digits of the means
  int8_t* k_digits;    //   in the int8 MFMA operand order
  int32_t* q_exp;      // [B*H, nBp] power-of-two exponent of each block's digits
  int32_t* k_exp;
  float* q_norm;       // [B*H, nBp, 2] L1 and L2 norm of each block's mean (rounded up)
  float* k_norm;
  int32_t* key_stat;   // [B*H, 4]: largest key exponent, largest key L1 and L2 norm (float bits)
  int32_t* fb_count;   // rows routed to the exact fallback
  int32_t* fb_rows;    // [B*H*nB] their row indices
  // threshold mode only
  double tau_raw;           // tau * sqrt(D): threshold offset on the unscaled dot products
  double* row_thr;          // workspace: [B*H*nB] per-row threshold
  int64_t* row_cnt;         // workspace: [B*H*nB] per-row kept count
  int64_t* row_ptr;         // [B*H*nB + 1]
  int32_t* col_idx;         // [col_capacity]
  int64_t col_capacity;
};

void launch_subblock_select(const SelectArgs& a, hipStream_t stream);
// norm+RoPE of (nr) with the pooling of its output into a's workspace (the selection's first step)
void launch_qk_norm_rope_pool(const NormRopeArgs& nr, const RopeTable& table, const SelectArgs& a,
                              hipStream_t stream);
// the selection after launch_qk_norm_rope_pool: key statistics, top-k, fallback
void launch_subblock_select_pooled(const SelectArgs& a, hipStream_t stream);
void launch_threshold_count(const SelectArgs& a, hipStream_t stream);
void launch_threshold_fill(const SelectArgs& a, hipStream_t stream);

struct AdaLNArgs {
  const uint16_t* x;
  const float* shift;   // [B, C]
  const float* scale;   // [B, C]
  uint16_t* out;
  int64_t n_tokens;
  int32_t batch, hidden;
  float eps;
};

void launch_adaln(const AdaLNArgs& a, hipStream_t stream);

struct SwiGLUArgs {
  const uint16_t* gate;
  const uint16_t* up;
  uint16_t* out;          // [rows, width] contiguous
  int64_t rows, width, gate_stride, up_stride;  // strides in elements
};

void launch_swiglu(const SwiGLUArgs& a, hipStream_t stream);

// chunks of 8 elements reduced per workgroup by the residual-change kernel
constexpr int64_t kResidualChunksPerBlock = 8192;

struct ResidualArgs {
  const uint16_t* cur;
  const uint16_t* prev;
  int64_t n;
  int64_t chunks_per_block;
  double* partial;   // workspace: 2 doubles per workgroup
  double* result;    // 2 doubles: sum |cur - prev|, sum |prev|
};

int residual_parts(int64_t n);
void launch_residual_change(const ResidualArgs& a, hipStream_t stream);

// The allocation-free residual change keeps its per-workgroup partial sums in a file-scope device
// array of this many (sum |cur - prev|, sum |prev|) pairs (2 MB; n up to 2^33 elements).
constexpr int64_t kResidualNoAllocParts = (int64_t)1 << 17;
// Device address of that array on the current device (looked up once per device with
// hipGetSymbolAddress); null if the lookup failed.
double* residual_noalloc_scratch();

// ---- fp8 (OCP e4m3) attention ----
// Quantised tensors: q8, k8 are [B, N, H, D] bytes (e4m3 codes of x / s, s the power-of-two
// scale of the (b, head, 64-token block)); v8t is [B, H, D, nB*64] bytes: V transposed, each
// 64-key block's keys stored in the order the P.V product consumes them (key 32m + 8a + 4h + r at
// slot 16 (2h + m) + 4a + r, r < 4, a < 4; the v8t layout comment in fp8_quant.hip derives it), and
// keys past N zero; scales are float32 q_scale/k_scale [B, H, nB], v_scale [B, H, D].
struct Fp8QuantArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8t;
  float* q_scale;
  float* k_scale;
  float* v_scale;
  float* v_partial;   // workspace: per (b, head, token chunk) channel maxima
  int32_t* v_exp;     // workspace: the channel scale exponents [B, H, D]
  int64_t n_tokens;
  int32_t batch, heads, head_dim, n_blocks, n_chunks;
};

constexpr int kFp8VChunk = 1024;  // tokens per V channel-maximum partial

// Kept-set validation: one row per (b, head, query block); a bitmap of n_blocks bits in LDS.
struct IndexCheckArgs {
  const int32_t* block_idx;  // top-k rows [rows, keep], or the CSR col_idx
  const int64_t* row_ptr;    // CSR only: [rows + 1]
  uint8_t* row_flags;        // [rows]
  int64_t rows;
  int64_t col_capacity;      // CSR only: entries in col_idx
  int32_t n_blocks, keep;
};
constexpr int64_t kIndexCheckLdsBytes = 128 * 1024;  // n_blocks <= 2^20

void launch_check_topk_rows(const IndexCheckArgs& a, hipStream_t stream);
void launch_check_csr_rows(const IndexCheckArgs& a, hipStream_t stream);

void launch_fp8_quantize(const Fp8QuantArgs& a, hipStream_t stream);

struct Fp8AttnArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_idx;  // sparse only
  uint16_t* out;
  float* lse;                // may be null
  int64_t n_tokens;
  int32_t batch, heads, head_dim, n_blocks, keep;
  int32_t group_stride;      // sparse only, as in AttnArgs
};

void launch_fp8_dense_fwd(const Fp8AttnArgs& a, hipStream_t stream);
void launch_fp8_block_sparse_fwd(const Fp8AttnArgs& a, hipStream_t stream);

}  // namespace h3attn
