// C ABI of the h3attn library: host-side argument validation, RoPE table construction and
// kernel dispatch. Every check runs before any HIP call; on failure nothing is launched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <hip/hip_runtime.h>

#include "../../include/h3attn.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

h3attn_status fail(h3attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

h3attn_status ok() {
  g_err[0] = '\0';
  return H3ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks that p is non-null and 16-byte aligned.
#define CHECK_PTR(p)                                                                      \
  do {                                                                                    \
    if ((p) == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "%s is NULL", #p);       \
    if (!aligned16(p)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", #p); \
  } while (0)

h3attn_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(H3ATTN_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

h3attn_status check_sizes(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim) {
  if (batch <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "batch must be > 0 (got %d)", batch);
  if (heads <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "heads must be > 0 (got %d)", heads);
  if (n_tokens <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "n_tokens must be > 0 (got %lld)", (long long)n_tokens);
  if (head_dim != 64 && head_dim != 128)
    return fail(H3ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  // every element offset must fit in int64 and the grid dimensions in 32 bits
  const double elems = (double)batch * (double)n_tokens * (double)heads * (double)head_dim;
  if (elems > 9.0e18) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "tensor too large");
  if (n_tokens > (int64_t)1 << 31) return fail(H3ATTN_ERR_UNSUPPORTED, "n_tokens above 2^31 is not supported");
  if (heads > 65535 || batch > 65535) return fail(H3ATTN_ERR_UNSUPPORTED, "batch and heads must be <= 65535");
  return H3ATTN_OK;
}

// Query-block grouping of the sparse kernels: 1 (four consecutive blocks) up to n_blocks.
h3attn_status check_group_stride(int32_t group_stride, int64_t n_blocks) {
  if (group_stride < 1 || group_stride > n_blocks)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "group_stride must be in [1, %lld] (got %d)", (long long)n_blocks,
                group_stride);
  return H3ATTN_OK;
}

}  // namespace

extern "C" {

const char* h3attn_version(void) { return "h3attn 0.1.0 gfx950"; }

const char* h3attn_last_error(void) { return g_err; }

int32_t h3attn_keep_count(int32_t n_kblocks, double sparsity) {
  if (n_kblocks <= 0 || !(sparsity >= 0.0 && sparsity < 1.0)) return -1;
  double k = std::ceil((1.0 - sparsity) * (double)n_kblocks - 1e-9);
  if (k < 1.0) k = 1.0;
  if (k > (double)n_kblocks) k = (double)n_kblocks;
  return (int32_t)k;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Regions of the selection workspace, each 256-byte aligned: float64 means of q and k
// [B*H, nB, D]; their base-256 digits [B*H, nBp, D, 3] int8 (nBp = nB rounded up to 32); the
// per-block exponents [B*H, nBp] int32 and norms [B*H, nBp, 2] float32 of q and k; per-head key
// maxima [B*H, 4] int32; the fallback row count and list [1 + B*H*nB] int32.
struct SelectLayout {
  size_t mean, digits, exps, norms, key_stat, fb, total;
};

static SelectLayout select_layout(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim, int32_t block_size) {
  SelectLayout L{};
  const size_t nb = (size_t)((n_tokens + block_size - 1) / block_size);
  const size_t nbp = (nb + 31) / 32 * 32;
  const size_t bh = (size_t)batch * (size_t)heads;
  L.mean = align256(bh * nb * (size_t)head_dim * sizeof(double));
  L.digits = align256(bh * nbp * (size_t)head_dim * 3);
  L.exps = align256(bh * nbp * sizeof(int32_t));
  L.norms = align256(bh * nbp * 2 * sizeof(float));
  L.key_stat = align256(bh * 4 * sizeof(int32_t));
  L.fb = align256((1 + bh * nb) * sizeof(int32_t));
  L.total = 2 * (L.mean + L.digits + L.exps + L.norms) + L.key_stat + L.fb;
  return L;
}

static void select_pointers(h3attn::SelectArgs& a, void* workspace, const SelectLayout& L) {
  unsigned char* p = static_cast<unsigned char*>(workspace);
  a.q_mean = reinterpret_cast<double*>(p); p += L.mean;
  a.k_mean = reinterpret_cast<double*>(p); p += L.mean;
  a.q_digits = reinterpret_cast<int8_t*>(p); p += L.digits;
  a.k_digits = reinterpret_cast<int8_t*>(p); p += L.digits;
  a.q_exp = reinterpret_cast<int32_t*>(p); p += L.exps;
  a.k_exp = reinterpret_cast<int32_t*>(p); p += L.exps;
  a.q_norm = reinterpret_cast<float*>(p); p += L.norms;
  a.k_norm = reinterpret_cast<float*>(p); p += L.norms;
  a.key_stat = reinterpret_cast<int32_t*>(p); p += L.key_stat;
  a.fb_count = reinterpret_cast<int32_t*>(p);
  a.fb_rows = reinterpret_cast<int32_t*>(p) + 1;
}

size_t h3attn_select_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens,
                                     int32_t head_dim, int32_t block_size) {
  if (batch <= 0 || heads <= 0 || n_tokens <= 0 || head_dim <= 0 || block_size <= 0) return 0;
  return select_layout(batch, heads, n_tokens, head_dim, block_size).total;
}

// Validates the norm+RoPE arguments and builds the kernel arguments and the rotation-rate table.
static h3attn_status prepare_norm_rope(const h3attn_bf16* q_in, const h3attn_bf16* k_in, h3attn_bf16* q_out,
                                       h3attn_bf16* k_out, const float* q_weight, const float* k_weight,
                                       int32_t batch, int32_t heads, int32_t head_dim, h3attn_grid grid,
                                       int32_t d_t, int32_t d_h, int32_t d_w, float rope_theta, float eps,
                                       h3attn::NormRopeArgs& a, h3attn::RopeTable& tab) {
  CHECK_PTR(q_in); CHECK_PTR(k_in); CHECK_PTR(q_out); CHECK_PTR(k_out);
  CHECK_PTR(q_weight); CHECK_PTR(k_weight);
  if (grid.t <= 0 || grid.h <= 0 || grid.w <= 0)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "grid sizes must be > 0 (got %d x %d x %d)", grid.t, grid.h, grid.w);
  const int64_t n_tokens = (int64_t)grid.t * grid.h * grid.w;
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (d_t < 0 || d_h < 0 || d_w < 0 || (d_t & 1) || (d_h & 1) || (d_w & 1))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "RoPE sections must be even and >= 0 (got %d/%d/%d)", d_t, d_h, d_w);
  if (d_t + d_h + d_w != head_dim)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "RoPE sections %d+%d+%d must add up to head_dim %d", d_t, d_h, d_w, head_dim);
  if (!(rope_theta > 0.0f) || !std::isfinite(rope_theta))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  const bool q_inplace = q_out == q_in, k_inplace = k_out == k_in;
  if (q_out == k_out || (q_out == k_in && !k_inplace) || (k_out == q_in && !q_inplace))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "q_out and k_out must be distinct and not alias the other input");

  if (((int64_t)batch * n_tokens / 8 + 1) * ((2 * (int64_t)heads + 3) / 4) >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*n_tokens*heads too large for one launch");
  std::memset(&tab, 0, sizeof(tab));
  const int32_t secs[3] = {d_t, d_h, d_w};
  int pair = 0;
  for (int ax = 0; ax < 3; ++ax) {
    for (int j = 0; j < secs[ax] / 2; ++j, ++pair) {
      tab.rate[pair] = std::pow((double)rope_theta, -2.0 * (double)j / (double)secs[ax]);
      tab.axis[pair] = ax;
    }
  }
  a = h3attn::NormRopeArgs{};
  a.q_in = q_in; a.k_in = k_in; a.q_out = q_out; a.k_out = k_out;
  a.q_weight = q_weight; a.k_weight = k_weight;
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.grid_h = grid.h; a.grid_w = grid.w; a.eps = eps;
  return H3ATTN_OK;
}

h3attn_status h3attn_qk_norm_rope(const h3attn_bf16* q_in, const h3attn_bf16* k_in,
                                  h3attn_bf16* q_out, h3attn_bf16* k_out,
                                  const float* q_weight, const float* k_weight,
                                  int32_t batch, int32_t heads, int32_t head_dim, h3attn_grid grid,
                                  int32_t d_t, int32_t d_h, int32_t d_w,
                                  float rope_theta, float eps, hipStream_t stream) {
  h3attn::NormRopeArgs a;
  h3attn::RopeTable tab;
  const h3attn_status st = prepare_norm_rope(q_in, k_in, q_out, k_out, q_weight, k_weight, batch, heads, head_dim,
                                             grid, d_t, d_h, d_w, rope_theta, eps, a, tab);
  if (st != H3ATTN_OK) return st;
  h3attn::launch_qk_norm_rope(a, tab, stream);
  return check_launch("h3attn_qk_norm_rope");
}

static h3attn_status check_attn(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                const h3attn_bf16* out, const float* lse,
                                int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim) {
  CHECK_PTR(q); CHECK_PTR(k); CHECK_PTR(v); CHECK_PTR(out);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (out == q || out == k || out == v) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "out must not alias q, k or v");
  return H3ATTN_OK;
}

h3attn_status h3attn_dense_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                               h3attn_bf16* out, float* lse,
                               int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                               hipStream_t stream) {
  h3attn_status st = check_attn(q, k, v, out, lse, batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  h3attn::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.block_idx = nullptr;
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.keep = 0; a.n_blocks = (int32_t)((n_tokens + 63) / 64);
  h3attn::launch_dense_fwd(a, stream);
  return check_launch("h3attn_dense_fwd");
}

// Checks shared by the selection entry points (sizes, block size, the fallback's LDS limit, the
// workspace) and the workspace pointers of the SelectArgs.
static h3attn_status prepare_select(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                    int32_t block_size, void* workspace, size_t workspace_bytes,
                                    h3attn::SelectArgs& a) {
  if (workspace == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  if ((int64_t)batch * heads > 65535) return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads must be <= 65535");
  const int64_t nb = (n_tokens + block_size - 1) / block_size;
  if (nb * 8 > h3attn::kSelectRowLdsBytes)
    return fail(H3ATTN_ERR_UNSUPPORTED, "%lld blocks exceed the per-row LDS budget of the selection kernels", (long long)nb);
  const size_t need = h3attn_select_workspace_bytes(batch, heads, n_tokens, head_dim, block_size);
  if (workspace_bytes < need)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  a = h3attn::SelectArgs{};
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.block_size = block_size; a.n_blocks = (int32_t)nb;
  select_pointers(a, workspace, select_layout(batch, heads, n_tokens, head_dim, block_size));
  return H3ATTN_OK;
}

// The top-k arguments: the output rows and keep = keep_count(nB, sparsity).
static h3attn_status prepare_topk(double sparsity, int32_t keep, int32_t* block_idx, h3attn::SelectArgs& a) {
  if (block_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is NULL");
  if (reinterpret_cast<uintptr_t>(block_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is not 4-byte aligned");
  if (!(sparsity >= 0.0 && sparsity < 1.0)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "sparsity must be in [0, 1) (got %g)", sparsity);
  const int32_t want = h3attn_keep_count(a.n_blocks, sparsity);
  if (keep != want) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "keep %d does not match keep_count(%d, %g) = %d", keep, a.n_blocks, sparsity, want);
  if ((uint64_t)a.batch * a.heads * (uint64_t)a.n_blocks * (uint64_t)keep > ((uint64_t)1 << 62))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx too large");
  a.keep = keep;
  a.block_idx = block_idx;
  return H3ATTN_OK;
}

h3attn_status h3attn_subblock_select(const h3attn_bf16* q, const h3attn_bf16* k,
                                     int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                     int32_t block_size, double sparsity, int32_t keep,
                                     int32_t* block_idx, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  CHECK_PTR(q); CHECK_PTR(k);
  h3attn::SelectArgs a;
  h3attn_status st = prepare_select(batch, heads, n_tokens, head_dim, block_size, workspace, workspace_bytes, a);
  if (st != H3ATTN_OK) return st;
  st = prepare_topk(sparsity, keep, block_idx, a);
  if (st != H3ATTN_OK) return st;
  a.q = q; a.k = k;
  h3attn::launch_subblock_select(a, stream);
  return check_launch("h3attn_subblock_select");
}

h3attn_status h3attn_qk_norm_rope_pool(const h3attn_bf16* q_in, const h3attn_bf16* k_in,
                                       h3attn_bf16* q_out, h3attn_bf16* k_out,
                                       const float* q_weight, const float* k_weight,
                                       int32_t batch, int32_t heads, int32_t head_dim, h3attn_grid grid,
                                       int32_t d_t, int32_t d_h, int32_t d_w,
                                       float rope_theta, float eps, int32_t block_size,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3attn::NormRopeArgs nr;
  h3attn::RopeTable tab;
  h3attn_status st = prepare_norm_rope(q_in, k_in, q_out, k_out, q_weight, k_weight, batch, heads, head_dim,
                                       grid, d_t, d_h, d_w, rope_theta, eps, nr, tab);
  if (st != H3ATTN_OK) return st;
  h3attn::SelectArgs a;
  st = prepare_select(batch, heads, nr.n_tokens, head_dim, block_size, workspace, workspace_bytes, a);
  if (st != H3ATTN_OK) return st;
  a.q = q_out; a.k = k_out;  // what is pooled: the outputs
  h3attn::launch_qk_norm_rope_pool(nr, tab, a, stream);
  return check_launch("h3attn_qk_norm_rope_pool");
}

h3attn_status h3attn_subblock_select_pooled(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                            int32_t block_size, double sparsity, int32_t keep,
                                            int32_t* block_idx, void* workspace, size_t workspace_bytes,
                                            hipStream_t stream) {
  h3attn::SelectArgs a;
  h3attn_status st = prepare_select(batch, heads, n_tokens, head_dim, block_size, workspace, workspace_bytes, a);
  if (st != H3ATTN_OK) return st;
  st = prepare_topk(sparsity, keep, block_idx, a);
  if (st != H3ATTN_OK) return st;
  h3attn::launch_subblock_select_pooled(a, stream);
  return check_launch("h3attn_subblock_select_pooled");
}

static h3attn_status block_sparse_topk(const char* name, const h3attn_bf16* q, const h3attn_bf16* k,
                                       const h3attn_bf16* v, const int32_t* block_idx, int32_t keep,
                                       h3attn_bf16* out, float* lse, int32_t batch, int32_t heads,
                                       int64_t n_tokens, int32_t head_dim, int32_t block_size,
                                       int32_t group_stride, hipStream_t stream) {
  h3attn_status st = check_attn(q, k, v, out, lse, batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (block_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is NULL");
  if (reinterpret_cast<uintptr_t>(block_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is not 4-byte aligned");
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  const int64_t nb = (n_tokens + block_size - 1) / block_size;
  if (keep < 1 || keep > nb) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "keep must be in [1, %lld] (got %d)", (long long)nb, keep);
  if (nb * heads * (int64_t)batch >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads*n_blocks must be below 2^31");
  st = check_group_stride(group_stride, nb);
  if (st != H3ATTN_OK) return st;
  h3attn::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.block_idx = block_idx;
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.keep = keep; a.n_blocks = (int32_t)nb; a.group_stride = group_stride;
  h3attn::launch_block_sparse_fwd(a, stream);
  return check_launch(name);
}

h3attn_status h3attn_block_sparse_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                      const int32_t* block_idx, int32_t keep,
                                      h3attn_bf16* out, float* lse,
                                      int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                      int32_t block_size, hipStream_t stream) {
  return block_sparse_topk("h3attn_block_sparse_fwd", q, k, v, block_idx, keep, out, lse, batch, heads, n_tokens,
                           head_dim, block_size, 1, stream);
}

h3attn_status h3attn_block_sparse_grouped_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                              const int32_t* block_idx, int32_t keep,
                                              h3attn_bf16* out, float* lse,
                                              int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                              int32_t block_size, int32_t group_stride, hipStream_t stream) {
  return block_sparse_topk("h3attn_block_sparse_grouped_fwd", q, k, v, block_idx, keep, out, lse, batch, heads,
                           n_tokens, head_dim, block_size, group_stride, stream);
}

static h3attn_status check_select_common(const h3attn_bf16* q, const h3attn_bf16* k, int32_t batch,
                                         int32_t heads, int64_t n_tokens, int32_t head_dim,
                                         int32_t block_size, const void* workspace, int64_t* nb_out) {
  if (q != nullptr || k != nullptr) { CHECK_PTR(q); CHECK_PTR(k); }
  if (workspace == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  if ((int64_t)batch * heads > 65535) return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads must be <= 65535");
  *nb_out = (n_tokens + block_size - 1) / block_size;
  if (*nb_out * 8 > h3attn::kSelectRowLdsBytes)
    return fail(H3ATTN_ERR_UNSUPPORTED, "%lld blocks exceed the per-row LDS budget of the threshold kernels",
                (long long)*nb_out);
  return H3ATTN_OK;
}

size_t h3attn_threshold_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens,
                                        int32_t head_dim, int32_t block_size) {
  const size_t base = h3attn_select_workspace_bytes(batch, heads, n_tokens, head_dim, block_size);
  if (base == 0) return 0;
  const size_t rows = (size_t)batch * heads * (size_t)((n_tokens + block_size - 1) / block_size);
  return base + 2 * align256(rows * 8);
}

static void threshold_layout(h3attn::SelectArgs& a, void* workspace, int32_t batch, int32_t heads,
                             int64_t nb, int32_t head_dim) {
  const SelectLayout L = select_layout(batch, heads, nb * 64, head_dim, 64);
  select_pointers(a, workspace, L);
  const size_t rows = align256((size_t)batch * heads * (size_t)nb * 8);
  unsigned char* ws = static_cast<unsigned char*>(workspace) + L.total;
  a.row_thr = reinterpret_cast<double*>(ws);
  a.row_cnt = reinterpret_cast<int64_t*>(ws + rows);
}

h3attn_status h3attn_subblock_threshold_count(const h3attn_bf16* q, const h3attn_bf16* k,
                                              int32_t batch, int32_t heads, int64_t n_tokens,
                                              int32_t head_dim, int32_t block_size, double tau,
                                              int64_t* row_ptr, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  if (q == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "q is NULL");
  if (k == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "k is NULL");
  int64_t nb = 0;
  h3attn_status st = check_select_common(q, k, batch, heads, n_tokens, head_dim, block_size, workspace, &nb);
  if (st != H3ATTN_OK) return st;
  if (row_ptr == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is NULL");
  if (reinterpret_cast<uintptr_t>(row_ptr) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is not 8-byte aligned");
  if (!(tau >= 0.0)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "tau must be >= 0 (got %g)", tau);
  const size_t need = h3attn_threshold_workspace_bytes(batch, heads, n_tokens, head_dim, block_size);
  if (workspace_bytes < need)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  h3attn::SelectArgs a{};
  a.q = q; a.k = k; a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.block_size = block_size; a.n_blocks = (int32_t)nb; a.keep = 0;
  threshold_layout(a, workspace, batch, heads, nb, head_dim);
  a.tau_raw = tau * std::sqrt((double)head_dim);
  a.row_ptr = row_ptr;
  h3attn::launch_threshold_count(a, stream);
  return check_launch("h3attn_subblock_threshold_count");
}

h3attn_status h3attn_subblock_threshold_fill(int32_t batch, int32_t heads, int64_t n_tokens,
                                             int32_t head_dim, int32_t block_size,
                                             const int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int64_t nb = 0;
  h3attn_status st = check_select_common(nullptr, nullptr, batch, heads, n_tokens, head_dim, block_size, workspace, &nb);
  if (st != H3ATTN_OK) return st;
  if (row_ptr == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is NULL");
  if (reinterpret_cast<uintptr_t>(row_ptr) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is not 8-byte aligned");
  if (col_capacity < 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_capacity must be >= 0");
  if (col_capacity > 0 && col_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is NULL");
  if (reinterpret_cast<uintptr_t>(col_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is not 4-byte aligned");
  const size_t need = h3attn_threshold_workspace_bytes(batch, heads, n_tokens, head_dim, block_size);
  if (workspace_bytes < need)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  h3attn::SelectArgs a{};
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.block_size = block_size; a.n_blocks = (int32_t)nb; a.keep = 0;
  threshold_layout(a, workspace, batch, heads, nb, head_dim);
  a.row_ptr = const_cast<int64_t*>(row_ptr);
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  h3attn::launch_threshold_fill(a, stream);
  return check_launch("h3attn_subblock_threshold_fill");
}

static h3attn_status block_sparse_csr(const char* name, const h3attn_bf16* q, const h3attn_bf16* k,
                                      const h3attn_bf16* v, const int64_t* row_ptr, const int32_t* col_idx,
                                      h3attn_bf16* out, float* lse, int32_t batch, int32_t heads,
                                      int64_t n_tokens, int32_t head_dim, int32_t block_size,
                                      int32_t group_stride, hipStream_t stream) {
  h3attn_status st = check_attn(q, k, v, out, lse, batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  if (row_ptr == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is NULL");
  if (reinterpret_cast<uintptr_t>(row_ptr) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is not 8-byte aligned");
  if (col_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is NULL");
  if (reinterpret_cast<uintptr_t>(col_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is not 4-byte aligned");
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  const int64_t nb = (n_tokens + block_size - 1) / block_size;
  if (nb * heads * (int64_t)batch >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads*n_blocks must be below 2^31");
  st = check_group_stride(group_stride, nb);
  if (st != H3ATTN_OK) return st;
  h3attn::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.block_idx = col_idx; a.row_ptr = row_ptr;
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.keep = 0; a.n_blocks = (int32_t)nb; a.group_stride = group_stride;
  h3attn::launch_block_sparse_csr_fwd(a, stream);
  return check_launch(name);
}

h3attn_status h3attn_block_sparse_csr_fwd(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                          const int64_t* row_ptr, const int32_t* col_idx,
                                          h3attn_bf16* out, float* lse,
                                          int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                          int32_t block_size, hipStream_t stream) {
  return block_sparse_csr("h3attn_block_sparse_csr_fwd", q, k, v, row_ptr, col_idx, out, lse, batch, heads,
                          n_tokens, head_dim, block_size, 1, stream);
}

h3attn_status h3attn_block_sparse_csr_grouped_fwd(const h3attn_bf16* q, const h3attn_bf16* k,
                                                  const h3attn_bf16* v, const int64_t* row_ptr,
                                                  const int32_t* col_idx, h3attn_bf16* out, float* lse,
                                                  int32_t batch, int32_t heads, int64_t n_tokens,
                                                  int32_t head_dim, int32_t block_size, int32_t group_stride,
                                                  hipStream_t stream) {
  return block_sparse_csr("h3attn_block_sparse_csr_grouped_fwd", q, k, v, row_ptr, col_idx, out, lse, batch,
                          heads, n_tokens, head_dim, block_size, group_stride, stream);
}

static h3attn_status check_rows_common(const uint8_t* row_flags, int32_t batch, int32_t heads, int32_t n_blocks) {
  if (row_flags == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_flags is NULL");
  if (batch <= 0 || heads <= 0 || n_blocks <= 0)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "batch, heads and n_blocks must be > 0");
  if ((int64_t)n_blocks > h3attn::kIndexCheckLdsBytes * 8)
    return fail(H3ATTN_ERR_UNSUPPORTED, "n_blocks must be at most %lld", (long long)(h3attn::kIndexCheckLdsBytes * 8));
  if ((int64_t)batch * heads * n_blocks >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads*n_blocks must be below 2^31");
  return H3ATTN_OK;
}

h3attn_status h3attn_check_block_idx(const int32_t* block_idx, int32_t batch, int32_t heads, int32_t n_blocks,
                                     int32_t keep, uint8_t* row_flags, hipStream_t stream) {
  if (block_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is NULL");
  if (reinterpret_cast<uintptr_t>(block_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is not 4-byte aligned");
  h3attn_status st = check_rows_common(row_flags, batch, heads, n_blocks);
  if (st != H3ATTN_OK) return st;
  if (keep < 1 || keep > n_blocks) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "keep must be in [1, %d] (got %d)", n_blocks, keep);
  h3attn::IndexCheckArgs a{};
  a.block_idx = block_idx; a.row_flags = row_flags; a.rows = (int64_t)batch * heads * n_blocks;
  a.n_blocks = n_blocks; a.keep = keep;
  h3attn::launch_check_topk_rows(a, stream);
  return check_launch("h3attn_check_block_idx");
}

h3attn_status h3attn_check_csr(const int64_t* row_ptr, const int32_t* col_idx, int64_t col_capacity, int32_t batch,
                               int32_t heads, int32_t n_blocks, uint8_t* row_flags, hipStream_t stream) {
  if (row_ptr == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is NULL");
  if (reinterpret_cast<uintptr_t>(row_ptr) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row_ptr is not 8-byte aligned");
  if (col_capacity < 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_capacity must be >= 0");
  if (col_capacity > 0 && col_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is NULL");
  if (reinterpret_cast<uintptr_t>(col_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "col_idx is not 4-byte aligned");
  h3attn_status st = check_rows_common(row_flags, batch, heads, n_blocks);
  if (st != H3ATTN_OK) return st;
  h3attn::IndexCheckArgs a{};
  a.block_idx = col_idx; a.row_ptr = row_ptr; a.row_flags = row_flags;
  a.rows = (int64_t)batch * heads * n_blocks; a.col_capacity = col_capacity; a.n_blocks = n_blocks;
  h3attn::launch_check_csr_rows(a, stream);
  return check_launch("h3attn_check_csr");
}

h3attn_status h3attn_adaln_modulate(const h3attn_bf16* x, const float* shift, const float* scale,
                                    h3attn_bf16* out, int32_t batch, int64_t n_tokens, int32_t hidden,
                                    float eps, hipStream_t stream) {
  CHECK_PTR(x); CHECK_PTR(shift); CHECK_PTR(scale); CHECK_PTR(out);
  if (batch <= 0 || n_tokens <= 0 || hidden <= 0)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "batch, n_tokens and hidden must be > 0");
  if (hidden % 8 != 0 || hidden > 16384)
    return fail(H3ATTN_ERR_UNSUPPORTED, "hidden must be a multiple of 8 and at most 16384 (got %d)", hidden);
  if ((int64_t)batch * n_tokens >= ((int64_t)1 << 31)) return fail(H3ATTN_ERR_UNSUPPORTED, "batch*n_tokens must be below 2^31");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  h3attn::AdaLNArgs a{};
  a.x = x; a.shift = shift; a.scale = scale; a.out = out;
  a.n_tokens = n_tokens; a.batch = batch; a.hidden = hidden; a.eps = eps;
  h3attn::launch_adaln(a, stream);
  return check_launch("h3attn_adaln_modulate");
}

h3attn_status h3attn_swiglu(const h3attn_bf16* gate, const h3attn_bf16* up, h3attn_bf16* out,
                            int64_t rows, int32_t width, int64_t gate_row_stride, int64_t up_row_stride,
                            hipStream_t stream) {
  CHECK_PTR(gate); CHECK_PTR(up); CHECK_PTR(out);
  if (rows <= 0 || width <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "rows and width must be > 0");
  if (gate_row_stride < width || up_row_stride < width)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "row strides must be >= width");
  if (width % 8 || gate_row_stride % 8 || up_row_stride % 8)
    return fail(H3ATTN_ERR_UNSUPPORTED, "width and row strides must be multiples of 8");
  if (rows * (int64_t)(width / 8) / 512 >= ((int64_t)1 << 31)) return fail(H3ATTN_ERR_UNSUPPORTED, "tensor too large for one launch");
  if ((out == gate && gate_row_stride != width) || (out == up && up_row_stride != width))
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "out may alias gate or up only when that row stride equals width");
  h3attn::SwiGLUArgs a{};
  a.gate = gate; a.up = up; a.out = out; a.rows = rows; a.width = width;
  a.gate_stride = gate_row_stride; a.up_stride = up_row_stride;
  h3attn::launch_swiglu(a, stream);
  return check_launch("h3attn_swiglu");
}

size_t h3attn_residual_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return align256((size_t)h3attn::residual_parts(n) * 2 * sizeof(double));
}

h3attn_status h3attn_residual_change(const h3attn_bf16* cur, const h3attn_bf16* prev, int64_t n,
                                     double* result, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  CHECK_PTR(cur); CHECK_PTR(prev);
  if (result == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "result is NULL");
  if (reinterpret_cast<uintptr_t>(result) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "result is not 8-byte aligned");
  if (n <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "n must be > 0");
  if (workspace == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  const size_t need = h3attn_residual_workspace_bytes(n);
  if (workspace_bytes < need)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  if (h3attn::residual_parts(n) >= (1 << 30)) return fail(H3ATTN_ERR_UNSUPPORTED, "tensor too large");
  h3attn::ResidualArgs a{};
  a.cur = cur; a.prev = prev; a.n = n; a.partial = static_cast<double*>(workspace); a.result = result;
  h3attn::launch_residual_change(a, stream);
  return check_launch("h3attn_residual_change");
}

h3attn_status h3attn_residual_change_noalloc(const h3attn_bf16* cur, const h3attn_bf16* prev, int64_t n,
                                             double* result, hipStream_t stream) {
  CHECK_PTR(cur); CHECK_PTR(prev);
  if (result == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "result is NULL");
  if (reinterpret_cast<uintptr_t>(result) & 7u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "result is not 8-byte aligned");
  if (n <= 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "n must be > 0");
  if (h3attn::residual_parts(n) > h3attn::kResidualNoAllocParts)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT,
                "n = %lld needs %d partial sums, more than the %lld of the allocation-free scratch (n <= %lld)",
                (long long)n, h3attn::residual_parts(n), (long long)h3attn::kResidualNoAllocParts,
                (long long)(h3attn::kResidualNoAllocParts * h3attn::kResidualChunksPerBlock * 8));
  double* partial = h3attn::residual_noalloc_scratch();
  if (partial == nullptr) return fail(H3ATTN_ERR_LAUNCH, "h3attn_residual_change_noalloc: device scratch lookup failed");
  h3attn::ResidualArgs a{};
  a.cur = cur; a.prev = prev; a.n = n; a.partial = partial; a.result = result;
  h3attn::launch_residual_change(a, stream);
  return check_launch("h3attn_residual_change_noalloc");
}

h3attn_status h3attn_cache_gate_init(h3attn_cache_gate* gate, double threshold, int32_t max_consecutive) {
  if (gate == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "gate is NULL");
  if (!(threshold >= 0.0)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "threshold must be >= 0");
  if (max_consecutive < 0) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "max_consecutive must be >= 0");
  gate->threshold = threshold;
  gate->max_consecutive = max_consecutive;
  gate->consecutive = 0;
  gate->steps = 0;
  return ok();
}

size_t h3attn_fp8_workspace_bytes(int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                  int32_t block_size) {
  if (batch <= 0 || heads <= 0 || n_tokens <= 0 || head_dim <= 0 || block_size <= 0) return 0;
  const size_t bh = (size_t)batch * (size_t)heads;
  const size_t chunks = (size_t)((n_tokens + h3attn::kFp8VChunk - 1) / h3attn::kFp8VChunk);
  return align256(bh * chunks * (size_t)head_dim * sizeof(float)) + align256(bh * (size_t)head_dim * sizeof(int32_t));
}

h3attn_status h3attn_fp8_quantize(const h3attn_bf16* q, const h3attn_bf16* k, const h3attn_bf16* v,
                                  uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                                  float* q_scale, float* k_scale, float* v_scale,
                                  int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                  int32_t block_size, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  CHECK_PTR(q); CHECK_PTR(k); CHECK_PTR(v); CHECK_PTR(q8); CHECK_PTR(k8); CHECK_PTR(v8t);
  CHECK_PTR(q_scale); CHECK_PTR(k_scale); CHECK_PTR(v_scale); CHECK_PTR(workspace);
  {
    const void* ins[] = {q, k, v};
    const void* outs[] = {q8, k8, v8t, q_scale, k_scale, v_scale, workspace};
    for (const void* o : outs)
      for (const void* i : ins)
        if (o == i) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "outputs must not alias the inputs");
  }
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  const size_t need = h3attn_fp8_workspace_bytes(batch, heads, n_tokens, head_dim, block_size);
  if (workspace_bytes < need)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  const int64_t nb = (n_tokens + 63) / 64;
  if (nb * heads * (int64_t)batch >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads*n_blocks must be below 2^31");
  h3attn::Fp8QuantArgs a{};
  a.q = q; a.k = k; a.v = v; a.q8 = q8; a.k8 = k8; a.v8t = v8t;
  a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.v_partial = static_cast<float*>(workspace);
  const size_t chunks = (size_t)((n_tokens + h3attn::kFp8VChunk - 1) / h3attn::kFp8VChunk);
  a.v_exp = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                       align256((size_t)batch * heads * chunks * head_dim * sizeof(float)));
  a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.n_blocks = (int32_t)nb; a.n_chunks = (int32_t)chunks;
  h3attn::launch_fp8_quantize(a, stream);
  return check_launch("h3attn_fp8_quantize");
}

namespace {
h3attn_status fp8_attn_args(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t, const float* q_scale,
                             const float* k_scale, const float* v_scale, h3attn_bf16* out, float* lse,
                             int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim, int32_t block_size,
                             h3attn::Fp8AttnArgs& a) {
  h3attn_status st = check_sizes(batch, heads, n_tokens, head_dim);
  if (st != H3ATTN_OK) return st;
  CHECK_PTR(q8); CHECK_PTR(k8); CHECK_PTR(v8t); CHECK_PTR(q_scale); CHECK_PTR(k_scale); CHECK_PTR(v_scale);
  CHECK_PTR(out);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  if ((const void*)out == q8 || (const void*)out == k8 || (const void*)out == v8t)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "out must not alias the quantised inputs");
  if (block_size != 64) return fail(H3ATTN_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", block_size);
  const int64_t nb = (n_tokens + 63) / 64;
  if (nb * heads * (int64_t)batch >= ((int64_t)1 << 31))
    return fail(H3ATTN_ERR_UNSUPPORTED, "batch*heads*n_blocks must be below 2^31");
  a = h3attn::Fp8AttnArgs{};
  a.q8 = q8; a.k8 = k8; a.v8t = v8t; a.q_scale = q_scale; a.k_scale = k_scale; a.v_scale = v_scale;
  a.out = out; a.lse = lse; a.n_tokens = n_tokens; a.batch = batch; a.heads = heads; a.head_dim = head_dim;
  a.n_blocks = (int32_t)nb;
  return H3ATTN_OK;
}
}  // namespace

h3attn_status h3attn_fp8_dense_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                   const float* q_scale, const float* k_scale, const float* v_scale,
                                   h3attn_bf16* out, float* lse, int32_t batch, int32_t heads, int64_t n_tokens,
                                   int32_t head_dim, int32_t block_size, hipStream_t stream) {
  h3attn::Fp8AttnArgs a;
  h3attn_status st = fp8_attn_args(q8, k8, v8t, q_scale, k_scale, v_scale, out, lse, batch, heads, n_tokens,
                                   head_dim, block_size, a);
  if (st != H3ATTN_OK) return st;
  h3attn::launch_fp8_dense_fwd(a, stream);
  return check_launch("h3attn_fp8_dense_fwd");
}

h3attn_status h3attn_fp8_block_sparse_fwd(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                                          const float* q_scale, const float* k_scale, const float* v_scale,
                                          const int32_t* block_idx, int32_t keep, h3attn_bf16* out, float* lse,
                                          int32_t batch, int32_t heads, int64_t n_tokens, int32_t head_dim,
                                          int32_t block_size, int32_t group_stride, hipStream_t stream) {
  h3attn::Fp8AttnArgs a;
  h3attn_status st = fp8_attn_args(q8, k8, v8t, q_scale, k_scale, v_scale, out, lse, batch, heads, n_tokens,
                                   head_dim, block_size, a);
  if (st != H3ATTN_OK) return st;
  if (block_idx == nullptr) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is NULL");
  if (reinterpret_cast<uintptr_t>(block_idx) & 3u) return fail(H3ATTN_ERR_INVALID_ARGUMENT, "block_idx is not 4-byte aligned");
  if (keep < 1 || keep > a.n_blocks)
    return fail(H3ATTN_ERR_INVALID_ARGUMENT, "keep must be in [1, %d] (got %d)", a.n_blocks, keep);
  st = check_group_stride(group_stride, a.n_blocks);
  if (st != H3ATTN_OK) return st;
  a.block_idx = block_idx;
  a.keep = keep;
  a.group_stride = group_stride;
  h3attn::launch_fp8_block_sparse_fwd(a, stream);
  return check_launch("h3attn_fp8_block_sparse_fwd");
}

int32_t h3attn_cache_gate_decide(h3attn_cache_gate* gate, double rel_change) {
  if (gate == nullptr) return -1;
  const bool reuse = gate->steps > 0 && rel_change < gate->threshold && gate->consecutive < gate->max_consecutive;
  gate->consecutive = reuse ? gate->consecutive + 1 : 0;
  gate->steps += 1;
  return reuse ? 1 : 0;
}

int32_t h3attn_cache_gate_decide_sums(h3attn_cache_gate* gate, const double* sums) {
  const double rel = (sums != nullptr && sums[1] > 0.0) ? sums[0] / sums[1] : INFINITY;
  return h3attn_cache_gate_decide(gate, rel);
}

}  // extern "C"
