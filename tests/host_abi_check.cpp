// Host-only check of the C-ABI's validation and argument marshalling, built together with
// csrc/api.cpp under AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
// The kernel launchers and the two HIP runtime calls that api.cpp makes are replaced by stubs
// that record their arguments, so every entry point runs on the CPU and nothing dereferences the
// (fake, aligned) device pointers. Exit status 0 when every expectation holds.
#include <cmath>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "../include/h3attn.h"
#include "../video_diffusion_transformer_qk_amd/csrc/kernels.h"

// ---- stubs ----
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace {
int g_launches = 0;
h3attn::NormRopeArgs g_nr;
h3attn::RopeTable g_tab;
h3attn::AttnArgs g_attn;
h3attn::SelectArgs g_sel;
h3attn::IndexCheckArgs g_chk;
h3attn::Fp8QuantArgs g_fq;
h3attn::Fp8AttnArgs g_fa;
h3attn::AdaLNArgs g_ad;
h3attn::SwiGLUArgs g_sw;
h3attn::ResidualArgs g_res;
}  // namespace

namespace h3attn {
void launch_qk_norm_rope(const NormRopeArgs& a, const RopeTable& t, hipStream_t) { g_nr = a; g_tab = t; ++g_launches; }
void launch_dense_fwd(const AttnArgs& a, hipStream_t) { g_attn = a; ++g_launches; }
void launch_block_sparse_fwd(const AttnArgs& a, hipStream_t) { g_attn = a; ++g_launches; }
void launch_block_sparse_csr_fwd(const AttnArgs& a, hipStream_t) { g_attn = a; ++g_launches; }
void launch_subblock_select(const SelectArgs& a, hipStream_t) { g_sel = a; ++g_launches; }
void launch_qk_norm_rope_pool(const NormRopeArgs& nr, const RopeTable& t, const SelectArgs& a, hipStream_t) {
  g_nr = nr; g_tab = t; g_sel = a; ++g_launches;
}
void launch_subblock_select_pooled(const SelectArgs& a, hipStream_t) { g_sel = a; ++g_launches; }
void launch_threshold_count(const SelectArgs& a, hipStream_t) { g_sel = a; ++g_launches; }
void launch_threshold_fill(const SelectArgs& a, hipStream_t) { g_sel = a; ++g_launches; }
void launch_check_topk_rows(const IndexCheckArgs& a, hipStream_t) { g_chk = a; ++g_launches; }
void launch_check_csr_rows(const IndexCheckArgs& a, hipStream_t) { g_chk = a; ++g_launches; }
void launch_fp8_quantize(const Fp8QuantArgs& a, hipStream_t) { g_fq = a; ++g_launches; }
void launch_fp8_dense_fwd(const Fp8AttnArgs& a, hipStream_t) { g_fa = a; ++g_launches; }
void launch_fp8_block_sparse_fwd(const Fp8AttnArgs& a, hipStream_t) { g_fa = a; ++g_launches; }
void launch_adaln(const AdaLNArgs& a, hipStream_t) { g_ad = a; ++g_launches; }
void launch_swiglu(const SwiGLUArgs& a, hipStream_t) { g_sw = a; ++g_launches; }
void launch_residual_change(const ResidualArgs& a, hipStream_t) { g_res = a; ++g_launches; }
double* residual_noalloc_scratch() { return reinterpret_cast<double*>(0xD00000); }
int residual_parts(int64_t n) {
  const int64_t chunks = (n + 7) / 8;
  return (int)((chunks + kResidualChunksPerBlock - 1) / kResidualChunksPerBlock);
}
}  // namespace h3attn

// ---- checks ----
namespace {
int g_fail = 0;
#define EXPECT(cond)                                                                  \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      std::printf("FAIL %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond,     \
                  h3attn_last_error());                                               \
      ++g_fail;                                                                       \
    }                                                                                 \
  } while (0)

template <typename T>
T* P(uintptr_t a) { return reinterpret_cast<T*>(a); }
const h3attn_bf16* Q = P<const h3attn_bf16>(0x10000);
const h3attn_bf16* K = P<const h3attn_bf16>(0x20000);
const h3attn_bf16* V = P<const h3attn_bf16>(0x30000);
h3attn_bf16* O = P<h3attn_bf16>(0x40000);
void* WS = P<void>(0x100000);

// expected launch: status OK and exactly one more recorded launch
bool launched(h3attn_status st, int before) { return st == H3ATTN_OK && g_launches == before + 1; }

void check_norm_rope() {
  const float* wq = P<const float>(0x50000);
  const float* wk = P<const float>(0x60000);
  h3attn_bf16* qo = P<h3attn_bf16>(0x70000);
  h3attn_bf16* ko = P<h3attn_bf16>(0x80000);
  const h3attn_grid g{4, 8, 8};
  int n0 = g_launches;
  EXPECT(launched(h3attn_qk_norm_rope(Q, K, qo, ko, wq, wk, 1, 2, 64, g, 16, 24, 24, 1e4f, 1e-6f, nullptr), n0));
  EXPECT(g_nr.n_tokens == 256 && g_nr.grid_h == 8 && g_nr.grid_w == 8 && g_nr.heads == 2 && g_nr.head_dim == 64);
  // the rotation table: pair p of section a (offset o_a, size d_a) turns at theta^(-2j/d_a), j = p - o_a/2
  const int dsz[3] = {16, 24, 24};
  int pair = 0;
  for (int ax = 0; ax < 3; ++ax)
    for (int j = 0; j < dsz[ax] / 2; ++j, ++pair) {
      EXPECT(g_tab.axis[pair] == ax);
      const double want = std::pow(1e4, -2.0 * j / dsz[ax]);
      EXPECT(std::fabs(g_tab.rate[pair] - want) <= 1e-15 * want);
    }
  n0 = g_launches;
  EXPECT(h3attn_qk_norm_rope(Q, K, qo, ko, wq, wk, 1, 2, 64, g, 16, 24, 20, 1e4f, 1e-6f, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_qk_norm_rope(Q, K, qo, ko, wq, wk, 1, 2, 72, g, 24, 24, 24, 1e4f, 1e-6f, nullptr) == H3ATTN_ERR_UNSUPPORTED);
  EXPECT(h3attn_qk_norm_rope(Q, K, qo, ko, wq, wk, 1, 2, 64, g, 16, 24, 24, -1.f, 1e-6f, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_qk_norm_rope(Q, K, qo, ko, wq, wk, 1, 2, 64, g, 16, 24, 24, 1e4f, NAN, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_qk_norm_rope(P<const h3attn_bf16>(0x10008), K, qo, ko, wq, wk, 1, 2, 64, g, 16, 24, 24, 1e4f, 1e-6f, nullptr) ==
         H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(g_launches == n0);  // nothing launched on any error
}

void check_attention() {
  int n0 = g_launches;
  EXPECT(launched(h3attn_dense_fwd(Q, K, V, O, nullptr, 2, 3, 333, 128, nullptr), n0));
  EXPECT(g_attn.n_tokens == 333 && g_attn.batch == 2 && g_attn.heads == 3 && g_attn.block_idx == nullptr);
  EXPECT(h3attn_dense_fwd(Q, K, V, O, nullptr, 2, 3, 333, 96, nullptr) == H3ATTN_ERR_UNSUPPORTED);
  EXPECT(h3attn_dense_fwd(Q, K, V, O, nullptr, 0, 3, 333, 128, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_dense_fwd(Q, K, V, O, P<float>(0x90002), 2, 3, 333, 128, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  const int32_t* idx = P<const int32_t>(0xA0000);
  n0 = g_launches;
  EXPECT(launched(h3attn_block_sparse_fwd(Q, K, V, idx, 3, O, nullptr, 1, 2, 640, 64, 64, nullptr), n0));
  EXPECT(g_attn.n_blocks == 10 && g_attn.keep == 3 && g_attn.group_stride == 1 && g_attn.block_idx == idx);
  EXPECT(launched(h3attn_block_sparse_grouped_fwd(Q, K, V, idx, 3, O, nullptr, 1, 2, 640, 64, 64, 7, nullptr), n0 + 1));
  EXPECT(g_attn.group_stride == 7);
  EXPECT(h3attn_block_sparse_grouped_fwd(Q, K, V, idx, 3, O, nullptr, 1, 2, 640, 64, 64, 11, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_block_sparse_fwd(Q, K, V, idx, 11, O, nullptr, 1, 2, 640, 64, 64, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  const int64_t* rp = P<const int64_t>(0xB0000);
  n0 = g_launches;
  EXPECT(launched(h3attn_block_sparse_csr_grouped_fwd(Q, K, V, rp, idx, O, nullptr, 1, 2, 640, 64, 64, 5, nullptr), n0));
  EXPECT(g_attn.row_ptr == rp && g_attn.keep == 0 && g_attn.group_stride == 5 && g_attn.n_blocks == 10);
}

void check_select() {
  const size_t ws = h3attn_select_workspace_bytes(1, 2, 640, 64, 64);
  EXPECT(ws >= 2 * 1 * 2 * 10 * 64 * sizeof(double) + 2 * 1 * 2 * 32 * 64 * 3);
  int32_t* idx = P<int32_t>(0xA0000);
  const int32_t keep = h3attn_keep_count(10, 0.75);
  EXPECT(keep == 3);
  int n0 = g_launches;
  EXPECT(launched(h3attn_subblock_select(Q, K, 1, 2, 640, 64, 64, 0.75, keep, idx, WS, ws, nullptr), n0));
  EXPECT(g_sel.n_blocks == 10 && g_sel.keep == 3 && g_sel.block_idx == idx);
  // the workspace regions are 256-byte aligned, in order, disjoint and inside the workspace
  // (B*H = 2, nB = 10 padded to 32, D = 64)
  {
    const uintptr_t w0 = (uintptr_t)WS;
    const uintptr_t reg[] = {(uintptr_t)g_sel.q_mean, (uintptr_t)g_sel.k_mean, (uintptr_t)g_sel.q_digits,
                             (uintptr_t)g_sel.k_digits, (uintptr_t)g_sel.q_exp, (uintptr_t)g_sel.k_exp,
                             (uintptr_t)g_sel.q_norm, (uintptr_t)g_sel.k_norm, (uintptr_t)g_sel.key_stat,
                             (uintptr_t)g_sel.fb_count};
    const size_t len[] = {2 * 10 * 64 * 8, 2 * 10 * 64 * 8, 2 * 32 * 64 * 3, 2 * 32 * 64 * 3, 2 * 32 * 4, 2 * 32 * 4,
                          2 * 32 * 8, 2 * 32 * 8, 2 * 16, (1 + 2 * 10) * 4};
    EXPECT(reg[0] == w0);
    for (int i = 0; i < 10; ++i) {
      EXPECT((reg[i] & 255) == 0);
      if (i > 0) EXPECT(reg[i] >= reg[i - 1] + len[i - 1]);
    }
    EXPECT(reg[9] + len[9] <= w0 + ws);
    EXPECT((uintptr_t)g_sel.fb_rows == reg[9] + 4);
  }
  EXPECT(h3attn_subblock_select(Q, K, 1, 2, 640, 64, 64, 0.75, keep, idx, WS, ws - 1, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_subblock_select(Q, K, 1, 2, 640, 64, 64, 1.0, keep, idx, WS, ws, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_subblock_select(Q, K, 1, 2, 19969LL * 64, 64, 64, 0.75, keep, idx, WS, ws, nullptr) == H3ATTN_ERR_UNSUPPORTED);
  // norm+RoPE with the pooling, then the pooled selection: the same workspace regions
  {
    const float* wq = P<const float>(0x50000);
    const float* wk = P<const float>(0x60000);
    h3attn_bf16* qo = P<h3attn_bf16>(0x70000);
    h3attn_bf16* ko = P<h3attn_bf16>(0x80000);
    const h3attn_grid g10{10, 8, 8};
    const void* qmean = g_sel.q_mean;
    n0 = g_launches;
    EXPECT(launched(h3attn_qk_norm_rope_pool(Q, K, qo, ko, wq, wk, 1, 2, 64, g10, 16, 24, 24, 1e4f, 1e-6f, 64, WS,
                                             ws, nullptr), n0));
    EXPECT(g_nr.n_tokens == 640 && g_nr.q_out == qo && g_nr.k_out == ko && g_nr.heads == 2);
    EXPECT(g_sel.n_blocks == 10 && g_sel.q == qo && g_sel.k == ko && (const void*)g_sel.q_mean == qmean);
    EXPECT(h3attn_qk_norm_rope_pool(Q, K, qo, ko, wq, wk, 1, 2, 64, g10, 16, 24, 24, 1e4f, 1e-6f, 64, WS, ws - 1,
                                    nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    EXPECT(h3attn_qk_norm_rope_pool(Q, K, qo, ko, wq, wk, 1, 2, 64, g10, 16, 24, 24, 1e4f, 1e-6f, 32, WS, ws,
                                    nullptr) == H3ATTN_ERR_UNSUPPORTED);
    EXPECT(h3attn_qk_norm_rope_pool(Q, K, qo, ko, wq, wk, 1, 2, 64, g10, 16, 24, 22, 1e4f, 1e-6f, 64, WS, ws,
                                    nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    EXPECT(h3attn_qk_norm_rope_pool(Q, K, qo, ko, wq, wk, 1, 2, 64, g10, 16, 24, 24, 1e4f, 1e-6f, 64, nullptr, ws,
                                    nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    n0 = g_launches;
    EXPECT(launched(h3attn_subblock_select_pooled(1, 2, 640, 64, 64, 0.75, keep, idx, WS, ws, nullptr), n0));
    EXPECT(g_sel.n_blocks == 10 && g_sel.keep == 3 && g_sel.block_idx == idx && (const void*)g_sel.q_mean == qmean);
    EXPECT(h3attn_subblock_select_pooled(1, 2, 640, 64, 64, 0.75, keep + 1, idx, WS, ws, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    EXPECT(h3attn_subblock_select_pooled(1, 2, 640, 64, 64, 1.0, keep, idx, WS, ws, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    EXPECT(h3attn_subblock_select_pooled(1, 2, 640, 64, 64, 0.75, keep, nullptr, WS, ws, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
    EXPECT(h3attn_subblock_select_pooled(1, 2, 640, 64, 64, 0.75, keep, idx, WS, ws - 1, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  }
  // threshold mode
  const size_t tws = h3attn_threshold_workspace_bytes(1, 2, 640, 64, 64);
  int64_t* rp = P<int64_t>(0xB0000);
  n0 = g_launches;
  EXPECT(launched(h3attn_subblock_threshold_count(Q, K, 1, 2, 640, 64, 64, 0.5, rp, WS, tws, nullptr), n0));
  EXPECT(std::fabs(g_sel.tau_raw - 0.5 * 8.0) < 1e-15 && g_sel.row_ptr == rp);
  EXPECT(launched(h3attn_subblock_threshold_fill(1, 2, 640, 64, 64, rp, idx, 100, WS, tws, nullptr), n0 + 1));
  EXPECT(g_sel.col_capacity == 100 && g_sel.col_idx == idx);
  EXPECT(h3attn_subblock_threshold_count(Q, K, 1, 2, 640, 64, 64, -1.0, rp, WS, tws, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  // kept-set checks
  uint8_t* fl = P<uint8_t>(0xC0000);
  n0 = g_launches;
  EXPECT(launched(h3attn_check_block_idx(idx, 1, 2, 10, 3, fl, nullptr), n0));
  EXPECT(g_chk.rows == 20 && g_chk.keep == 3 && g_chk.n_blocks == 10);
  EXPECT(launched(h3attn_check_csr(rp, idx, 17, 1, 2, 10, fl, nullptr), n0 + 1));
  EXPECT(g_chk.rows == 20 && g_chk.col_capacity == 17 && g_chk.row_ptr == rp);
}

void check_keep_count() {
  EXPECT(h3attn_keep_count(4, 0.5) == 2);
  EXPECT(h3attn_keep_count(1953, 0.75) == 489);
  EXPECT(h3attn_keep_count(3843, 0.80) == 769);
  EXPECT(h3attn_keep_count(5733, 0.75) == 1434);
  EXPECT(h3attn_keep_count(63, 0.0) == 63);
  EXPECT(h3attn_keep_count(10, 0.9999999) == 1);
  EXPECT(h3attn_keep_count(0, 0.5) == -1 && h3attn_keep_count(10, 1.0) == -1 && h3attn_keep_count(10, NAN) == -1);
}

void check_block_ops() {
  const float* sh = P<const float>(0x50000);
  const float* scl = P<const float>(0x60000);
  int n0 = g_launches;
  EXPECT(launched(h3attn_adaln_modulate(Q, sh, scl, O, 2, 100, 3072, 1e-6f, nullptr), n0));
  EXPECT(g_ad.hidden == 3072 && g_ad.n_tokens == 100 && g_ad.batch == 2);
  EXPECT(h3attn_adaln_modulate(Q, sh, scl, O, 2, 100, 3070, 1e-6f, nullptr) == H3ATTN_ERR_UNSUPPORTED);
  n0 = g_launches;
  EXPECT(launched(h3attn_swiglu(Q, K, O, 10, 64, 128, 128, nullptr), n0));
  EXPECT(g_sw.rows == 10 && g_sw.width == 64 && g_sw.gate_stride == 128);
  EXPECT(h3attn_swiglu(Q, K, O, 10, 64, 60, 128, nullptr) != H3ATTN_OK);
  const size_t rws = h3attn_residual_workspace_bytes(655371);
  EXPECT(rws > 0);
  double* res = P<double>(0xD0000);
  n0 = g_launches;
  EXPECT(launched(h3attn_residual_change(Q, K, 655371, res, WS, rws, nullptr), n0));
  EXPECT(g_res.n == 655371 && g_res.result == res);
  EXPECT(h3attn_residual_change(Q, K, 655371, res, WS, rws - 1, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  // the allocation-free variant: the partial sums go to the library's device array; sizes past
  // its 2^17 pairs are refused before any launch
  n0 = g_launches;
  EXPECT(launched(h3attn_residual_change_noalloc(Q, K, 655371, res, nullptr), n0));
  EXPECT(g_res.n == 655371 && g_res.result == res && g_res.partial == reinterpret_cast<double*>(0xD00000));
  const int64_t max_n = h3attn::kResidualNoAllocParts * h3attn::kResidualChunksPerBlock * 8;
  n0 = g_launches;
  EXPECT(launched(h3attn_residual_change_noalloc(Q, K, max_n, res, nullptr), n0));
  EXPECT(h3attn_residual_change_noalloc(Q, K, max_n + 1, res, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_residual_change_noalloc(Q, K, 0, res, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_residual_change_noalloc(Q, K, 100, nullptr, nullptr) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(g_launches == n0 + 1);
  // the reuse policy is host code on a caller-owned struct
  h3attn_cache_gate gate;
  EXPECT(h3attn_cache_gate_init(&gate, 0.05, 1) == H3ATTN_OK);
  EXPECT(h3attn_cache_gate_decide(&gate, 0.0) == 0);   // the first step always computes
  EXPECT(h3attn_cache_gate_decide(&gate, 0.01) == 1);  // small change: reuse
  EXPECT(h3attn_cache_gate_decide(&gate, 0.01) == 0);  // at most one reuse in a row
  EXPECT(h3attn_cache_gate_decide(&gate, 0.2) == 0);
  {
    const double small[2] = {0.5, 100.0}, zero_prev[2] = {0.0, 0.0};
    EXPECT(h3attn_cache_gate_init(&gate, 0.05, 3) == H3ATTN_OK);
    EXPECT(h3attn_cache_gate_decide_sums(&gate, nullptr) == 0);    // first step: nothing to compare with
    EXPECT(h3attn_cache_gate_decide_sums(&gate, small) == 1);      // 0.005 < 0.05
    EXPECT(h3attn_cache_gate_decide_sums(&gate, zero_prev) == 0);  // no positive denominator: compute
    EXPECT(h3attn_cache_gate_decide_sums(nullptr, small) == -1);
  }
  EXPECT(h3attn_cache_gate_init(&gate, -1.0, 1) == H3ATTN_ERR_INVALID_ARGUMENT);
  EXPECT(h3attn_cache_gate_init(nullptr, 0.05, 1) == H3ATTN_ERR_INVALID_ARGUMENT);
}

void check_fp8() {
  const size_t fws = h3attn_fp8_workspace_bytes(1, 2, 640, 128, 64);
  EXPECT(fws > 0);
  uint8_t* q8 = P<uint8_t>(0x110000);
  uint8_t* k8 = P<uint8_t>(0x120000);
  uint8_t* v8 = P<uint8_t>(0x130000);
  float* qs = P<float>(0x140000);
  float* ks = P<float>(0x150000);
  float* vs = P<float>(0x160000);
  int n0 = g_launches;
  EXPECT(launched(h3attn_fp8_quantize(Q, K, V, q8, k8, v8, qs, ks, vs, 1, 2, 640, 128, 64, WS, fws, nullptr), n0));
  EXPECT(g_fq.n_blocks == 10 && g_fq.n_chunks == 1 && g_fq.head_dim == 128);
  EXPECT(h3attn_fp8_quantize(Q, K, V, P<uint8_t>(0x10000), k8, v8, qs, ks, vs, 1, 2, 640, 128, 64, WS, fws, nullptr) ==
         H3ATTN_ERR_INVALID_ARGUMENT);  // an output aliasing an input
  n0 = g_launches;
  EXPECT(launched(h3attn_fp8_block_sparse_fwd(q8, k8, v8, qs, ks, vs, P<const int32_t>(0xA0000), 3, O, nullptr, 1, 2,
                                              640, 128, 64, 3, nullptr), n0));
  EXPECT(g_fa.keep == 3 && g_fa.group_stride == 3 && g_fa.n_blocks == 10);
  EXPECT(h3attn_fp8_dense_fwd(q8, k8, v8, qs, ks, vs, O, nullptr, 1, 2, 640, 128, 32, nullptr) == H3ATTN_ERR_UNSUPPORTED);
}
}  // namespace

int main() {
  check_keep_count();
  check_norm_rope();
  check_attention();
  check_select();
  check_block_ops();
  check_fp8();
  EXPECT(std::strlen(h3attn_version()) > 0);
  std::printf("%s: %d launches recorded, %d failures\n", g_fail ? "FAILED" : "ok", g_launches, g_fail);
  return g_fail ? 1 : 0;
}
