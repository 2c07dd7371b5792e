// A plain C++ host program that drives the whole attention path through the C-ABI alone (no
// Python, no torch): QK norm+RoPE -> dense attention -> SubBlock selection -> block-sparse
// attention, on device buffers it allocates itself and one stream of its own.
//
// usage: c_abi_consumer IN OUT
//   IN  (little-endian): int32 batch, t, h, w, heads, head_dim, d_t, d_h, d_w; float theta, eps;
//       double sparsity; then q, k, v as raw bf16 [batch, t*h*w, heads, head_dim]; then the
//       float32 norm weights w_q, w_k [head_dim].
//   OUT: q', k', the dense output (bf16, same shape), the dense LSE (float32 [batch, heads, N]),
//       int32 keep, the kept key blocks (int32 [batch, heads, nB, keep]), the block-sparse output.
// Exit status 0 on success; on any failure the entry point's error text goes to stderr.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "h3attn.h"

namespace {

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    const hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      std::exit(2);                                                                    \
    }                                                                                  \
  } while (0)

#define H3_OK(call)                                                                    \
  do {                                                                                 \
    const h3attn_status s_ = (call);                                                   \
    if (s_ != H3ATTN_OK) {                                                             \
      std::fprintf(stderr, "%s returned %d: %s\n", #call, (int)s_, h3attn_last_error()); \
      std::exit(3);                                                                    \
    }                                                                                  \
  } while (0)

template <typename T>
void read_into(FILE* f, T* dst, size_t count) {
  if (std::fread(dst, sizeof(T), count, f) != count) {
    std::fprintf(stderr, "input file too short\n");
    std::exit(4);
  }
}

template <typename T>
void write_from(FILE* f, const T* src, size_t count) {
  if (std::fwrite(src, sizeof(T), count, f) != count) {
    std::fprintf(stderr, "cannot write the output file\n");
    std::exit(5);
  }
}

template <typename T>
T* device_copy(const std::vector<T>& host) {
  T* d = nullptr;
  HIP_OK(hipMalloc(&d, host.size() * sizeof(T)));
  HIP_OK(hipMemcpy(d, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

template <typename T>
T* device_alloc(size_t count) {
  T* d = nullptr;
  HIP_OK(hipMalloc(&d, count * sizeof(T)));
  return d;
}

template <typename T>
std::vector<T> host_copy(const T* d, size_t count) {
  std::vector<T> h(count);
  HIP_OK(hipMemcpy(h.data(), d, count * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) {
    std::fprintf(stderr, "cannot open %s\n", argv[1]);
    return 1;
  }
  int32_t hdr[9];
  float theta_eps[2];
  double sparsity;
  read_into(in, hdr, 9);
  read_into(in, theta_eps, 2);
  read_into(in, &sparsity, 1);
  const int32_t batch = hdr[0], heads = hdr[4], head_dim = hdr[5];
  const h3attn_grid grid{hdr[1], hdr[2], hdr[3]};
  const int64_t n = (int64_t)grid.t * grid.h * grid.w;
  const size_t elems = (size_t)batch * n * heads * head_dim;
  std::vector<h3attn_bf16> q(elems), k(elems), v(elems);
  std::vector<float> wq(head_dim), wk(head_dim);
  read_into(in, q.data(), elems);
  read_into(in, k.data(), elems);
  read_into(in, v.data(), elems);
  read_into(in, wq.data(), head_dim);
  read_into(in, wk.data(), head_dim);
  std::fclose(in);

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  h3attn_bf16 *dq = device_copy(q), *dk = device_copy(k), *dv = device_copy(v);
  float *dwq = device_copy(wq), *dwk = device_copy(wk);
  h3attn_bf16* dqo = device_alloc<h3attn_bf16>(elems);
  h3attn_bf16* dko = device_alloc<h3attn_bf16>(elems);
  h3attn_bf16* dout = device_alloc<h3attn_bf16>(elems);
  h3attn_bf16* dsparse = device_alloc<h3attn_bf16>(elems);
  float* dlse = device_alloc<float>((size_t)batch * heads * n);

  H3_OK(h3attn_qk_norm_rope(dq, dk, dqo, dko, dwq, dwk, batch, heads, head_dim, grid, hdr[6], hdr[7], hdr[8],
                            theta_eps[0], theta_eps[1], stream));
  H3_OK(h3attn_dense_fwd(dqo, dko, dv, dout, dlse, batch, heads, n, head_dim, stream));
  const int32_t nb = (int32_t)((n + 63) / 64);
  const int32_t keep = h3attn_keep_count(nb, sparsity);
  if (keep < 1) {
    std::fprintf(stderr, "h3attn_keep_count(%d, %g) = %d\n", nb, sparsity, keep);
    return 3;
  }
  const size_t ws_bytes = h3attn_select_workspace_bytes(batch, heads, n, head_dim, 64);
  void* ws = device_alloc<unsigned char>(ws_bytes);  // hipMalloc memory is 256-byte aligned
  const size_t idx_count = (size_t)batch * heads * nb * keep;
  int32_t* didx = device_alloc<int32_t>(idx_count);
  H3_OK(h3attn_subblock_select(dqo, dko, batch, heads, n, head_dim, 64, sparsity, keep, didx, ws, ws_bytes, stream));
  H3_OK(h3attn_block_sparse_fwd(dqo, dko, dv, didx, keep, dsparse, nullptr, batch, heads, n, head_dim, 64, stream));

  // the same selection with the pooling inside the norm+RoPE pass: q', k' and the kept sets must be
  // the same bits as the stand-alone calls' above
  h3attn_bf16* dqo2 = device_alloc<h3attn_bf16>(elems);
  h3attn_bf16* dko2 = device_alloc<h3attn_bf16>(elems);
  int32_t* didx2 = device_alloc<int32_t>(idx_count);
  void* ws2 = device_alloc<unsigned char>(ws_bytes);
  H3_OK(h3attn_qk_norm_rope_pool(dq, dk, dqo2, dko2, dwq, dwk, batch, heads, head_dim, grid, hdr[6], hdr[7], hdr[8],
                                 theta_eps[0], theta_eps[1], 64, ws2, ws_bytes, stream));
  H3_OK(h3attn_subblock_select_pooled(batch, heads, n, head_dim, 64, sparsity, keep, didx2, ws2, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  if (host_copy(dqo, elems) != host_copy(dqo2, elems) || host_copy(dko, elems) != host_copy(dko2, elems) ||
      host_copy(didx, idx_count) != host_copy(didx2, idx_count)) {
    std::fprintf(stderr, "the pooled path differs from the stand-alone calls\n");
    return 4;
  }
  for (void* p : {(void*)dqo2, (void*)dko2, (void*)didx2, ws2}) HIP_OK(hipFree(p));

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) {
    std::fprintf(stderr, "cannot open %s\n", argv[2]);
    return 1;
  }
  write_from(out, host_copy(dqo, elems).data(), elems);
  write_from(out, host_copy(dko, elems).data(), elems);
  write_from(out, host_copy(dout, elems).data(), elems);
  write_from(out, host_copy(dlse, (size_t)batch * heads * n).data(), (size_t)batch * heads * n);
  write_from(out, &keep, 1);
  write_from(out, host_copy(didx, idx_count).data(), idx_count);
  write_from(out, host_copy(dsparse, elems).data(), elems);
  std::fclose(out);

  for (void* p : {(void*)dq, (void*)dk, (void*)dv, (void*)dwq, (void*)dwk, (void*)dqo, (void*)dko, (void*)dout,
                  (void*)dsparse, (void*)dlse, ws, (void*)didx})
    HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(stream));
  std::printf("c_abi_consumer: %s ok (N=%lld, heads=%d, D=%d, keep=%d; pooled path identical)\n", h3attn_version(),
              (long long)n, heads,
              head_dim, keep);
  return 0;
}
