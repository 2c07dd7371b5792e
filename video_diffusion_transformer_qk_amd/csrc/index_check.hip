// Validation of caller-built kept sets for the block-sparse entry points.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section
// "6.24 倍里，真正有损的部分大约是三倍": each query block attends to a set of kept 64-token key
// blocks. The attention kernels take such a set as given (distinct indices in [0, nB)) and do not
// check it on the hot path; these kernels check it on request and flag each bad row instead of
// trapping.
//
// One workgroup per row: a bitmap of nB bits in LDS marks the indices seen (an atomic OR returns
// whether the bit was already set), so a row is checked in one pass whatever its index order.
// Row flags: bit 0 an index outside [0, nB), bit 1 a repeated index, bit 2 (CSR) a row whose end
// is below its start or beyond the column capacity.
#include "device_util.h"
#include "kernels.h"
#include "launch_util.h"

namespace h3attn {
namespace {

constexpr int kCheckThreads = 256;

__device__ uint32_t check_entries(const int32_t* cols, int64_t count, int32_t nb, uint32_t* bitmap) {
  uint32_t bad = 0;
  for (int64_t e = threadIdx.x; e < count; e += kCheckThreads) {
    const int32_t j = cols[e];
    if (j < 0 || j >= nb) {
      bad |= 1u;
      continue;
    }
    const uint32_t bit = 1u << (j & 31);
    if (atomicOr(&bitmap[j >> 5], bit) & bit) bad |= 2u;
  }
  return bad;
}

__device__ void finish_row(uint32_t bad, uint8_t* flag) {
  __shared__ uint32_t s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) *flag = (uint8_t)s_bad;
}

__device__ void clear_bitmap(uint32_t* bitmap, int32_t nb) {
  for (int i = threadIdx.x; i < (nb + 31) / 32; i += kCheckThreads) bitmap[i] = 0u;
  __syncthreads();
}

// grid (rows): row r = (b * heads + head) * nB + i holds keep indices at block_idx[r * keep]
__global__ __launch_bounds__(kCheckThreads) void topk_rows_check_kernel(IndexCheckArgs a) {
  extern __shared__ uint32_t bitmap[];
  const int64_t r = blockIdx.x;
  clear_bitmap(bitmap, a.n_blocks);
  const uint32_t bad = check_entries(a.block_idx + r * a.keep, a.keep, a.n_blocks, bitmap);
  finish_row(bad, a.row_flags + r);
}

// grid (rows): row r holds col_idx[row_ptr[r] .. row_ptr[r+1])
__global__ __launch_bounds__(kCheckThreads) void csr_rows_check_kernel(IndexCheckArgs a) {
  extern __shared__ uint32_t bitmap[];
  const int64_t r = blockIdx.x;
  clear_bitmap(bitmap, a.n_blocks);
  const int64_t beg = a.row_ptr[r], end = a.row_ptr[r + 1];
  uint32_t bad = 0;
  if (beg < 0 || end < beg || end > a.col_capacity) bad = 4u;
  else bad = check_entries(a.block_idx + beg, end - beg, a.n_blocks, bitmap);
  finish_row(bad, a.row_flags + r);
}

template <typename K>
void launch_check(K kern, const IndexCheckArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)((a.n_blocks + 31) / 32) * sizeof(uint32_t);
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), (int)kIndexCheckLdsBytes);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.rows), dim3(kCheckThreads), lds, stream, a);
}

}  // namespace

void launch_check_topk_rows(const IndexCheckArgs& a, hipStream_t stream) {
  launch_check(topk_rows_check_kernel, a, stream);
}

void launch_check_csr_rows(const IndexCheckArgs& a, hipStream_t stream) {
  launch_check(csr_rows_check_kernel, a, stream);
}

}  // namespace h3attn
