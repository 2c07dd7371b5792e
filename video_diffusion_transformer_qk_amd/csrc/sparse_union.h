// Union of the kept key blocks of G query blocks, for the block-sparse kernels that give one
// workgroup several query blocks ("MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai),
// section "6.24 倍里，真正有损的部分大约是三倍": each query block attends to its kept 64-token key
// blocks only). Neighbouring query blocks keep largely the same key blocks, so a workgroup that
// loads each key block of the union once serves all of them.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace h3attn {

// The query blocks of workgroup `group`: with stride 1, G consecutive blocks; with stride S > 1,
// the blocks p + S*(f0 + j), j < G, of column p = group % S and first row f0 = G*(group / S) of
// the blocks laid out S per row (for a video latent with S = H*W/64, the same spatial position
// in G consecutive frames). Blocks past n_blocks are -1. group and S are below 2^31.
template <int G>
__device__ __forceinline__ int64_t group_block(uint32_t group, int j, uint32_t stride, int64_t n_blocks) {
  const int64_t qb = stride <= 1 ? (int64_t)group * G + j
                                 : (int64_t)(group % stride) + (int64_t)stride * ((int64_t)G * (group / stride) + j);
  return qb < n_blocks ? qb : -1;
}

// Number of workgroups for n_blocks query blocks with group stride S.
template <int G>
__host__ __device__ __forceinline__ int64_t n_groups(int64_t n_blocks, int64_t stride) {
  if (stride <= 1) return (n_blocks + G - 1) / G;
  const int64_t rows = (n_blocks + stride - 1) / stride;
  return (rows + G - 1) / G * stride;
}

// The kept list [beg, end) of query block qb inside block_idx (row row0 + qb: a top-k row of
// `keep` entries, or a CSR row through row_ptr); empty for qb = -1.
template <bool CSR>
__device__ __forceinline__ void kept_range(const int64_t* row_ptr, int32_t keep, int64_t row0, int64_t qb,
                                           int64_t& beg, int64_t& end) {
  if (qb < 0) {
    beg = end = 0;
  } else if constexpr (CSR) {
    beg = row_ptr[row0 + qb];
    end = row_ptr[row0 + qb + 1];
  } else {
    beg = (row0 + qb) * keep;
    end = beg + keep;
  }
}

// Threads 0..G-1 store the kept range of the group's block `tid` as s_range[2 tid], s_range[2 tid + 1]
// (LDS, read by build_union_window after its first barrier): the G ranges stay out of registers
// for the whole key loop.
template <int G, bool CSR>
__device__ __forceinline__ void stash_group_ranges(int64_t* s_range, const int64_t* row_ptr, int32_t keep,
                                                   int64_t row0, uint32_t group, uint32_t stride, int64_t n_blocks) {
  const int tid = threadIdx.x;
  if (tid < G) {
    int64_t b, e;
    kept_range<CSR>(row_ptr, keep, row0, group_block<G>(group, tid, stride, n_blocks), b, e);
    s_range[2 * tid] = b;
    s_range[2 * tid + 1] = e;
  }
}

// Builds, in `ulist` (KW words of LDS), the ascending list of the key blocks j0 .. j0+nw-1 that
// at least one of the G lists [s_range[2g], s_range[2g+1]) of block_idx keeps, each entry
// (j - j0) << 8 | bits (bit g: block g keeps it), and returns its length. NT threads take part;
// s_wave_tot holds NT/64 ints. Every thread must call it (it contains barriers); on return the
// list is visible to all threads. Entries outside the window are ignored, so indices are merged
// whatever their order within a list.
template <int G, int KW, int NT>
__device__ __forceinline__ int build_union_window(uint32_t* ulist, int* s_wave_tot, int* s_nu,
                                                  const int32_t* block_idx, const int64_t* s_range, int64_t j0,
                                                  int nw) {
  constexpr int WAVES = NT / 64;
  constexpr int PER = KW / NT;  // window slots per thread in the compaction
  static_assert(KW % NT == 0 && G <= 8, "window must split evenly; at most 8 membership bits");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < KW; i += NT) ulist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t end = s_range[2 * g + 1];
    for (int64_t e = s_range[2 * g] + tid; e < end; e += NT) {
      const int64_t j = block_idx[e] - j0;
      if (j >= 0 && j < nw) atomicOr(&ulist[j], 1u << g);
    }
  }
  __syncthreads();
  // compaction into (slot << 8 | bits); each thread owns PER consecutive slots
  uint32_t mk[PER];
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    mk[i] = ulist[tid * PER + i];
    c += mk[i] != 0u;
  }
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave_tot[wave] = incl;
  __syncthreads();  // also orders every read of the bit array before the writes below
  int pre = 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) pre += v < wave ? s_wave_tot[v] : 0;
  int pos = pre + incl - c;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (mk[i] != 0u) ulist[pos++] = ((uint32_t)(tid * PER + i) << 8) | mk[i];
  if (tid == NT - 1) *s_nu = pos;
  __syncthreads();
  return *s_nu;
}

}  // namespace h3attn
