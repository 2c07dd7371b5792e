// Union of the kept key blocks of G query blocks, for the block-sparse kernels that give one
// workgroup several query blocks ("MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai),
// section "6.24 倍里，真正有损的部分大约是三倍": each query block attends to its kept 64-token key
// blocks only). Neighbouring query blocks keep largely the same key blocks, so a workgroup that
// loads each key block of the union once serves all of them.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace h3attn {

// The kept list [beg[g], end[g]) of each of the G query blocks of group `group`, inside
// block_idx (top-k rows of `keep` entries, or CSR rows through row_ptr). Blocks past n_blocks
// get an empty list.
template <int G, bool CSR>
__device__ __forceinline__ void group_lists(const int64_t* row_ptr, int32_t keep, int64_t row0, int64_t group,
                                            int64_t n_blocks, int64_t (&beg)[G], int64_t (&end)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (group * G + g >= n_blocks) {
      beg[g] = end[g] = 0;
    } else if constexpr (CSR) {
      beg[g] = row_ptr[row0 + g];
      end[g] = row_ptr[row0 + g + 1];
    } else {
      beg[g] = (row0 + g) * keep;
      end[g] = beg[g] + keep;
    }
  }
}

// Builds, in `ulist` (KW words of LDS), the ascending list of the key blocks j0 .. j0+nw-1 that
// at least one of the G lists keeps, each entry (j - j0) << 8 | bits (bit g: block g keeps it),
// and returns its length. NT threads take part; s_wave_tot holds NT/64 ints. Every thread must
// call it (it contains barriers); on return the list is visible to all threads. Entries outside
// the window are ignored, so indices are merged whatever their order within a list.
template <int G, int KW, int NT>
__device__ __forceinline__ int build_union_window(uint32_t* ulist, int* s_wave_tot, int* s_nu,
                                                  const int32_t* block_idx, const int64_t (&beg)[G],
                                                  const int64_t (&end)[G], int64_t j0, int nw) {
  constexpr int WAVES = NT / 64;
  constexpr int PER = KW / NT;  // window slots per thread in the compaction
  static_assert(KW % NT == 0 && G <= 8, "window must split evenly; at most 8 membership bits");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < KW; i += NT) ulist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g)
    for (int64_t e = beg[g] + tid; e < end[g]; e += NT) {
      const int64_t j = block_idx[e] - j0;
      if (j >= 0 && j < nw) atomicOr(&ulist[j], 1u << g);
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
