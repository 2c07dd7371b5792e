// Dense and block-sparse flash-style attention forward for gfx950 (bf16 MFMA, fp32 softmax).
//
// Sources: "MiniMax-H3 在 8×H200 上基准测试…" (chat-gpts.plus), section "为什么重要" — attention over
// the long latent sequence is a main cost; "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能"
// (xiaodao.ai), section "6.24 倍里，真正有损的部分大约是三倍" — SubBlock sends only the kept
// 64-token key blocks of each query block to a block-sparse attention kernel.
//
// Formulation. Each wave owns 32 query rows (two 16-query column tiles) and computes the
// transposed score tile
//   S^T (keys x queries) = K (keys x D) . Q^T (D x queries)
// with v_mfma_f32_16x16x32_bf16 on 16x16 tiles, K as the A operand (read from LDS, each fragment
// used for both query tiles) and Q^T as the B operand (held in registers for the whole loop). In
// the accumulator layout a lane holds 4 keys of each 16-key tile for one query per query tile, so
// a query's row statistics span the 4 lanes l, l^16, l^32, l^48 (two cross-lane swaps, shared by
// both query tiles, for the max; the row sum stays a per-lane partial until the epilogue). The exponentials P^T are
// converted to bf16 in place and used directly as the B operand of
//   O^T (D x queries) += V^T (D x keys) . P^T (keys x queries),
// whose A operand (V^T) is read from a row-major V tile with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16). The key order inside each 32-key MFMA step is permuted identically on
// both operands so that it matches the registers that already hold P^T. The softmax uses exp2
// with log2(e)/sqrt(D) folded into one FMA, and the running max only moves (with a wave-uniform
// O rescale) when a tile exceeds it by more than 2^8. (The same work on 32x32x16 tiles, one query
// per lane, measured 2.1 % slower in the dense kernel.)
//
// Pipeline: tile t+1 is loaded from global memory straight into the other half of a
// double-buffered LDS tile while tile t is computed (one barrier per tile). Dense:
// 8 waves (256 queries) share each 64-key K/V tile, two waves per SIMD (256-register budget) so
// one wave's MFMAs overlap the other's softmax. Block-sparse: a workgroup takes 4 query blocks
// (consecutive, or one per frame at the same position with a group stride) and walks the union
// of their kept key blocks (see attn_sparse_group_kernel).
#include "device_util.h"
#include "kernels.h"
#include "launch_util.h"
#include "sparse_union.h"

namespace h3attn {
namespace {

constexpr int kBN = 64;  // keys per tile (= SubBlock block size)

#define kOnes2 (__builtin_bit_cast(bf16x2, 0x3f803f80u))  // bf16 pair (1.0, 1.0)

// SwzLayout: the K and V tiles of 64 keys in LDS, unpadded rows of 2D bytes (CPR = D/8 chunks),
// filled by direct global -> LDS loads, which write each wave instruction's 64 x 16 bytes to
// consecutive LDS addresses, so rows cannot be padded. The chunks of a row are rotated instead,
// by a function of the row, so that the chunks one read instruction touches fall on distinct
// banks whether a read cycle serves 256 or 128 bytes. A K read takes one chunk of 16 consecutive
// rows per 16 lanes; a V transpose read takes 2 adjacent chunks of 4 consecutive rows per 16 lanes
// (8 rows per 32 lanes):
//   D = 128 (16 chunks per row): K chunk c of row r at column (c + r) mod 16, V at (c + 2r) mod 16;
//   D = 64 (8 chunks, two rows per 256 bytes): K at (c + (r xor bit3(r))) mod 8, V at
//   (c + 2 ((r mod 4) xor bit2(r))) mod 8.
// The rotations only use the row's low 4 bits, so a lane's columns do not change with the 16-key
// tile or the 32-key step. (V rotated by 4r, as for reads of 4 rows x 4 chunks, conflicted 2-way
// here: 1.0 bank conflicts per LDS access in the PMC counters.)
template <int D>
struct SwzLayout {
  static constexpr int ROW = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int K_BYTES = kBN * ROW;
  static constexpr int BUF_BYTES = 2 * K_BYTES;
  __device__ static __forceinline__ int krot(int r) { return D == 128 ? r : r ^ ((r >> 3) & 1); }
  __device__ static __forceinline__ int vrot(int r) { return D == 128 ? 2 * r : 2 * ((r & 3) ^ ((r >> 2) & 1)); }
  __device__ static __forceinline__ int kcol(int r, int c) { return (c + krot(r)) & (CPR - 1); }
  __device__ static __forceinline__ int vcol(int r, int c) { return (c + vrot(r)) & (CPR - 1); }
  // logical chunk stored at column col of row r (the inverses)
  __device__ static __forceinline__ int kchunk(int r, int col) { return (col - krot(r)) & (CPR - 1); }
  __device__ static __forceinline__ int vchunk(int r, int col) { return (col - vrot(r)) & (CPR - 1); }
};

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// sum over the lanes l, l^16, l^32 and l^48 (the four lanes that hold one query)
__device__ __forceinline__ float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// One wave's share of the forward pass: 32 query rows q0 .. q0+31 as two 16-query tiles, their
// Q^T fragments (B operand: [query tile][32-channel step]), the O^T accumulators ([16-channel
// tile][query tile]), the running softmax statistics per query tile, and the lane's LDS read
// offsets. Lane l holds query 16 qt + l%16 of each tile; within a 16-key (16-channel) MFMA tile,
// rows 4 (l/16) .. +3.
// K fragment of k step ks, 16-key tile kt: key row 16 kt + l%16, chunk 4 ks + l/16 (koff[ks]; kt
// adds whole rotations). V transpose reads of 32-key step s, 16-channel tile dt: within each group
// of 16 lanes, rows 32 s + 4 (l/16) + s' (s' = 0..3, then the same + 16) at channels 16 dt + l%16
// (voff[dt]).
template <int D>
struct WaveRows {
  bf16x8 qf[2][D / 32];
  f32x4 o[D / 16][2];
  float m_run[2];     // running max of s*sc (log2 units) per query tile, shared by the query's 4 lanes
  float m_thr[2];     // m_run + 8: a tile max above it moves the running max
  float thr_mix;      // m_thr of query tile (l/16)&1, the tile whose maximum lane l's row holds
  float l_part[2][2]; // per-lane partial row sums, two chains per query tile across all tiles
  int koff[D / 32];
  int voff[D / 16];
};

template <int D>
__device__ __forceinline__ void rows_begin(WaveRows<D>& w, const uint16_t* q, int64_t base, int64_t q0, int64_t N,
                                           int64_t row_stride, int lane) {
  using L = SwzLayout<D>;
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    int64_t my = q0 + 16 * qt + i16;
    my = my < N ? my : N - 1;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      w.qf[qt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + base + my * row_stride + 32 * ks + 8 * g));
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) w.o[dt][qt] = f32x4{};
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    w.m_run[qt] = -INFINITY;
    w.m_thr[qt] = -INFINITY;
    w.thr_mix = -INFINITY;
    w.l_part[qt][0] = w.l_part[qt][1] = 0.f;
  }
  // the rotations depend on bits of the row that 16-key and 32-key steps leave unchanged
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) w.koff[ks] = i16 * L::ROW + L::kcol(i16, 4 * ks + g) * 16;
  const int r = 4 * g + (i16 >> 2);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int byte = 32 * dt + 8 * (i16 & 3);
    w.voff[dt] = r * L::ROW + L::vcol(r, byte / 16) * 16 + byte % 16;
  }
}

// One K/V tile of 64 keys (K rows at kb, V rows at vb in LDS; first key key0) applied to the
// wave's rows: S^T = K . Q^T, online softmax, O^T += V^T . P^T. In the tile that holds the last
// token when N is not a multiple of 64, keys at or past N get a score of -inf. MASK selects how
// that tile is told apart: 0 (the tile is whole) and 1 (it is the partial tile) are separate
// instances, so that the dense loop's tile code has no branch between the score MFMAs and the
// softmax; 2 tests `partial` (wave-uniform) at run time, which the block-sparse kernel keeps (two
// instances inside its loop needed more than 256 registers). The running max only moves when the tile max exceeds it by more than 8 (a factor
// 256): until then exp2 values stay <= 256, which fp32 sums and bf16 P hold exactly enough, and
// the rescale (a wave-uniform branch) is skipped. The row sum of the bf16-rounded P that P.V uses
// is accumulated with packed dot products against (1, 1).
template <int D, int MASK>
__device__ __forceinline__ void rows_tile(WaveRows<D>& w, const unsigned char* kb, const unsigned char* vb,
                                          int64_t key0, int64_t N, bool partial, int lane, float sc) {
  using L = SwzLayout<D>;
  const int g = lane >> 4;
  f32x4 s[4][2];  // [16-key tile][query tile]
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) s[kt][qt] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    bf16x8 a[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) a[kt] = *reinterpret_cast<const bf16x8*>(kb + 16 * kt * L::ROW + w.koff[ks]);
    // query-tile-major: in the last k step query tile 0's scores are complete four MFMAs early
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt][qt] = mfma16x16x32(a[kt], w.qf[qt][ks], s[kt][qt]);
  }
  if (MASK == 1 || (MASK == 2 && partial)) {
    const int valid = (int)(N - key0);  // below 64
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * kt + 4 * g + i >= valid) {
          s[kt][0][i] = -INFINITY;
          s[kt][1][i] = -INFINITY;
        }
  }
  // Row maxima. The lane's 16 scores of each query tile reduce as one chain of 3-input maxima (8
  // instructions); the four lanes of a query then combine them across lanes.
  float ml[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    ml[qt] = fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), s[0][qt][2]);
#pragma unroll
    for (int i = 3; i + 1 < 16; i += 2)
      ml[qt] = fmaxf(fmaxf(ml[qt], s[i / 4][qt][i % 4]), s[(i + 1) / 4][qt][(i + 1) % 4]);
    ml[qt] = fmaxf(ml[qt], s[3][qt][3]);
  }
  // rescale query tile qt when its running max moves; mx: this lane's query's scaled tile max
  auto rescale = [&](int qt, float mx) {
    const float m_new = fmaxf(w.m_run[qt], mx);
    const float alpha = fast_exp2(w.m_run[qt] - m_new);
    w.m_run[qt] = m_new;
    w.m_thr[qt] = m_new + 8.0f;
    w.l_part[qt][0] *= alpha;
    w.l_part[qt][1] *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) w.o[dt][qt][i] *= alpha;
  };
  // Both query tiles in one cross-lane pass: one v_permlane16_swap of the two partial maxima and
  // a max leave, in 16-lane rows 0 and 2, query tile 0's maximum over the lane pair (l, l^16)
  // and, in rows 1 and 3, query tile 1's; v_permlane32_swap completes the four-lane maximum. So
  // z is the scaled tile max of query l%16 of query tile (l/16)&1, compared with that tile's
  // threshold (thr_mix) in one instruction. Only when a running max moves (rare) is z swapped
  // once more, which gives every lane both tiles' maxima.
  const auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(ml[0]), __float_as_uint(ml[1]), false, false);
  const float z = pair_max(fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1]))) * sc;
  const uint64_t over = __ballot(z > w.thr_mix);
  if (over) {
    const auto zz = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
      if (over & (qt ? 0xFFFF0000FFFF0000ull : 0x0000FFFF0000FFFFull)) rescale(qt, __uint_as_float(zz[qt]));
    w.thr_mix = (g & 1) ? w.m_thr[1] : w.m_thr[0];
  }
  bf16x8 pb[2][2];  // P^T B operands [query tile][32-key step]
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float mr = w.m_run[qt];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      u32x4 pk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // operand bytes 0..7: keys 32 ks2 + 4 g + i; 8..15: the same + 16
        const f32x4 t = s[2 * ks2 + h][qt];
        const uint32_t p01 = pack_bf16x2(fast_exp2(fmaf(t[0], sc, -mr)), fast_exp2(fmaf(t[1], sc, -mr)));
        const uint32_t p23 = pack_bf16x2(fast_exp2(fmaf(t[2], sc, -mr)), fast_exp2(fmaf(t[3], sc, -mr)));
        pk[2 * h] = p01;
        pk[2 * h + 1] = p23;
        w.l_part[qt][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p01), kOnes2, w.l_part[qt][0], false);
        w.l_part[qt][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p23), kOnes2, w.l_part[qt][1], false);
      }
      pb[qt][ks2] = __builtin_bit_cast(bf16x8, pk);
    }
  }
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const unsigned char* p1 = vb + 32 * ks2 * L::ROW + w.voff[dt];
      const i16x4 lo = lds_read_tr16(p1);
      const i16x4 hi4 = lds_read_tr16(p1 + 16 * L::ROW);
      typedef __attribute__((ext_vector_type(8))) short i16x8;
      const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      const bf16x8 av = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) w.o[dt][qt] = mfma16x16x32(av, pb[qt][ks2], w.o[dt][qt]);
    }
  }
}

// Epilogue: combine the lane-partial sums over the query's 4 lanes, normalise and store the rows
// inside the sequence (out: the output tensor at the (batch, head) base; lse_row: the LSE row of
// the (batch, head), or null). Rows that saw no key (an empty kept set) are written as zeros with
// LSE -inf.
template <int D>
__device__ __forceinline__ void rows_end(const WaveRows<D>& w, uint16_t* out, float* lse_row, int64_t q0,
                                         int64_t N, int64_t row_stride, bool empty, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float l_tot = quad_sum(w.l_part[qt][0] + w.l_part[qt][1]);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const int64_t my = q0 + 16 * qt + i16;
    if (my < N) {
      uint16_t* op = out + my * row_stride;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        u32x2 v;
        v[0] = pack_bf16x2(w.o[dt][qt][0] * inv, w.o[dt][qt][1] * inv);
        v[1] = pack_bf16x2(w.o[dt][qt][2] * inv, w.o[dt][qt][3] * inv);
        *reinterpret_cast<u32x2*>(op + 16 * dt + 4 * g) = v;
      }
      if (lse_row != nullptr && g == 0)
        lse_row[my] = empty ? -INFINITY : (w.m_run[qt] + __log2f(l_tot)) * 0.6931471805599453f;
    }
  }
}

// Direct global -> LDS staging of one K/V tile into the SwzLayout (gfx950 global_load_lds_dwordx4:
// no staging registers, no LDS write instructions). A wave instruction writes 64 lanes x 16 bytes
// to consecutive LDS addresses, so LDS slot p = 64 (J w + j) + lane of wave w's instruction j is
// row p / CPR, column p % CPR of the tile, and the lane fetches the logical chunk that the
// rotation puts at that column. The loads take the tile's first K and V rows as wave-uniform
// scalar bases and the lane's byte offset inside the tile (fixed for the whole kernel), so moving
// to another tile costs scalar adds only. Rows past the end of the sequence are clamped to the
// last token, only in the tile that holds it (the clamped offsets stay non-negative). The loads
// are counted by vmcnt: a wave waits for its own (wait_dma) before the barrier that hands the
// tile to the other waves.
template <int D, int NT>
struct TileDma {
  using L = SwzLayout<D>;
  static constexpr int WAVES = NT / 64;
  static constexpr int J = L::CPR / WAVES;  // instructions per wave and tensor
  static_assert(L::CPR % WAVES == 0, "the tile's 1 KB slices must split evenly over the waves");
  int krow[J];
  uint32_t koff[J], voff[J];  // byte offsets inside the tile: below 2^31 (rows < 64, heads <= 65535)
  int rs_bytes;               // bytes between consecutive tokens
  int lds0;                   // byte offset of the wave's first slice (wave-uniform)

  __device__ __forceinline__ void init(int tid, int64_t row_stride) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    lds0 = wave * J * 1024;
    rs_bytes = 2 * (int)row_stride;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int p = 64 * (J * wave + j) + lane;
      const int r = p / L::CPR, col = p % L::CPR;
      krow[j] = r;
      koff[j] = (uint32_t)(r * rs_bytes + 16 * L::kchunk(r, col));
      voff[j] = (uint32_t)(r * rs_bytes + 16 * L::vchunk(r, col));
    }
  }
  // tk, tv: the tile's first K and V rows (wave-uniform); whole: all 64 rows lie inside the
  // sequence, else last = index of the last valid row in the tile; buf: LDS byte address of the
  // tile buffer (wave-uniform)
  __device__ __forceinline__ void fetch(const unsigned char* tk, const unsigned char* tv, bool whole, int last,
                                        uint32_t buf) const {
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(buf + lds0);
    if (whole) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        lds_dma16_s(tk, koff[j], l0 + 1024 * j);
        lds_dma16_s(tv, voff[j], l0 + L::K_BYTES + 1024 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int adj = krow[j] < last ? 0 : (last - krow[j]) * rs_bytes;  // row min(r, last)
        lds_dma16_s(tk, (uint32_t)((int)koff[j] + adj), l0 + 1024 * j);
        lds_dma16_s(tv, (uint32_t)((int)voff[j] + adj), l0 + L::K_BYTES + 1024 * j);
      }
    }
  }
};

// Dense attention. WAVES waves per workgroup (32 queries each); OCC minimum waves per SIMD (2
// caps the kernel at 256 registers so that two waves share each SIMD and overlap each other's
// MFMA and softmax work).
template <int D, int WAVES, int OCC>
__global__ __launch_bounds__(WAVES * 64, OCC) void attn_fwd_kernel(AttnArgs a) {
  using L = SwzLayout<D>;
  constexpr int NT = WAVES * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int64_t N = a.n_tokens;
  const int64_t qtile = blockIdx.x;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t row_stride = (int64_t)a.heads * D;  // elements between consecutive tokens
  const int64_t base = ((int64_t)b * N) * row_stride + (int64_t)head * D;

  const int64_t q0 = qtile * (WAVES * 32) + wave * 32;  // the wave's first query row
  WaveRows<D> w;
  rows_begin(w, a.q, base, q0, N, row_stride, lane);

  const int n_tiles = (int)((N + kBN - 1) / kBN);
  const int last_partial = N % kBN ? n_tiles - 1 : -1;  // the tile to mask, if any
  TileDma<D, NT> dma;
  dma.init(tid, row_stride);
  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k + base);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v + base);
  const int64_t tile_bytes = (int64_t)kBN * 2 * row_stride;
  const int n_full = (int)(N / kBN);  // tiles that lie inside the sequence
  auto fetch_tile = [&](int tt, uint32_t buf) {
    dma.fetch(kbase + tt * tile_bytes, vbase + tt * tile_bytes, tt < n_full, (int)(N - 1 - (int64_t)tt * kBN), buf);
  };

  // LDS byte address of the tile buffers
  const uint32_t smem_lds = lds_address(smem);
  wait_own_loads();  // the Q fragments
  fetch_tile(0, smem_lds);
  wait_dma();
  __syncthreads();
  // the tiles that lie inside the sequence, then the one that holds the last token (if partial),
  // so that the loop's tile code has no masking branch between the score MFMAs and the softmax
  const int n_loop = last_partial >= 0 ? n_tiles - 1 : n_tiles;
  for (int t = 0; t < n_loop; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) fetch_tile(t + 1, smem_lds + (buf ^ 1) * L::BUF_BYTES);
    const unsigned char* kb = smem + buf * L::BUF_BYTES;
    rows_tile<D, 0>(w, kb, kb + L::K_BYTES, (int64_t)t * kBN, N, false, lane, sc);
    wait_dma();
    __syncthreads();
  }
  if (last_partial >= 0) {
    const unsigned char* kb = smem + (last_partial & 1) * L::BUF_BYTES;
    rows_tile<D, 1>(w, kb, kb + L::K_BYTES, (int64_t)last_partial * kBN, N, true, lane, sc);
  }
  rows_end(w, a.out + base, a.lse != nullptr ? a.lse + ((int64_t)b * a.heads + head) * N : nullptr, q0, N,
           row_stride, false, lane);
}

// Block-sparse attention over groups of G query blocks per workgroup (2 waves per block, 32
// queries each; the blocks i, i+S, ..., i+(G-1)S of the group stride S, 1 for consecutive
// blocks). Neighbouring query blocks (in the sequence or frame to frame) keep largely the same
// key blocks, so the workgroup merges the G kept lists into their union (ascending key-block
// order, with a bit per query block that keeps it) and loads each union tile into LDS once; a
// wave runs the tile only
// when its own block keeps it (a wave-uniform branch), otherwise it just joins the barrier.
// Each wave therefore sees exactly its block's kept tiles in ascending order, the same
// arithmetic as the one-block kernel on ascending lists. The union is built in windows of KW
// key blocks so that LDS use is bounded for any sequence length. Blocks of a group are spread
// so that the two waves of a SIMD (w and w+4) belong to different blocks.
template <int D, int G, int KW, bool CSR>
__global__ __launch_bounds__(G * 128, 2) void attn_sparse_group_kernel(AttnArgs a) {
  using L = SwzLayout<D>;
  static_assert(G == 2 || G == 4, "2 or 4 query blocks per workgroup");
  constexpr int WAVES = 2 * G;
  constexpr int NT = WAVES * 64;
  static_assert(KW <= (1 << 24), "window slots must fit in 24 bits");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* ulist = reinterpret_cast<uint32_t*>(smem + 2 * L::BUF_BYTES);  // KW words
  __shared__ int s_wave_tot[WAVES];
  __shared__ int s_nu;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int64_t N = a.n_tokens;
  const int64_t nb = a.n_blocks;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t row_stride = (int64_t)a.heads * D;
  const int64_t base = ((int64_t)b * N) * row_stride + (int64_t)head * D;

  const int gblk = __builtin_amdgcn_readfirstlane((wave & 1) + 2 * (wave >> 2));  // this wave's block in the group
  const int half = (wave >> 1) & 1;               // and its 32-query half
  const int64_t row0 = ((int64_t)b * a.heads + head) * nb;
  const int64_t qb = group_block<G>(blockIdx.x, gblk, a.group_stride, nb);
  const int64_t q0 = (qb < 0 ? 0 : qb) * kBN + half * 32;  // the wave's first query row

  // the kept list of each block of the group inside block_idx, in LDS; this wave's own length
  __shared__ int64_t s_range[2 * G];
  stash_group_ranges<G, CSR>(s_range, a.row_ptr, a.keep, row0, blockIdx.x, a.group_stride, nb);
  int64_t my_beg, my_end;
  kept_range<CSR>(a.row_ptr, a.keep, row0, qb, my_beg, my_end);
  const int64_t my_count = my_end - my_beg;

  WaveRows<D> w;
  rows_begin(w, a.q, base, q0, N, row_stride, lane);
  TileDma<D, NT> dma;
  dma.init(tid, row_stride);
  const uint32_t smem_lds = lds_address(smem);
  const float sc = 1.4426950408889634f / sqrtf((float)D);
  const uint32_t my_bit = 1u << gblk;

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(a.k + base);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(a.v + base);
  const int64_t tile_bytes = (int64_t)kBN * 2 * row_stride;
  const int n_full = (int)(N / kBN);  // key blocks that lie inside the sequence
  auto fetch_block = [&](int kblk, uint32_t buf) {  // kblk wave-uniform
    dma.fetch(kbase + kblk * tile_bytes, vbase + kblk * tile_bytes, kblk < n_full, (int)(N - 1 - (int64_t)kblk * kBN),
              buf);
  };

  for (int64_t j0 = 0; j0 < nb; j0 += KW) {
    const int nw = (int)(nb - j0 < KW ? nb - j0 : KW);
    const int nu = build_union_window<G, KW, NT>(ulist, s_wave_tot, &s_nu, a.block_idx, s_range, j0, nw);
    if (nu == 0) continue;

    // union entry t: (slot << 8) | (bit per block of the group that keeps it), read wave-uniform
    auto entry = [&](int t) -> uint32_t { return __builtin_amdgcn_readfirstlane(ulist[t]); };
    wait_own_loads();  // Q fragments, kept ranges and block lists
    fetch_block((int)j0 + (int)(entry(0) >> 8), smem_lds);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < nu; ++t) {
      const int buf = t & 1;
      const uint32_t e = entry(t);
      if (t + 1 < nu) fetch_block((int)j0 + (int)(entry(t + 1) >> 8), smem_lds + (buf ^ 1) * L::BUF_BYTES);
      if (e & my_bit) {
        const unsigned char* kb = smem + buf * L::BUF_BYTES;
        // a 64-bit compare here: the 32-bit block-index compare of the dense kernel measured 8 %
        // slower in this kernel
        const int64_t key0 = (j0 + (int64_t)(e >> 8)) * kBN;
        rows_tile<D, 2>(w, kb, kb + L::K_BYTES, key0, N, key0 + kBN > N, lane, sc);
      }
      wait_dma();
      __syncthreads();
    }
  }
  if (qb >= 0)
    rows_end(w, a.out + base, a.lse != nullptr ? a.lse + ((int64_t)b * a.heads + head) * N : nullptr, q0, N,
             row_stride, my_count <= 0, lane);
}

template <int D, int WAVES, int OCC>
void launch_dense(const AttnArgs& a, hipStream_t stream) {
  const size_t lds = 2 * SwzLayout<D>::BUF_BYTES;
  auto kern = attn_fwd_kernel<D, WAVES, OCC>;
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds);
  const dim3 grid((unsigned)((a.n_tokens + WAVES * 32 - 1) / (WAVES * 32)), (unsigned)a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), lds, stream, a);
}

template <int D, int G, int KW, bool CSR>
void launch_group(const AttnArgs& a, hipStream_t stream) {
  const size_t lds = 2 * SwzLayout<D>::BUF_BYTES + (size_t)KW * 4;
  auto kern = attn_sparse_group_kernel<D, G, KW, CSR>;
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds);
  const dim3 grid((unsigned)n_groups<G>(a.n_blocks, a.group_stride), (unsigned)a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL(kern, grid, dim3(G * 128), lds, stream, a);
}

}  // namespace

// 8 waves (256 queries) per workgroup, two waves per SIMD
void launch_dense_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_dense<128, 8, 2>(a, stream);
  else launch_dense<64, 8, 2>(a, stream);
}

// 4 query blocks per workgroup; union windows of 4096 key blocks (16 KB of LDS)
void launch_block_sparse_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_group<128, 4, 4096, false>(a, stream);
  else launch_group<64, 4, 4096, false>(a, stream);
}

void launch_block_sparse_csr_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_group<128, 4, 4096, true>(a, stream);
  else launch_group<64, 4, 4096, true>(a, stream);
}

}  // namespace h3attn
