// Dense and block-sparse flash-style attention forward for gfx950 (bf16 MFMA, fp32 softmax).
//
// Sources: "MiniMax-H3 在 8×H200 上基准测试…" (chat-gpts.plus), section "为什么重要" — attention over
// the long latent sequence is a main cost; "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能"
// (xiaodao.ai), section "6.24 倍里，真正有损的部分大约是三倍" — SubBlock sends only the kept
// 64-token key blocks of each query block to a block-sparse attention kernel.
//
// Formulation. Each wave owns 32 query rows and computes the transposed score tile
//   S^T (keys x queries) = K (keys x D) . Q^T (D x queries)
// with v_mfma_f32_32x32x16_bf16, K as the A operand (read from LDS) and Q^T as the B operand
// (held in registers for the whole loop). In the MFMA accumulator layout a lane holds one query
// column and 16 key rows, so the softmax row statistics are mostly per-lane: the max needs one
// exchange with the lane 32 away, and the row sum stays a per-lane partial until the epilogue.
// The exponentials P^T are converted to bf16 in place and used directly as the B operand of
//   O^T (D x queries) += V^T (D x keys) . P^T (keys x queries),
// whose A operand (V^T) is read from a row-major V tile with the gfx950 LDS transpose read
// (ds_read_b64_tr_b16). The key order inside each 16-key MFMA step is permuted identically on
// both operands so that it matches the registers that already hold P^T.
//
// Pipeline: tile t+1 is fetched from global memory into registers while tile t is computed,
// then stored to LDS. Dense: 8 waves (256 queries) share each 64-key K/V tile, double-buffered
// in LDS (one barrier per tile), two waves per SIMD (256-register budget) so one wave's MFMAs
// overlap the other's softmax. Sparse: the workgroup is one 64-query block (2 waves) with a
// single LDS tile (two barriers per tile) so four workgroups fit per CU, and workgroups are
// ordered in windows of 1024 so that the resident ones cover one head (its K/V stays in the
// MALL) with each XCD on consecutive query blocks. The softmax uses exp2 with
// log2(e)/sqrt(D) folded into one FMA, and the running max only moves (with a wave-uniform O
// rescale) when a tile exceeds it by more than 2^8.
#include "device_util.h"
#include "kernels.h"

namespace h3attn {
namespace {

constexpr int kBN = 64;  // keys per tile (= SubBlock block size)
#define kOnes2 (__builtin_bit_cast(bf16x2, 0x3f803f80u))  // bf16 pair (1.0, 1.0)

template <int D, int BN>
struct Tile {
  static constexpr int KS = 2 * D + 16;   // K row stride in LDS (bytes): conflict-free b128 reads
  static constexpr int VS = 2 * D + 64;   // V row stride in LDS (bytes) for the transpose reads
  static constexpr int K_BYTES = BN * KS;
  static constexpr int V_BYTES = BN * VS;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int CHUNKS = BN * D / 8;  // 16-byte chunks per tensor tile
};

// Maps the linear workgroup id to a work item so that each of the 8 XCDs (which receive
// workgroups round-robin) processes one contiguous range of (query tile, head, batch) items:
// neighbouring query tiles of one head then share an XCD and its L2.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t lin, int64_t total) {
  const int64_t x = lin % 8, k = lin / 8, q = total / 8, r = total % 8;
  return x * q + (x < r ? x : r) + k;
}

// Same idea applied per window of 8*C consecutive workgroups: the workgroups resident at any
// time then cover one narrow range of items (one head's K/V stays in the 256 MB MALL), and
// inside the window each XCD gets C consecutive items.
template <int C>
__device__ __forceinline__ int64_t xcd_grouped(int64_t lin, int64_t total) {
  const int64_t base = lin / (8 * C) * (8 * C), k = lin - base, rem = total - base;
  if (rem >= 8 * C) return base + (k % 8) * C + k / 8;
  return base + xcd_contiguous(k, rem);
}

// Tuning knobs: WAVES waves per workgroup (32 queries each); OCC minimum waves per SIMD (2 caps
// the kernel at 256 registers so two waves share each SIMD and overlap each other's MFMA and
// softmax work); DBUF double-buffers the K/V tile in LDS (one barrier per tile) instead of
// keeping a single LDS tile (two barriers per tile, half the LDS, more workgroups per CU); XCD
// selects the workgroup order (0: grid order, 1: one contiguous range per XCD, C > 1: windows
// of 8*C workgroups); BN keys per tile (64, or 128 for dense: fewer barriers and less per-tile
// bookkeeping per MFMA).
template <int D, int WAVES, int OCC, bool DBUF, bool SPARSE, int XCD = 0, int BN = 64, bool CSR = false>
__global__ __launch_bounds__(WAVES * 64, OCC) void attn_fwd_kernel(AttnArgs a) {
  using T = Tile<D, BN>;
  static_assert(!SPARSE || BN == kBN, "block-sparse tiles are single 64-token blocks");
  constexpr int MT = BN / 32;  // 32-key sub-tiles per tile
  constexpr int NT = WAVES * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int LOADS = T::CHUNKS / NT;  // 16-byte loads per thread per tensor
  static_assert(T::CHUNKS % NT == 0, "tile must split evenly");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int64_t N = a.n_tokens;
  int64_t qtile;
  int head, b;
  if constexpr (XCD != 0) {
    const int64_t n_qt = SPARSE ? a.n_blocks : (N + WAVES * 32 - 1) / (WAVES * 32);
    const int64_t total = n_qt * a.heads * a.batch;
    const int64_t item = XCD == 1 ? xcd_contiguous(blockIdx.x, total) : xcd_grouped<XCD>(blockIdx.x, total);
    qtile = item % n_qt;
    head = (int)((item / n_qt) % a.heads);
    b = (int)(item / (n_qt * a.heads));
  } else {
    qtile = blockIdx.x;
    head = blockIdx.y;
    b = blockIdx.z;
  }
  const int64_t row_stride = (int64_t)a.heads * D;  // elements between consecutive tokens
  const int64_t base = ((int64_t)b * N) * row_stride + (int64_t)head * D;

  const int64_t qtile0 = qtile * (WAVES * 32);
  const int64_t q0 = qtile0 + wave * 32;
  const int64_t my_q = q0 + l32;
  const int64_t my_q_c = my_q < N ? my_q : N - 1;

  // Q^T fragments (B operand), one bf16x8 per 16-wide k step.
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = a.q + base + my_q_c * row_stride + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
  }

  int n_tiles;
  const int32_t* idx_row = nullptr;
  if constexpr (SPARSE && CSR) {
    const int64_t r = ((int64_t)b * a.heads + head) * a.n_blocks + qtile;
    const int64_t p0 = a.row_ptr[r];
    n_tiles = (int)(a.row_ptr[r + 1] - p0);
    idx_row = a.block_idx + p0;
  } else if constexpr (SPARSE) {
    n_tiles = a.keep;
    idx_row = a.block_idx + (((int64_t)b * a.heads + head) * a.n_blocks + qtile) * a.keep;
  } else {
    n_tiles = (int)((N + BN - 1) / BN);
  }
  if (n_tiles <= 0) {  // an empty kept set (CSR rows only): zero output, lse = -inf
    if (my_q < N) {
      uint16_t* op = a.out + base + my_q * row_stride;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * g + 4 * hi) = u32x2{0u, 0u};
      if (a.lse != nullptr && hi == 0) a.lse[((int64_t)b * a.heads + head) * N + my_q] = -INFINITY;
    }
    return;
  }
  auto tile_key0 = [&](int t) -> int64_t {
    if constexpr (SPARSE) return (int64_t)idx_row[t] * kBN;
    else return (int64_t)t * BN;
  };

  // global -> register staging of one K/V tile. Each thread's chunks sit at fixed offsets from
  // the tile's first row (32-bit: < 64 rows x row_stride); rows past the end of the sequence are
  // clamped to the last token, only in the tile that holds it.
  int toff[LOADS], trow[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int ci = tid + i * NT;
    trow[i] = ci / (D / 8);
    toff[i] = trow[i] * (int)row_stride + (ci % (D / 8)) * 8;
  }
  u32x4 kst[LOADS], vst[LOADS];
  auto fetch = [&](int t) {
    const int64_t key0 = tile_key0(t);
    const int64_t tile = base + key0 * row_stride;
    if (key0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        kst[i] = *reinterpret_cast<const u32x4*>(a.k + tile + toff[i]);
        vst[i] = *reinterpret_cast<const u32x4*>(a.v + tile + toff[i]);
      }
    } else {
      const int last = (int)(N - 1 - key0);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = trow[i] < last ? trow[i] : last;
        const int64_t off = tile + toff[i] + (int64_t)(r - trow[i]) * row_stride;
        kst[i] = *reinterpret_cast<const u32x4*>(a.k + off);
        vst[i] = *reinterpret_cast<const u32x4*>(a.v + off);
      }
    }
  };
  auto stash = [&](int buf) {
    unsigned char* kb = smem + buf * T::BUF_BYTES;
    unsigned char* vb = kb + T::K_BYTES;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int ci = tid + i * NT;
      const int row = ci / (D / 8);
      const int col = ci % (D / 8);
      *reinterpret_cast<u32x4*>(kb + row * T::KS + col * 16) = kst[i];
      *reinterpret_cast<u32x4*>(vb + row * T::VS + col * 16) = vst[i];
    }
  };

  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
  float m_run = -INFINITY;  // running max of s*sc (log2 units), shared by lanes l and l^32
  float l_run = 0.f;        // per-lane partial row sum
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};

  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = DBUF ? (t & 1) : 0;
    if (t + 1 < n_tiles) fetch(t + 1);

    const unsigned char* kb = smem + buf * T::BUF_BYTES;
    const unsigned char* vb = kb + T::K_BYTES;

    // S^T = K . Q^T for the 32-key sub-tiles of the tile
    f32x16 s[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) s[m] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kb + (32 * m + l32) * T::KS + (16 * ks + 8 * hi) * 2);
        s[m] = mfma32x32x16(kf, qf[ks], s[m]);
      }
    }

    // mask keys past the end of the sequence (only the tile that holds the last token)
    const int64_t key0 = tile_key0(t);
    if (key0 + BN > N) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t kidx = key0 + 32 * m + 8 * (r / 4) + 4 * hi + (r % 4);
          if (kidx >= N) s[m][r] = -INFINITY;
        }
    }

    // online softmax (log2 domain). The running max only moves when the tile max exceeds it by
    // more than 8 (a factor 256): until then exp2 values stay <= 256, which fp32 sums and bf16 P
    // hold exactly enough, and the O/l rescale (a wave-uniform branch) is skipped.
    // tile max as a shallow tree (independent partial maxima) rather than one long chain
    float mp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mp[j] = fmaxf(s[0][4 * j], s[0][4 * j + 1]);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (m > 0 || (r % 4) >= 2) mp[r / 4] = fmaxf(mp[r / 4], s[m][r]);
    float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
    mx = pair_max(mx) * sc;
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    float psum[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial row sums
    u32x4 pk[2 * MT];  // P^T as bf16, 8 values per 16-key step: step kk covers s[kk/2] regs 8*(kk%2) .. +7
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[m][r], sc, -m_run));
        const float p1 = fast_exp2(fmaf(s[m][r + 1], sc, -m_run));
        const uint32_t pp = pack_bf16x2(p0, p1);
        pk[2 * m + r / 8][(r % 8) / 2] = pp;
        // row sum of the bf16-rounded P that P.V uses: one packed dot product with (1, 1)
        psum[(r / 2) % 4] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes2, psum[(r / 2) % 4], false);
      }
    }
    l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);

    // O^T += V^T . P^T
    const int ig = lane & 15;  // index inside the 16-lane group
#pragma unroll
    for (int kk = 0; kk < 2 * MT; ++kk) {
      const int m = kk >> 1, half = kk & 1;
      const int k0 = 32 * m + 16 * half + 4 * hi;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[kk]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d0 = 32 * dt + 16 * ((lane >> 4) & 1);
        const unsigned char* p1 = vb + (k0 + (ig >> 2)) * T::VS + (d0 + 4 * (ig & 3)) * 2;
        const i16x4 lo = lds_read_tr16(p1);
        const i16x4 hi4 = lds_read_tr16(p1 + 8 * T::VS);
        typedef __attribute__((ext_vector_type(8))) short i16x8;
        const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pb, o[dt]);
      }
    }

    if constexpr (DBUF) {
      if (t + 1 < n_tiles) stash(buf ^ 1);
      __syncthreads();
    } else {
      __syncthreads();  // every wave is done reading the single tile
      if (t + 1 < n_tiles) {
        stash(0);
        __syncthreads();
      }
    }
  }

  // epilogue: combine the two lane-partial sums, normalise, store
  const float l_tot = pair_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (my_q < N) {
    uint16_t* op = a.out + base + my_q * row_stride;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hi;
        u32x2 w;
        w[0] = pack_bf16x2(o[dt][4 * g + 0] * inv, o[dt][4 * g + 1] * inv);
        w[1] = pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
    if (a.lse != nullptr && hi == 0)
      a.lse[((int64_t)b * a.heads + head) * N + my_q] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
  }
}


template <int D, int WAVES, int OCC, bool DBUF, bool SPARSE, int XCD = 0, int BN = 64, bool CSR = false>
void launch(const AttnArgs& a, hipStream_t stream) {
  const size_t lds = (DBUF ? 2 : 1) * Tile<D, BN>::BUF_BYTES;
  auto kern = attn_fwd_kernel<D, WAVES, OCC, DBUF, SPARSE, XCD, BN, CSR>;
  static const bool lds_ok = [&] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
  }();
  (void)lds_ok;
  dim3 grid;
  const int64_t n_qt = SPARSE ? a.n_blocks : (a.n_tokens + WAVES * 32 - 1) / (WAVES * 32);
  if constexpr (XCD != 0) grid = dim3((unsigned)(n_qt * a.heads * a.batch));
  else grid = dim3((unsigned)n_qt, (unsigned)a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), lds, stream, a);
}

}  // namespace

#ifndef H3ATTN_DENSE_CFG
#define H3ATTN_DENSE_CFG 8, 2, true
#endif
#ifndef H3ATTN_SPARSE_CFG
#define H3ATTN_SPARSE_CFG 2, 2, false
#endif
#ifndef H3ATTN_SPARSE_XCD
#define H3ATTN_SPARSE_XCD 128
#endif

void launch_dense_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch<128, H3ATTN_DENSE_CFG, false>(a, stream);
  else launch<64, H3ATTN_DENSE_CFG, false>(a, stream);
}

void launch_block_sparse_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch<128, H3ATTN_SPARSE_CFG, true, H3ATTN_SPARSE_XCD>(a, stream);
  else launch<64, H3ATTN_SPARSE_CFG, true, H3ATTN_SPARSE_XCD>(a, stream);
}

void launch_block_sparse_csr_fwd(const AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch<128, H3ATTN_SPARSE_CFG, true, H3ATTN_SPARSE_XCD, 64, true>(a, stream);
  else launch<64, H3ATTN_SPARSE_CFG, true, H3ATTN_SPARSE_XCD, 64, true>(a, stream);
}

}  // namespace h3attn
