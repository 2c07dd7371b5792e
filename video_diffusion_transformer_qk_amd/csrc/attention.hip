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
// both operands so that it matches the registers that already hold P^T. The softmax uses exp2
// with log2(e)/sqrt(D) folded into one FMA, and the running max only moves (with a wave-uniform
// O rescale) when a tile exceeds it by more than 2^8.
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

// One wave's share of the forward pass: 32 query rows, their Q^T fragments (B operand, one
// bf16x8 per 16-wide k step), the O^T accumulator and the running softmax statistics.
template <int D>
struct WaveRows {
  static constexpr int KSTEPS = D / 16;
  static constexpr int DT = D / 32;
  bf16x8 qf[KSTEPS];
  f32x16 o[DT];
  float m_run;  // running max of s*sc (log2 units), shared by lanes l and l^32
  float l_part[4];  // per-lane partial row sums, four independent chains across all tiles
};

template <int D>
__device__ __forceinline__ void rows_begin(WaveRows<D>& w, const uint16_t* qp) {
#pragma unroll
  for (int ks = 0; ks < WaveRows<D>::KSTEPS; ++ks)
    w.qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
#pragma unroll
  for (int dt = 0; dt < WaveRows<D>::DT; ++dt) w.o[dt] = f32x16{};
  w.m_run = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) w.l_part[j] = 0.f;
}

// Where a lane's operands sit in a K/V tile in LDS, for the MFMA fragment reads.
//
// qk_tile's fragment i (k step i/2, 32-key half i%2): this lane's key row 32 (i%2) + lane%32 and
// its 16-byte chunk 2 (i/2) + lane/32 of the K row. pv_tile's read (16-key step kk, 32-channel
// step dt): within each group of 16 lanes, 4 rows x 4 8-byte pieces of V, the lane's row
// 16 kk + 4 (lane/32) + (lane%16)/4 and channels 32 dt + 16 ((lane/16)%2) + 4 (lane%4); the second
// read of the pair is 8 rows further.
//
// SwzLayout: unpadded rows of 2D bytes (CPR = D/8 chunks), filled by direct global -> LDS loads,
// which write each wave instruction's 64 x 16 bytes to consecutive LDS addresses, so rows cannot
// be padded. The chunks of a row are rotated instead, so that the chunks one read instruction
// touches fall on distinct banks (the bank positions of rows padded to 17 (K) or 20 (V) chunks):
//   K: chunk c of row r at column (c + r) mod 16 (D = 128) or (c + r/2) mod 8 (D = 64);
//   V: chunk c of row r at column (c + 4r) mod 16 (D = 128) or (c + 4 (r/2)) mod 8 (D = 64).
// A lane's columns depend only on the lane and the k (channel) step, never on the 32-key half or
// the 16-key step, so the offsets are computed once per kernel (D/16 for K, D/32 for V) and the
// steps add constants.
template <int D>
struct SwzLayout {
  static constexpr int ROW = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int K_BYTES = kBN * ROW;
  static constexpr int BUF_BYTES = 2 * K_BYTES;
  static constexpr int V8 = 8 * ROW;
  __device__ static __forceinline__ int kcol(int r, int c) {
    return D == 128 ? (c + r) & 15 : (c + (r >> 1)) & 7;
  }
  __device__ static __forceinline__ int vcol(int r, int c) {
    return D == 128 ? (c + 4 * r) & 15 : (c + 4 * (r >> 1)) & 7;
  }
  // logical chunk stored at column col of row r (the inverses)
  __device__ static __forceinline__ int kchunk(int r, int col) {
    return D == 128 ? (col - r) & 15 : (col - (r >> 1)) & 7;
  }
  __device__ static __forceinline__ int vchunk(int r, int col) {
    return D == 128 ? (col - 4 * r) & 15 : (col - 4 * (r >> 1)) & 7;
  }
  int koff[D / 16], voff[D / 32];
  __device__ __forceinline__ explicit SwzLayout(int lane) {
    const int l32 = lane & 31, hi = lane >> 5, ig = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) koff[k] = l32 * ROW + kcol(l32, 2 * k + hi) * 16;
    const int r = 4 * hi + (ig >> 2);  // the row inside the 16-key step; 16 kk adds whole rotations
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int byte = (32 * dt + 16 * g16 + 4 * (ig & 3)) * 2;
      voff[dt] = r * ROW + vcol(r, byte / 16) * 16 + byte % 16;
    }
  }
  __device__ __forceinline__ int kfrag(int i) const { return koff[i >> 1] + (i & 1) * 32 * ROW; }
  __device__ __forceinline__ int vfrag(int kk, int dt) const { return 16 * kk * ROW + voff[dt]; }
};

// The three parts of one 64-key tile for one wave. qk_tile: S^T = K . Q^T from the K tile at kb.
// The K fragments (k step ks, 32-key half m) are read in MFMA order through a ring of kQkInFlight
// registers, and the schedule is pinned (kQkInFlight reads, then one MFMA per read, then the
// last MFMAs): left alone, the compiler reuses one register quad and every MFMA waits for its
// own LDS read (3 % slower at 4 reads in flight).
constexpr int kQkInFlight = 4;
template <int D, typename L>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const bf16x8 (&qf)[D / 16], const unsigned char* kb,
                                        const L& lay) {
  constexpr int NF = 2 * (D / 16);  // fragments i = 2 ks + m
  constexpr int PF = kQkInFlight;
  auto frag = [&](int i) { return *reinterpret_cast<const bf16x8*>(kb + lay.kfrag(i)); };
  s[0] = f32x16{};
  s[1] = f32x16{};
  bf16x8 kf[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) kf[i] = frag(i);
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    s[i & 1] = mfma32x32x16(kf[i % PF], qf[i >> 1], s[i & 1]);
    if (i + PF < NF) kf[i % PF] = frag(i + PF);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NF - PF; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
}

// Keys at or past N get a score of -inf; only called for the tile that holds the last token,
// so the number of valid keys in it, N - key0, is below 64.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int64_t key0, int64_t N, int lane) {
  const int valid = (int)(N - key0) - 4 * (lane >> 5);  // valid keys counted from this lane's first row
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * m + 8 * (r / 4) + (r % 4) >= valid) s[m][r] = -INFINITY;
}

// Online softmax of one score tile in the log2 domain (sc = log2(e)/sqrt(D)), in two parts.
// softmax_max moves the running max and rescales O and the row sum. The running max only moves
// when the tile max exceeds it by more than 8 (a factor 256): until then exp2 values stay <= 256,
// which fp32 sums and bf16 P hold exactly enough, and the rescale (a wave-uniform branch) is
// skipped.
template <int D>
__device__ __forceinline__ void softmax_max(WaveRows<D>& w, const f32x16 (&s)[2], float sc) {
  // tile max as a shallow tree (independent partial maxima) rather than one long chain
  float mp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mp[j] = fmaxf(s[0][4 * j], s[0][4 * j + 1]);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (m > 0 || (r % 4) >= 2) mp[r / 4] = fmaxf(mp[r / 4], s[m][r]);
  float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
  mx = pair_max(mx) * sc;
  if (__any(mx > w.m_run + 8.0f)) {
    const float m_new = fmaxf(w.m_run, mx);
    const float alpha = fast_exp2(w.m_run - m_new);
    w.m_run = m_new;
#pragma unroll
    for (int j = 0; j < 4; ++j) w.l_part[j] *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.o[dt][r] *= alpha;
  }
}

// softmax_exp: P^T = exp2(s*sc - m_run) as bf16 (pk, 8 values per 16-key step: step kk covers
// s[kk/2] regs 8*(kk%2) .. +7). The row sum of the bf16-rounded P that P.V uses is accumulated
// with packed dot products against (1, 1) straight into the wave's four running per-lane
// chains, which are added up only in the epilogue.
__device__ __forceinline__ void softmax_exp(const f32x16 (&s)[2], u32x4 (&pk)[4], float m_run, float sc,
                                                float (&lp)[4]) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(s[m][r], sc, -m_run));
      const float p1 = fast_exp2(fmaf(s[m][r + 1], sc, -m_run));
      const uint32_t pp = pack_bf16x2(p0, p1);
      pk[2 * m + r / 8][(r % 8) / 2] = pp;
      lp[(r / 2) % 4] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnes2, lp[(r / 2) % 4], false);
    }
  }
}

// O^T += V^T . P^T with V^T read from the row-major V tile at vb through the LDS transpose read;
// the key order inside each 16-key step matches the registers that hold P^T.
template <int D, typename L>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const u32x4 (&pk)[4], const unsigned char* vb,
                                        const L& lay) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[kk]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const unsigned char* p1 = vb + lay.vfrag(kk, dt);
      const i16x4 lo = lds_read_tr16(p1);
      const i16x4 hi4 = lds_read_tr16(p1 + L::V8);
      typedef __attribute__((ext_vector_type(8))) short i16x8;
      const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pb, o[dt]);
    }
  }
}

// One K/V tile of 64 keys (K rows at kb, V rows at vb in LDS; first key key0) applied to the
// wave's rows: S^T = K . Q^T, online softmax, O^T += V^T . P^T. `partial` (wave-uniform) marks
// the tile that holds the last token when N is not a multiple of 64.
template <int D, int BN, typename L>
__device__ __forceinline__ void rows_tile(WaveRows<D>& w, const unsigned char* kb, const unsigned char* vb,
                                          int64_t key0, int64_t N, bool partial, int lane, float sc, const L& lay) {
  static_assert(BN == kBN, "64-key tiles");
  f32x16 s[2];
  qk_tile<D>(s, w.qf, kb, lay);
  if (partial) mask_tile(s, key0, N, lane);
  softmax_max(w, s, sc);
  u32x4 pk[4];
  softmax_exp(s, pk, w.m_run, sc, w.l_part);
  pv_tile<D>(w.o, pk, vb, lay);
}

// Epilogue: combine the two lane-partial sums, normalise and store query row my_q if it is
// inside the sequence (out: the output tensor at the (batch, head) base; lse_row: the LSE row of
// the (batch, head), or null). A row that saw no key (an empty kept set) is written as zeros
// with LSE -inf.
template <int D>
__device__ __forceinline__ void rows_end(const WaveRows<D>& w, uint16_t* out, float* lse_row, int64_t my_q,
                                         int64_t N, int64_t row_stride, bool empty, int hi) {
  constexpr int DT = D / 32;
  const float l_tot = pair_sum((w.l_part[0] + w.l_part[1]) + (w.l_part[2] + w.l_part[3]));
  const float inv = empty ? 0.f : 1.0f / l_tot;
  if (my_q >= N) return;
  uint16_t* op = out + my_q * row_stride;
  float* lse_p = lse_row != nullptr ? lse_row + my_q : nullptr;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hi;
      u32x2 v;
      v[0] = pack_bf16x2(w.o[dt][4 * g + 0] * inv, w.o[dt][4 * g + 1] * inv);
      v[1] = pack_bf16x2(w.o[dt][4 * g + 2] * inv, w.o[dt][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(op + d) = v;
    }
  if (lse_p != nullptr && hi == 0)
    *lse_p = empty ? -INFINITY : (w.m_run + __log2f(l_tot)) * 0.6931471805599453f;
}

// Direct global -> LDS staging of one K/V tile into the SwzLayout (gfx950 global_load_lds_dwordx4:
// no staging registers, no LDS write instructions). A wave instruction writes 64 lanes x 16 bytes
// to consecutive LDS addresses, so LDS slot p = 64 (J w + j) + lane of wave w's instruction j is
// row p / CPR, column p % CPR of the tile, and the lane fetches the logical chunk that the
// rotation puts at that column. Rows past the end of the sequence are clamped to the last token,
// only in the tile that holds it. The loads are counted by vmcnt: a wave waits for its own
// (wait_dma) before the barrier that hands the tile to the other waves.
template <int D, int NT>
struct TileDma {
  using L = SwzLayout<D>;
  static constexpr int WAVES = NT / 64;
  static constexpr int J = L::CPR / WAVES;  // instructions per wave and tensor
  static_assert(L::CPR % WAVES == 0, "the tile's 1 KB slices must split evenly over the waves");
  int krow[J], koff[J], voff[J];
  int lds0;  // byte offset of the wave's first slice (wave-uniform)

  __device__ __forceinline__ void init(int tid, int64_t row_stride) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    lds0 = wave * J * 1024;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int p = 64 * (J * wave + j) + lane;
      const int r = p / L::CPR, col = p % L::CPR;
      krow[j] = r;
      koff[j] = r * (int)row_stride + 8 * L::kchunk(r, col);
      voff[j] = r * (int)row_stride + 8 * L::vchunk(r, col);
    }
  }
  // buf: LDS byte address of the tile buffer (wave-uniform)
  __device__ __forceinline__ void fetch(const uint16_t* k, const uint16_t* v, int64_t base, int64_t key0,
                                        int64_t N, int64_t row_stride, uint32_t buf) const {
    const int64_t tile = base + key0 * row_stride;
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(buf + lds0);
    if (key0 + kBN <= N) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        lds_dma16(k + tile + koff[j], l0 + 1024 * j);
        lds_dma16(v + tile + voff[j], l0 + L::K_BYTES + 1024 * j);
      }
    } else {
      const int last = (int)(N - 1 - key0);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t adj = krow[j] < last ? 0 : (int64_t)(last - krow[j]) * row_stride;
        lds_dma16(k + tile + koff[j] + adj, l0 + 1024 * j);
        lds_dma16(v + tile + voff[j] + adj, l0 + L::K_BYTES + 1024 * j);
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
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int64_t N = a.n_tokens;
  const int64_t qtile = blockIdx.x;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t row_stride = (int64_t)a.heads * D;  // elements between consecutive tokens
  const int64_t base = ((int64_t)b * N) * row_stride + (int64_t)head * D;

  const int64_t my_q = qtile * (WAVES * 32) + wave * 32 + l32;
  const int64_t my_q_c = my_q < N ? my_q : N - 1;
  WaveRows<D> w;
  rows_begin(w, a.q + base + my_q_c * row_stride + 8 * hi);

  const int n_tiles = (int)((N + kBN - 1) / kBN);
  const int last_partial = N % kBN ? n_tiles - 1 : -1;  // the tile to mask, if any
  TileDma<D, NT> dma;
  dma.init(tid, row_stride);
  const L lay(lane);
  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)

  // LDS byte address of the tile buffers
  const uint32_t smem_lds = lds_address(smem);
  wait_own_loads();  // the Q fragments
  dma.fetch(a.k, a.v, base, 0, N, row_stride, smem_lds);
  wait_dma();
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles)
      dma.fetch(a.k, a.v, base, (int64_t)(t + 1) * kBN, N, row_stride, smem_lds + (buf ^ 1) * L::BUF_BYTES);
    const unsigned char* kb = smem + buf * L::BUF_BYTES;
    rows_tile<D, kBN>(w, kb, kb + L::K_BYTES, (int64_t)t * kBN, N, t == last_partial, lane, sc, lay);
    wait_dma();
    __syncthreads();
  }
  rows_end(w, a.out + base, a.lse != nullptr ? a.lse + ((int64_t)b * a.heads + head) * N : nullptr, my_q, N,
           row_stride, false, hi);
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
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int64_t N = a.n_tokens;
  const int64_t nb = a.n_blocks;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t row_stride = (int64_t)a.heads * D;
  const int64_t base = ((int64_t)b * N) * row_stride + (int64_t)head * D;

  const int gblk = __builtin_amdgcn_readfirstlane((wave & 1) + 2 * (wave >> 2));  // this wave's block in the group
  const int half = (wave >> 1) & 1;               // and its 32-query half
  const int64_t row0 = ((int64_t)b * a.heads + head) * nb;
  const int64_t qb = group_block<G>(blockIdx.x, gblk, a.group_stride, nb);
  const int64_t my_q = (qb < 0 ? 0 : qb) * kBN + half * 32 + l32;
  const int64_t my_q_c = my_q < N ? my_q : N - 1;

  // the kept list of each block of the group inside block_idx, in LDS; this wave's own length
  __shared__ int64_t s_range[2 * G];
  stash_group_ranges<G, CSR>(s_range, a.row_ptr, a.keep, row0, blockIdx.x, a.group_stride, nb);
  int64_t my_beg, my_end;
  kept_range<CSR>(a.row_ptr, a.keep, row0, qb, my_beg, my_end);
  const int64_t my_count = my_end - my_beg;

  WaveRows<D> w;
  rows_begin(w, a.q + base + my_q_c * row_stride + 8 * hi);
  TileDma<D, NT> dma;
  dma.init(tid, row_stride);
  const L lay(lane);
  const uint32_t smem_lds = lds_address(smem);
  const float sc = 1.4426950408889634f / sqrtf((float)D);
  const uint32_t my_bit = 1u << gblk;

  for (int64_t j0 = 0; j0 < nb; j0 += KW) {
    const int nw = (int)(nb - j0 < KW ? nb - j0 : KW);
    const int nu = build_union_window<G, KW, NT>(ulist, s_wave_tot, &s_nu, a.block_idx, s_range, j0, nw);
    if (nu == 0) continue;

    auto key0_of = [&](int t) -> int64_t { return (j0 + (int64_t)(ulist[t] >> 8)) * kBN; };
    wait_own_loads();  // Q fragments, kept ranges and block lists
    dma.fetch(a.k, a.v, base, key0_of(0), N, row_stride, smem_lds);
    wait_dma();
    __syncthreads();
    for (int t = 0; t < nu; ++t) {
      const int buf = t & 1;
      const uint32_t e = __builtin_amdgcn_readfirstlane(ulist[t]);  // uniform: scalar tests and loads
      if (t + 1 < nu) dma.fetch(a.k, a.v, base, key0_of(t + 1), N, row_stride, smem_lds + (buf ^ 1) * L::BUF_BYTES);
      if (e & my_bit) {
        const unsigned char* kb = smem + buf * L::BUF_BYTES;
        // a 64-bit compare here: the 32-bit block-index compare of the dense kernel measured 8 %
        // slower in this kernel
        const int64_t key0 = (j0 + (int64_t)(e >> 8)) * kBN;
        rows_tile<D, kBN>(w, kb, kb + L::K_BYTES, key0, N, key0 + kBN > N, lane, sc, lay);
      }
      wait_dma();
      __syncthreads();
    }
  }
  if (qb >= 0)
    rows_end(w, a.out + base, a.lse != nullptr ? a.lse + ((int64_t)b * a.heads + head) * N : nullptr, my_q, N,
             row_stride, my_count <= 0, hi);
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
