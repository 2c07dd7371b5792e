// FP8 (OCP e4m3) dense and block-sparse attention forward for gfx950.
//
// Sources: "智東西…H3 Lightning" (hao.cnyes.com), section "02. 從50步壓到9步三層最佳化實現12倍提速"
// (SageAttention2 speeds up attention) and "VDN-MiniMax-H3：基于MiniMax H3的视频生成加速开源项目"
// (aipuzi.cn), sections "二、功能特色" / "三、技术细节" (FP8 quantised inference); the block-sparse
// form follows "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section "6.24 倍里，真正有
// 损的部分大约是三倍".
//
// Inputs are the e4m3 tensors of launch_fp8_quantize. Each wave owns 32 queries and computes
//   S^T = K8 . Q8^T with v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulation),
// scaled by q_scale * k_scale * log2(e)/sqrt(D). The running max m is kept as an integer (the
// ceiling of the row max in log2 units); when it moves, O and the row sum are rescaled by an exact
// power of two. The probabilities 2^(8 + x - m) (at most 256) are rounded to e4m3 in the score
// registers and used directly as the B operand of
//   O^T += V8^T . P^T   (A operand: a V^T tile whose keys are stored in the order the score
//                        registers hold them) and
//   L   += 1 . P^T      (a ones A operand: every row of L is the row sum of the rounded P).
// Per lane, an MFMA operand is 32 bytes; the probe-checked rule of this instruction is that byte
// j of lane half h in A multiplies byte j of lane half h in B, so the k index order is free as
// long as both operands agree. K tiles (64 x D bytes) and V^T tiles (D x 64 bytes) are fetched
// into registers one tile ahead and double-buffered in LDS, one barrier per tile.
#include "device_util.h"
#include "kernels.h"
#include "launch_util.h"
#include "sparse_union.h"

namespace h3attn {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ f32x16 mfma_e4m3(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats 0/0: e4m3 x e4m3; scale operands unused
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_read_32b(const unsigned char* p) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int D>
struct Fp8Tile {
  static constexpr int KS = D + 16;   // K row stride in LDS (bytes): conflict-free 16-byte reads
  static constexpr int VS = 64 + 16;  // V^T row stride in LDS (bytes)
  static constexpr int K_BYTES = 64 * KS;
  static constexpr int V_BYTES = D * VS;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_CHUNKS = 64 * D / 16;  // 16-byte chunks per tile
  static constexpr int V_CHUNKS = D * 64 / 16;
};

// Global -> register staging of one K tile (rows key0 .. key0+63 of k8, clamped to the last
// token) and one V^T tile (columns key0 .. key0+63 of v8t, zero past N), then -> LDS. A thread's
// chunks sit at fixed offsets from the tile's first K row and first V^T column, so the per-lane
// offsets are computed once (init) and moving to the next tile only moves wave-uniform bases.
template <int D, int NT>
struct Fp8Stage {
  using T = Fp8Tile<D>;
  static constexpr int LK = (T::K_CHUNKS + NT - 1) / NT;
  static constexpr int LV = (T::V_CHUNKS + NT - 1) / NT;
  u32x4 kst[LK], vst[LV];
  int krow[LK];
  uint32_t koff[LK];       // byte offset from the tile's first K row: below 2^31 (rows < 64, heads <= 65535)
  const uint8_t* vp[LV];   // the lane's V^T chunks for key 0 (row (ci >> 2), bytes 16 (ci & 3))
  int rs;                  // bytes between consecutive tokens of k8

  __device__ __forceinline__ void init(const uint8_t* v8t, int64_t vbase, int64_t row_stride, int64_t np, int tid) {
    rs = (int)row_stride;
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int ci = tid + i * NT;
      krow[i] = ci / (D / 16);
      koff[i] = (uint32_t)(krow[i] * rs + (ci % (D / 16)) * 16);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int ci = tid + i * NT;
      vp[i] = v8t + vbase + (int64_t)(ci >> 2) * np + (ci & 3) * 16;
    }
  }
  // ktile: the tile's first K row (wave-uniform); key0 its first key; whole: all 64 keys lie
  // inside the sequence
  __device__ __forceinline__ void fetch(const uint8_t* ktile, int64_t key0, bool whole, int64_t N, int tid) {
    if (whole) {
#pragma unroll
      for (int i = 0; i < LK; ++i)
        if (T::K_CHUNKS % NT == 0 || tid + i * NT < T::K_CHUNKS)
          kst[i] = *reinterpret_cast<const u32x4*>(ktile + koff[i]);
    } else {
      const int last = (int)(N - 1 - key0);
#pragma unroll
      for (int i = 0; i < LK; ++i)
        if (T::K_CHUNKS % NT == 0 || tid + i * NT < T::K_CHUNKS) {
          const int adj = krow[i] < last ? 0 : (last - krow[i]) * rs;  // row min(r, last)
          kst[i] = *reinterpret_cast<const u32x4*>(ktile + (uint32_t)((int)koff[i] + adj));
        }
    }
#pragma unroll
    for (int i = 0; i < LV; ++i)
      if (T::V_CHUNKS % NT == 0 || tid + i * NT < T::V_CHUNKS)
        vst[i] = *reinterpret_cast<const u32x4*>(vp[i] + key0);
  }
  // The same tile addressed from the key index (the block-sparse kernel, whose key blocks come
  // from the LDS union list): there this form measured 2.5 % faster than the fixed offsets above
  // (78.2 against 80.2 ms at the 5 s workload; 78.8 ms with vector-held bases).
  __device__ __forceinline__ void fetch_keys(const uint8_t* k8, const uint8_t* v8t, int64_t kbase, int64_t vbase,
                                             int64_t key0, int64_t N, int64_t rs, int64_t np, int tid) {
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int ci = tid + i * NT;
      if (T::K_CHUNKS % NT == 0 || ci < T::K_CHUNKS) {
        int64_t key = key0 + ci / (D / 16);
        key = key < N ? key : N - 1;
        kst[i] = *reinterpret_cast<const u32x4*>(k8 + kbase + key * rs + (ci % (D / 16)) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int ci = tid + i * NT;
      if (T::V_CHUNKS % NT == 0 || ci < T::V_CHUNKS)
        vst[i] = *reinterpret_cast<const u32x4*>(v8t + vbase + (int64_t)(ci >> 2) * np + key0 + (ci & 3) * 16);
    }
  }
  __device__ __forceinline__ void stash(unsigned char* kb, int tid) const {
    unsigned char* vb = kb + T::K_BYTES;
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int ci = tid + i * NT;
      if (T::K_CHUNKS % NT == 0 || ci < T::K_CHUNKS)
        *reinterpret_cast<u32x4*>(kb + (ci / (D / 16)) * T::KS + (ci % (D / 16)) * 16) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int ci = tid + i * NT;
      if (T::V_CHUNKS % NT == 0 || ci < T::V_CHUNKS)
        *reinterpret_cast<u32x4*>(vb + (ci >> 2) * T::VS + (ci & 3) * 16) = vst[i];
    }
  }
};

// One wave's 32 query rows: Q8^T fragments, O^T and row-sum accumulators, running max.
template <int D>
struct Fp8Rows {
  i32x8 qf[D / 64];
  f32x16 o[D / 32];
  f32x16 lsum;   // 1 . P^T: every register holds the row sum of the lane's query
  float m_run;   // integer-valued running max (log2 units), shared by lanes l and l^32
  float cq;      // query block scale * log2(e)/sqrt(D)
  i32x8 ones;    // e4m3 ones (the row-sum operand), built once
};

template <int D>
__device__ __forceinline__ void fp8_rows_begin(Fp8Rows<D>& w, const uint8_t* qrow, int hi, float cq) {
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hi);
    const u32x4 h4 = *reinterpret_cast<const u32x4*>(qrow + 64 * ks + 32 * hi + 16);
    w.qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)h4[0], (int)h4[1], (int)h4[2], (int)h4[3]};
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) w.o[dt] = f32x16{};
  w.lsum = f32x16{};
  w.m_run = -INFINITY;
  int one4 = 0x38383838;          // four e4m3 ones
  asm volatile("" : "+v"(one4));  // opaque: kept in registers, not rebuilt from a constant every tile
  w.ones = i32x8{one4, one4, one4, one4, one4, one4, one4, one4};
  w.cq = cq;
}

// QK half of one 64-key tile: S^T = K8 . Q8^T from the K tile at kb. Every K fragment is read
// before the first MFMA (left alone, the compiler issues each read just before its MFMA and
// waits for it).
template <int D>
__device__ __forceinline__ void fp8_qk(const Fp8Rows<D>& w, const unsigned char* kb, int lane, f32x16 (&s)[2]) {
  using T = Fp8Tile<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  i32x8 kf[2][D / 64];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) kf[m][ks] = lds_read_32b(kb + (32 * m + l32) * T::KS + 64 * ks + 32 * hi);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    s[m] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) s[m] = mfma_e4m3(kf[m][ks], w.qf[ks], s[m]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4 * (D / 64), 0);  // K reads (two per fragment)
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 64), 0);  // QK MFMAs
}

// Softmax and P.V half of the tile whose scores are s (V^T rows at vb; first key key0; ck its
// key-block scale). The V^T fragments are read first, so they arrive during the softmax.
template <int D>
__device__ __forceinline__ void fp8_soft_pv(Fp8Rows<D>& w, f32x16 (&s)[2], const unsigned char* vb, int64_t key0,
                                            int64_t N, bool partial, int lane, float ck) {
  using T = Fp8Tile<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  i32x8 vf[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vf[dt] = lds_read_32b(vb + (32 * dt + l32) * T::VS + 32 * hi);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);  // V reads
  if (partial) {  // keys past the end of the sequence (the tile that holds the last token)
    const int valid = (int)(N - key0) - 4 * hi;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * m + 8 * (r / 4) + (r % 4) >= valid) s[m][r] = -INFINITY;
  }
  const float c = w.cq * ck;
  float mp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mp[j] = fmaxf(s[0][4 * j], s[0][4 * j + 1]);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (m > 0 || (r % 4) >= 2) mp[r / 4] = fmaxf(mp[r / 4], s[m][r]);
  const float t = ceilf(pair_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]))) * c);
  if (__any(t > w.m_run)) {  // the integer max moves: rescale by an exact power of two
    const float m_new = fmaxf(w.m_run, t);
    const float alpha = w.m_run == -INFINITY ? 0.f : ldexpf(1.0f, (int)(w.m_run - m_new));
    w.m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.o[dt][r] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) w.lsum[r] *= alpha;
  }
  // P^T = e4m3(2^(8 + x - m)), byte j = 16m + r of the lane's 32-byte operand
  const float off = 8.0f - w.m_run;
  int pk[8];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      // both halves of the word are written, so the first conversion's "old" operand is any
      // dying register (no zeroing move)
      const float e1 = fast_exp2(fmaf(s[m][r + 1], c, off));
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(s[m][r], c, off)), e1, __builtin_bit_cast(int, e1), false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(fmaf(s[m][r + 2], c, off)), fast_exp2(fmaf(s[m][r + 3], c, off)), v, true);
      pk[4 * m + r / 4] = v;
    }
  const i32x8 pb = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) w.o[dt] = mfma_e4m3(vf[dt], pb, w.o[dt]);
  w.lsum = mfma_e4m3(w.ones, pb, w.lsum);
}

// one whole 64-key tile (K rows at kb, V^T rows at vb in LDS; first key key0; ck its scale;
// partial: the tile holds the last token and keys past it)
template <int D>
__device__ __forceinline__ void fp8_rows_tile(Fp8Rows<D>& w, const unsigned char* kb, const unsigned char* vb,
                                              int64_t key0, int64_t N, bool partial, int lane, float ck) {
  f32x16 s[2];
  fp8_qk(w, kb, lane, s);
  fp8_soft_pv(w, s, vb, key0, N, partial, lane, ck);
}

// normalise by the row sum, apply the channel scales, store the row of query my_q (if < N)
template <int D>
__device__ __forceinline__ void fp8_rows_end(const Fp8Rows<D>& w, uint16_t* out, float* lse_row, const float* vscale,
                                             int64_t my_q, int64_t N, int64_t rs, int hi) {
  const float l = w.lsum[0];
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.0f / l;
  if (my_q >= N) return;
  uint16_t* op = out + my_q * rs;
  f32x4 vsc[D / 32][4];  // all channel scales first: the stores below may alias them for the compiler
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) vsc[dt][g] = *reinterpret_cast<const f32x4*>(vscale + 32 * dt + 8 * g + 4 * hi);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hi;
      const f32x4 vs = vsc[dt][g];
      u32x2 v;
      v[0] = pack_bf16x2(w.o[dt][4 * g + 0] * vs[0] * inv, w.o[dt][4 * g + 1] * vs[1] * inv);
      v[1] = pack_bf16x2(w.o[dt][4 * g + 2] * vs[2] * inv, w.o[dt][4 * g + 3] * vs[3] * inv);
      *reinterpret_cast<u32x2*>(op + d) = v;
    }
  if (lse_row != nullptr && hi == 0)
    lse_row[my_q] = empty ? -INFINITY : (w.m_run - 8.0f + __log2f(l)) * 0.6931471805599453f;
}

constexpr float kLog2e = 1.4426950408889634f;

// Dense: 8 waves (256 queries) per workgroup, two waves per SIMD.
template <int D>
__global__ __launch_bounds__(512, 2) void attn_fp8_dense_kernel(Fp8AttnArgs a) {
  using T = Fp8Tile<D>;
  constexpr int NT = 512;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int64_t N = a.n_tokens, nb = a.n_blocks;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.heads + head;
  const int64_t rs = (int64_t)a.heads * D;          // bytes (q8, k8) or elements (out) per token
  const int64_t np = nb * 64;
  const int64_t kbase = ((int64_t)b * N) * rs + (int64_t)head * D;
  const int64_t vbase = bh * D * np;
  const int64_t q0 = (int64_t)blockIdx.x * 256 + wave * 32;
  const int64_t my_q = q0 + l32, my_q_c = my_q < N ? my_q : N - 1;
  const int64_t qblk = (q0 < N ? q0 : N - 1) / 64;

  Fp8Rows<D> w;
  fp8_rows_begin(w, a.q8 + kbase + my_q_c * rs, hi, a.q_scale[bh * nb + qblk] * (kLog2e / sqrtf((float)D)));
  Fp8Stage<D, NT> st;
  st.init(a.v8t, vbase, rs, np, tid);
  const uint8_t* k0p = a.k8 + kbase;  // first K row of the (batch, head)
  const int64_t tile_bytes = 64 * rs;
  // a tile's key scale is staged in LDS with the tile (see the sparse kernel below)
  __shared__ float s_ks[2];
  const int n_full = (int)(N / 64);                  // tiles that lie inside the sequence
  const int last_partial = N % 64 ? (int)nb - 1 : -1;  // the tile to mask, if any
  float ks = a.k_scale[bh * nb];
  st.fetch(k0p, 0, 0 < n_full, N, tid);
  st.stash(smem, tid);
  if (tid == 0) s_ks[0] = ks;
  __syncthreads();
  for (int t = 0; t < nb; ++t) {
    const int buf = t & 1;
    if (t + 1 < nb) {
      ks = a.k_scale[bh * nb + t + 1];
      st.fetch(k0p + (t + 1) * tile_bytes, (int64_t)(t + 1) * 64, t + 1 < n_full, N, tid);
    }
    const unsigned char* kb = smem + buf * T::BUF_BYTES;
    fp8_rows_tile<D>(w, kb, kb + T::K_BYTES, (int64_t)t * 64, N, t == last_partial, lane, s_ks[buf]);
    if (t + 1 < nb) {
      st.stash(smem + (buf ^ 1) * T::BUF_BYTES, tid);
      if (tid == 0) s_ks[buf ^ 1] = ks;
    }
    __syncthreads();
  }
  fp8_rows_end(w, a.out + ((int64_t)b * N) * rs + (int64_t)head * D,
               a.lse != nullptr ? a.lse + bh * N : nullptr, a.v_scale + bh * D, my_q, N, rs, hi);
}

// Block-sparse over groups of 4 query blocks (2 waves each; blocks i, i+S, i+2S, i+3S of the
// group stride S), walking the union of their kept key blocks (see sparse_union.h); a wave runs a
// union tile only if its block keeps it.
template <int D, int KW>
__global__ __launch_bounds__(512, 2) void attn_fp8_sparse_kernel(Fp8AttnArgs a) {
  using T = Fp8Tile<D>;
  constexpr int G = 4, NT = 512;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* ulist = reinterpret_cast<uint32_t*>(smem + 2 * T::BUF_BYTES);
  __shared__ int s_wave_tot[NT / 64];
  __shared__ int s_nu;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int64_t N = a.n_tokens, nb = a.n_blocks;
  const int head = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.heads + head;
  const int64_t rs = (int64_t)a.heads * D;
  const int64_t np = nb * 64;
  const int64_t kbase = ((int64_t)b * N) * rs + (int64_t)head * D;
  const int64_t vbase = bh * D * np;
  const int gblk = __builtin_amdgcn_readfirstlane((wave & 1) + 2 * (wave >> 2));  // block in the group; SIMD-mates differ
  const int half = (wave >> 1) & 1;
  const int64_t qb = group_block<G>(blockIdx.x, gblk, a.group_stride, nb);
  const int64_t my_q = (qb < 0 ? 0 : qb) * 64 + half * 32 + l32, my_q_c = my_q < N ? my_q : N - 1;

  // the kept list of each block of the group inside block_idx, in LDS
  __shared__ int64_t s_range[2 * G];
  __shared__ float s_ks[2];  // key scale of the tile in each buffer
  stash_group_ranges<G, false>(s_range, nullptr, a.keep, bh * nb, blockIdx.x, a.group_stride, nb);

  Fp8Rows<D> w;
  fp8_rows_begin(w, a.q8 + kbase + my_q_c * rs, hi,
                 a.q_scale[bh * nb + (qb < 0 ? 0 : qb)] * (kLog2e / sqrtf((float)D)));
  Fp8Stage<D, NT> st;
  const uint32_t my_bit = 1u << gblk;
  for (int64_t j0 = 0; j0 < nb; j0 += KW) {
    const int nw = (int)(nb - j0 < KW ? nb - j0 : KW);
    const int nu = build_union_window<G, KW, NT>(ulist, s_wave_tot, &s_nu, a.block_idx, s_range, j0, nw);
    if (nu == 0) continue;
    auto kblk_of = [&](int t) -> int64_t { return j0 + (int64_t)(ulist[t] >> 8); };
    // a tile's key scale is staged in LDS with the tile, so the tile's compute never waits on a
    // global load (vmcnt counts in issue order: it would also wait for the next tile's prefetch)
    float ks = a.k_scale[bh * nb + kblk_of(0)];
    st.fetch_keys(a.k8, a.v8t, kbase, vbase, kblk_of(0) * 64, N, rs, np, tid);
    st.stash(smem, tid);
    if (tid == 0) s_ks[0] = ks;
    __syncthreads();
    for (int t = 0; t < nu; ++t) {
      const int buf = t & 1;
      const uint32_t e = __builtin_amdgcn_readfirstlane(ulist[t]);  // uniform: scalar tests
      if (t + 1 < nu) {
        const int64_t next = kblk_of(t + 1);
        ks = a.k_scale[bh * nb + next];
        st.fetch_keys(a.k8, a.v8t, kbase, vbase, next * 64, N, rs, np, tid);
      }
      if (e & my_bit) {
        const unsigned char* kb = smem + buf * T::BUF_BYTES;
        const int64_t key0 = (j0 + (int64_t)(e >> 8)) * 64;
        fp8_rows_tile<D>(w, kb, kb + T::K_BYTES, key0, N, key0 + 64 > N, lane, s_ks[buf]);
      }
      if (t + 1 < nu) {
        st.stash(smem + (buf ^ 1) * T::BUF_BYTES, tid);
        if (tid == 0) s_ks[buf ^ 1] = ks;
      }
      __syncthreads();
    }
  }
  if (qb >= 0)
    fp8_rows_end(w, a.out + ((int64_t)b * N) * rs + (int64_t)head * D,
                 a.lse != nullptr ? a.lse + bh * N : nullptr, a.v_scale + bh * D, my_q, N, rs, hi);
}

template <int D>
void launch_dense(const Fp8AttnArgs& a, hipStream_t stream) {
  const size_t lds = 2 * Fp8Tile<D>::BUF_BYTES;
  allow_dynamic_lds(reinterpret_cast<const void*>(attn_fp8_dense_kernel<D>), (int)lds);
  hipLaunchKernelGGL(attn_fp8_dense_kernel<D>, dim3((unsigned)((a.n_tokens + 255) / 256), (unsigned)a.heads, (unsigned)a.batch),
                     dim3(512), lds, stream, a);
}

template <int D>
void launch_sparse(const Fp8AttnArgs& a, hipStream_t stream) {
  constexpr int KW = 4096;
  const size_t lds = 2 * Fp8Tile<D>::BUF_BYTES + (size_t)KW * 4;
  auto kern = attn_fp8_sparse_kernel<D, KW>;
  allow_dynamic_lds(reinterpret_cast<const void*>(kern), (int)lds);
  hipLaunchKernelGGL(kern, dim3((unsigned)n_groups<4>(a.n_blocks, a.group_stride), (unsigned)a.heads, (unsigned)a.batch),
                     dim3(512), lds, stream, a);
}

}  // namespace

void launch_fp8_dense_fwd(const Fp8AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_dense<128>(a, stream);
  else launch_dense<64>(a, stream);
}

void launch_fp8_block_sparse_fwd(const Fp8AttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_sparse<128>(a, stream);
  else launch_sparse<64>(a, stream);
}

}  // namespace h3attn
