// SubBlock key-block selection for gfx950: block pooling, block scores and the per-row selection,
// with the scores kept on chip.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section
// "6.24 倍里，真正有损的部分大约是三倍": queries and keys are cut into 64-token blocks, the key
// blocks that would contribute little are estimated and dropped, and the fraction dropped is
// the sparsity. The pages leave the estimator open; this library scores key block j for query
// block i by s_ij = mean(q over block i) . mean(k over block j) and keeps the keep highest per
// row, equal scores ranking the lower key index first, indices written in ascending order. The
// 1/sqrt(D) of the definition is a positive factor and does not change the order.
//
// Exactness. Block sums of bf16 values are exact in float64, so the float64 block means are the
// definition's means. Ranking by a float64 dot product of them would need the float64 matrix
// cores for every score (4.7e10 flop at the 5 s workload); instead every score is first bounded:
//   * each mean vector x is written as integers X = round(x * 2^-e) with |X| <= 2^22 (one power of
//     two e per block), each X split into three signed base-256 digits d2 d1 d0;
//   * the int8 matrix cores form, exactly in int32, the digit products of weight 2^32, 2^24 and
//     2^16 (six of the nine digit pairs); the rest, and the rounding of x to X, is bounded
//     rigorously per row (row_bound below);
//   * so every approximate score v_ij carries |v_ij - s_ij * scale_i| <= E_i.
// A row's keep-th largest v is bracketed by a histogram of its v values (one more pass of the
// same products when a bin holds too many); every entry above the bracket by more than 2 E_i is
// kept, every entry below it by more than 2 E_i dropped, and only the entries in between are
// decided on their float64 scores (a handful per row). The kept sets are therefore those of the
// float64 scores, the same as the float64 definition except where two float64 scores differ in
// their last bits. Rows that do not resolve this way (ties of many equal scores) go to a
// fallback kernel that computes the whole row's float64 scores and selects with an exact radix
// select.
//
// Kernels (top-k mode):
//  pool_kernel          one workgroup per (batch, head, block): fp64 means, their integer digits in
//                       the int8 MFMA operand order, exponent and norms.
//  key_stats_kernel     per (batch, head): largest key exponent and norms (for the bounds).
//  topk_select_kernel   per (batch, head, 32 query blocks): histogram pass(es), classification
//                       pass, resolution on float64 scores, ordered write of the kept indices.
//  fallback_kernel      rows routed there: float64 row in LDS, radix select.
// Threshold mode (keep j iff s_ij >= max_j s_ij - tau): threshold_count_kernel (exact row maximum
// and kept counts), row_ptr_scan_kernel, threshold_fill_kernel (the same decisions, written as CSR).
#include <type_traits>

#include "device_util.h"
#include "kernels.h"
#include "launch_util.h"
#include "norm_rope_math.h"

namespace h3attn {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

constexpr int kPoolThreads = 256;
constexpr int kRows = 32;                   // query blocks per selection workgroup (the MFMA's columns)
constexpr int kSelThreads = 256;            // 4 waves
constexpr int kWaves = kSelThreads / 64;
constexpr int kBins = 1024;                 // histogram bins per row and level
constexpr int kHistStride = kBins / 2 + 4;  // 32-bit words per row (two 16-bit counts each; word 512 is the
                                            // pad, 16-byte aligned rows)
constexpr int kCap = 160;                   // candidate slots per row
constexpr int kDigitShift = 21;             // |x| * 2^-e in [2^21, 2^22): |X| <= 2^22
constexpr int kZeroExp = -1000;             // exponent recorded for an all-zero mean vector
// |P1 * 2^8 + P0| per channel for the dropped digit pairs (d1 d0', d0 d1' and d0 d0', digits in
// [-128, 127]) plus the 1/4 of the rounding product term: 128*128*(2*256 + 1) + 1/4
constexpr double kDropPerChannel = 8404992.25;

__device__ __forceinline__ int64_t n_pad(int32_t nb) { return ((int64_t)nb + kRows - 1) / kRows * kRows; }

// ------------------------------------------------------------------------------------ pooling

// The end of a block's pooling, shared by pool_kernel and norm_rope_pool_kernel: from the thread's
// float64 sums acc of its 8 channels over the block's rows (all D/8 threads of the head present),
// the means, max |x|, sum |x| and sum x^2 over the head's channels (a fixed xor-shuffle tree), the
// digits, exponent and norms, written to the workspace.
template <int D>
__device__ __forceinline__ void pool_store(const SelectArgs& a, int tensor, int b, int head, int chunk, int j,
                                           int rows, const double (&acc)[8]) {
  constexpr int CH = D / 8;
  constexpr int KS = D / 32;
  const int64_t bh = (int64_t)b * a.heads + head;
  // a full block divides by 64 = 2^6: the product by 2^-6 is the same correctly rounded quotient
  const bool full = rows == 64;
  const double cnt = (double)rows;
  double m[8];
  double amax = 0.0, l1 = 0.0, l2 = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m[e] = full ? acc[e] * 0x1p-6 : acc[e] / cnt;
    amax = fmax(amax, fabs(m[e]));
    l1 += fabs(m[e]);
    l2 += m[e] * m[e];
  }
  {
    double* dst = (tensor == 0 ? a.q_mean : a.k_mean) + (bh * a.n_blocks + j) * D + chunk * 8;
#pragma unroll
    for (int e = 0; e < 8; e += 2) *reinterpret_cast<double2*>(dst + e) = double2{m[e], m[e + 1]};
  }
  // reduce over the CH lanes of the head (xor offsets below CH stay inside the group)
#pragma unroll
  for (int off = 1; off < CH; off <<= 1) {
    amax = fmax(amax, __shfl_xor(amax, off));
    l1 += __shfl_xor(l1, off);
    l2 += __shfl_xor(l2, off);
  }
  const int ex = amax > 0.0 ? ilogb(amax) - kDigitShift : 0;
  // digits: X = d0 + 256 d1 + 65536 d2, each digit in [-128, 127]; |X| <= 2^22 so |d2| <= 64
  uint32_t dig[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int x = (int)rint(ldexp(m[e], -ex));
    const int d0 = ((x & 255) ^ 128) - 128;
    const int x1 = (x - d0) >> 8;
    const int d1 = ((x1 & 255) ^ 128) - 128;
    const int d2 = (x1 - d1) >> 8;
    dig[0][e / 4] |= (uint32_t)(d0 & 255) << (8 * (e % 4));
    dig[1][e / 4] |= (uint32_t)(d1 & 255) << (8 * (e % 4));
    dig[2][e / 4] |= (uint32_t)(d2 & 255) << (8 * (e % 4));
  }
  // operand slot of this 8-channel chunk: k step t = chunk / 4, lane group g = (chunk % 4) / 2,
  // bytes 8 * (chunk % 2) of lane (j % 32) + 32 g in the 1 KB fragment of (chunk-of-32 j / 32, t, digit)
  const int t = chunk / 4, g = (chunk % 4) / 2, half = chunk % 2;
  const int64_t nchunks = n_pad(a.n_blocks) / kRows;
  int8_t* base = (tensor == 0 ? a.q_digits : a.k_digits);
#pragma unroll
  for (int L = 0; L < 3; ++L) {
    int8_t* p = base + (((bh * nchunks + j / kRows) * KS + t) * 3 + L) * 1024 + ((j % kRows) + 32 * g) * 16 + 8 * half;
    *reinterpret_cast<u32x2*>(p) = u32x2{dig[L][0], dig[L][1]};
  }
  if (chunk == 0) {
    const int64_t r = bh * n_pad(a.n_blocks) + j;
    (tensor == 0 ? a.q_exp : a.k_exp)[r] = amax > 0.0 ? ex : kZeroExp;
    // norms rounded up (with a margin for the float64 sums' own rounding): they only bound errors
    const float n1 = __double2float_ru(l1 * (1.0 + 0x1p-40));
    const float n2 = __double2float_ru(sqrt(l2) * (1.0 + 0x1p-40));
    *reinterpret_cast<float2*>((tensor == 0 ? a.q_norm : a.k_norm) + 2 * r) = float2{n1, n2};
  }
}

// One workgroup per (batch, tensor, block j, group of heads): thread t owns the 16-byte chunk t of
// the group's slice of every token row (kPoolThreads * 16 bytes of consecutive heads), so each
// wave reads 1 KB contiguous per row and the 64 rows stream in with 16 loads in flight per
// thread. Each thread sums its 8 channels over the block in float64 (exact whenever a channel's
// nonzero values in the block lie within a factor 2^39 of each other: 8-bit significands, 64
// terms, 53 bits; always so for data of these workloads' ranges), then the
// D / 8 threads of a head finish the block (pool_store). No LDS, no barriers.
template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(SelectArgs a) {
  constexpr int CH = D / 8;                 // 16-byte chunks per head row
  constexpr int HPW = kPoolThreads / CH;    // heads per workgroup
  constexpr int UNROLL = 16;                // rows in flight per thread
  const int tid = threadIdx.x;
  const int groups = (a.heads + HPW - 1) / HPW;
  const int hg = (int)(blockIdx.x % (unsigned)groups), j = (int)(blockIdx.x / (unsigned)groups);
  const int tensor = (int)(blockIdx.z & 1u), b = (int)(blockIdx.z >> 1);
  const int head = hg * HPW + tid / CH, chunk = tid % CH;
  if (head >= a.heads) return;  // whole heads drop out together (CH divides 64)
  const int64_t N = a.n_tokens;
  const int64_t row_stride = (int64_t)a.heads * D;
  const int64_t t0 = (int64_t)j * a.block_size;
  const int rows = (int)(t0 + a.block_size < N ? a.block_size : N - t0);
  const uint16_t* src = (tensor == 0 ? a.q : a.k) + ((int64_t)b * N + t0) * row_stride + (int64_t)head * D + chunk * 8;

  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // blocks are 64 tokens (the entry points accept no other size)
#pragma unroll 1
  for (int g = 0; g < 64; g += UNROLL) {
    u32x4 w[UNROLL];
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) {
      w[i] = u32x4{0u, 0u, 0u, 0u};
      if (g + i < rows) w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(g + i) * row_stride));
    }
#pragma unroll
    for (int i = 0; i < UNROLL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_lo(w[i][e]);
        acc[2 * e + 1] += (double)bf16_hi(w[i][e]);
      }
  }
  pool_store<D>(a, tensor, b, head, chunk, j, rows, acc);
}

// QK RMSNorm + 3D RoPE with the SubBlock pooling of its output in the same pass: the pooling's
// own read of q' and k' (4 B N heads D bytes) disappears. Same workgroups and lanes as
// pool_kernel; for every row of the block a thread loads its chunk of q (or k), normalises and
// rotates it exactly as the stand-alone kernel does (norm_rope_chunk, so the bits are the same),
// stores it, and adds the rounded bf16 outputs to its float64 sums. The rotation's cos and sin
// depend on the token and the channel pair, not on the head, so the workgroup computes them once
// for its 64 rows into LDS (64 x CH x 4 pairs), while the first 16 rows' loads are in flight
// (measured 2 % faster than computing the table first; 8 rows in flight or a two-group prefetch
// pipeline measured the same as the table first).
template <int D>
__global__ __launch_bounds__(kPoolThreads) void norm_rope_pool_kernel(NormRopeArgs nr, RopeTable tab, SelectArgs a) {
  constexpr int CH = D / 8;
  constexpr int HPW = kPoolThreads / CH;
  constexpr int UNROLL = 16;                // rows in flight per thread
  __shared__ float2 s_rot[64][CH][4];       // (cos, sin) per row, chunk and pair
  const int tid = threadIdx.x;
  const int groups = (a.heads + HPW - 1) / HPW;
  const int hg = (int)(blockIdx.x % (unsigned)groups), j = (int)(blockIdx.x / (unsigned)groups);
  const int tensor = (int)(blockIdx.z & 1u), b = (int)(blockIdx.z >> 1);
  const int head = hg * HPW + tid / CH, chunk = tid % CH;
  const int64_t N = a.n_tokens;
  const int64_t row_stride = (int64_t)a.heads * D;
  const int64_t t0 = (int64_t)j * a.block_size;
  const int rows = (int)(t0 + a.block_size < N ? a.block_size : N - t0);
  const bool live = head < a.heads;         // whole heads (CH lanes) are live or not
  const int64_t off = ((int64_t)b * N + t0) * row_stride + (int64_t)(live ? head : 0) * D + chunk * 8;
  const uint16_t* src = (tensor == 0 ? nr.q_in : nr.k_in) + off;
  uint16_t* dst = (tensor == 0 ? nr.q_out : nr.k_out) + off;

  u32x4 x[UNROLL];
  auto load_rows = [&](int g) {
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) {
      x[i] = u32x4{0u, 0u, 0u, 0u};
      if (live && g + i < rows)
        x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(g + i) * row_stride));
    }
  };
  load_rows(0);
  for (int i = tid; i < rows * CH * 4; i += kPoolThreads) {
    const int r = i / (CH * 4), cc = (i / 4) % CH, p = i % 4;
    int64_t pos[3];
    rope_position(t0 + r, nr.grid_h, nr.grid_w, pos);
    float cs, sn;
    rope_pair(pos, 4 * cc + p, tab, cs, sn);
    s_rot[r][cc][p] = float2{cs, sn};
  }
  __syncthreads();
  if (!live) return;

  float w[8];
  {
    const f32x4* wp = reinterpret_cast<const f32x4*>((tensor == 0 ? nr.q_weight : nr.k_weight) + 8 * chunk);
    const f32x4 w0 = wp[0], w1 = wp[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { w[e] = w0[e]; w[4 + e] = w1[e]; }
  }
  const float inv_d = 1.0f / (float)D;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
  for (int g = 0; g < 64; g += UNROLL) {
    if (g > 0) load_rows(g);
#pragma unroll
    for (int i = 0; i < UNROLL; ++i) {
      if (g + i >= rows) break;  // uniform across the workgroup
      float cs[4], sn[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float2 t = s_rot[g + i][chunk][p];
        cs[p] = t.x;
        sn[p] = t.y;
      }
      const u32x4 o = norm_rope_chunk<CH>(x[i], w, cs, sn, inv_d, nr.eps);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst + (int64_t)(g + i) * row_stride));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_lo(o[e]);
        acc[2 * e + 1] += (double)bf16_hi(o[e]);
      }
    }
  }
  pool_store<D>(a, tensor, b, head, chunk, j, rows, acc);
}

// Per (batch, head): the largest key exponent F and the largest key norms (for the bounds); then
// every key block's exponent is rewritten in place as its shift e_j - F, the power of two the
// score passes scale its products by. Also clears the count of fallback rows (this kernel runs
// after pooling and before any selection kernel).
__global__ __launch_bounds__(256) void key_stats_kernel(SelectArgs a) {
  __shared__ int s_e[4];
  __shared__ float s_1[4], s_2[4];
  __shared__ int s_f;
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int e = kZeroExp;
  float n1 = 0.f, n2 = 0.f;
  const int64_t r0 = bh * n_pad(a.n_blocks);
  for (int j = tid; j < a.n_blocks; j += 256) {
    e = max(e, a.k_exp[r0 + j]);
    const float2 nn = *reinterpret_cast<const float2*>(a.k_norm + 2 * (r0 + j));
    n1 = fmaxf(n1, nn.x);
    n2 = fmaxf(n2, nn.y);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    e = max(e, __shfl_xor(e, off));
    n1 = fmaxf(n1, __shfl_xor(n1, off));
    n2 = fmaxf(n2, __shfl_xor(n2, off));
  }
  if (lane == 0) { s_e[wave] = e; s_1[wave] = n1; s_2[wave] = n2; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) { e = max(e, s_e[w]); n1 = fmaxf(n1, s_1[w]); n2 = fmaxf(n2, s_2[w]); }
    a.key_stat[4 * bh + 0] = e;
    a.key_stat[4 * bh + 1] = __float_as_int(n1);
    a.key_stat[4 * bh + 2] = __float_as_int(n2);
    a.key_stat[4 * bh + 3] = 0;
    s_f = e;
    if (bh == 0) *a.fb_count = 0;
  }
  __syncthreads();
  const int F = s_f;
  for (int j = tid; j < a.n_blocks; j += 256) a.k_exp[r0 + j] -= F;
}

// ------------------------------------------------------------------------------- the bounds

// Row i's approximate scores are v_ij = I_ij * 2^(f_j - F) (I_ij the kept digit products over
// 2^16, f_j key block j's exponent, F the largest over the head's key blocks), in float32. They
// stand for s_ij * 2^-(e_i + 16 + F). With X = x 2^-e + dx, |dx| <= 1/2 per channel (likewise Y):
//   |X.Y - 2^-(e+f) s| <= |x|_1 2^-e / 2 + |y|_1 2^-f / 2 + D/4,   dropped pairs <= D * 8404992,
// hence in v units |v - s 2^-(e+16+F)| <= D 8404992.25 2^-16 + |x|_1 2^-(e+17) + max|y|_1 2^-(F+17).
// The float32 evaluation of v (two roundings, of the 2^8-weight products and of the sum with the
// 2^0-weight ones, |p2| <= D 2^15) adds at most 2^-23 |v| + D 2^-9, float32 underflow 2^-126.
// The range bound |v| <= |x|_2 max|y|_2 2^-(e+16+F) + E gives the histogram's span.
struct RowBound {
  double e_v;      // error bound E (v units)
  double b_v;      // |v| <= b_v
  double to_v;     // v units per unit of s: 2^-(e+16+F)
};

template <int D>
__device__ __forceinline__ RowBound row_bound(const SelectArgs& a, int64_t bh, int i) {
  const int64_t r = bh * n_pad(a.n_blocks) + i;
  const int e = a.q_exp[r];
  const float2 qn = *reinterpret_cast<const float2*>(a.q_norm + 2 * r);
  const int F = a.key_stat[4 * bh + 0];
  const double y1 = (double)__int_as_float(a.key_stat[4 * bh + 1]);
  const double y2 = (double)__int_as_float(a.key_stat[4 * bh + 2]);
  RowBound rb;
  const double to_v = ldexp(1.0, -(e + 16 + F));
  double ev = (double)D * kDropPerChannel * 0x1p-16;
  if (qn.x > 0.f) ev += (double)qn.x * ldexp(1.0, -(e + 17));
  if (y1 > 0.0) ev += y1 * ldexp(1.0, -(F + 17));
  double bv = (double)qn.y * y2 * to_v + ev;
  bv *= 1.0 + 0x1p-10;
  rb.e_v = (ev + 0x1p-22 * bv + (double)D * 0x1p-9) * (1.0 + 0x1p-10) + 0x1p-126;
  rb.b_v = bv;
  rb.to_v = to_v;
  return rb;
}

// The float64 score q_mean_i . k_mean_j, summed in channel order (the evaluation of the kernels
// that decide single entries: the threshold passes and the fallback).
template <int D>
__device__ __forceinline__ double exact_score(const double* qm, const double* km) {
  double s = 0.0;
#pragma unroll 8
  for (int d = 0; d < D; d += 2) {
    const double2 x = *reinterpret_cast<const double2*>(qm + d);
    const double2 y = *reinterpret_cast<const double2*>(km + d);
    s = fma(x.x, y.x, s);
    s = fma(x.y, y.y, s);
  }
  return s;
}

// ---------------------------------------------------------------------------- the score pass

// Query operand of a workgroup's 32 rows: for each k step and digit, lane l holds the 16 bytes
// of row (i0 + l % 32) for channels 32 t + 16 (l / 32) ..; the key operand is laid out alike.
template <int D>
struct QueryOperand {
  i32x4 f[D / 32][3];
  __device__ __forceinline__ void load(const SelectArgs& a, int64_t bh, int chunk, int lane) {
    const int64_t nchunks = n_pad(a.n_blocks) / kRows;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int L = 0; L < 3; ++L)
        f[t][L] = *reinterpret_cast<const i32x4*>(a.q_digits + (((bh * nchunks + chunk) * (D / 32) + t) * 3 + L) * 1024 + lane * 16);
  }
};

// Every (row, key) score of the workgroup's rows, key chunks of 32 spread over the waves. For
// each entry calls fn(q, j, v, valid): the lane's q-th product (0..15), key block j, the
// approximate score v of row r = lane % 32 (every entry a lane sees belongs to that row) and
// whether j is a real key block (the last chunk is padded); then done(c) once the 16 entries of
// chunk c are through. The MFMA's output holds key 8 (q / 4) + 4 (l / 32) + q % 4 of query
// l % 32 in accumulator q of lane l, so lanes r and r + 32 together see all 32 keys of a chunk.
// The next chunk's operands are loaded once the products are issued and arrive under the
// per-entry work. Every lane runs every pass (the MFMA operands of a lane feed the outputs of
// the other lanes), so callers fold row liveness and validity into their arithmetic, and the
// loop bounds are uniform over the wave. PIPE = false loads each chunk just before its products
// (fewer registers, for the passes that also evaluate float64 scores).
template <int D, bool PIPE = true, typename Fn, typename Done>
__device__ __forceinline__ void score_pass(const SelectArgs& a, const QueryOperand<D>& qo, int64_t bh, int wave,
                                           int lane, Fn&& fn, Done&& done) {
  const int nb = a.n_blocks;
  const int nchunks = (int)(n_pad(nb) / kRows);
  const int w = __builtin_amdgcn_readfirstlane(wave);
  if (w >= nchunks) return;
  const int last = nchunks - 1;
  const int8_t* kd = a.k_digits + bh * nchunks * (D / 32) * 3 * 1024 + lane * 16;
  const int* ks = a.k_exp + bh * n_pad(nb) + 4 * (lane >> 5);
  typedef i32x4 Digits[D / 32][3];
  auto load = [&](int c, Digits& f) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int L = 0; L < 3; ++L)
        f[t][L] = *reinterpret_cast<const i32x4*>(kd + ((int64_t)(c * (D / 32) + t) * 3 + L) * 1024);
  };
  Digits f;
  if (PIPE) load(w, f);
  // TAIL: the last chunk, where key blocks past nb are padding
  auto chunk = [&](int c, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    if (!PIPE) load(c, f);
    i32x4 sh[4];  // needed after the products: loaded under them
#pragma unroll
    for (int g = 0; g < 4; ++g) sh[g] = *reinterpret_cast<const i32x4*>(ks + 32 * c + 8 * g);
    i32x16 p4 = {}, p3 = {}, p2 = {};
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      p4 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][2], qo.f[t][2], p4, 0, 0, 0);
      p3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][2], qo.f[t][1], p3, 0, 0, 0);
      p3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][1], qo.f[t][2], p3, 0, 0, 0);
      p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][2], qo.f[t][0], p2, 0, 0, 0);
      p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][1], qo.f[t][1], p2, 0, 0, 0);
      p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[t][0], qo.f[t][2], p2, 0, 0, 0);
    }
    if (PIPE && !TAIL) load(c + kWaves <= last ? c + kWaves : last, f);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int j = 32 * c + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
      // 2^8 p4 + p3 is exact in int32: |p4| <= D 2^12 (|d2| <= 64), |p3| <= D 2^14
      const int m = (p4[q] << 8) + p3[q];
      const float v = ldexpf(fmaf((float)m, 256.f, (float)p2[q]), sh[q / 4][q % 4]);
      fn(q, j, v, TAIL ? j < nb : true);
    }
    done(c);
  };
  int c = w;
  for (; c < last; c += kWaves) chunk(c, std::false_type{});
  if (c == last) chunk(c, std::true_type{});
}

// ---------------------------------------------------------------------- histogram bracketing

// Bin position of v in a row's first-level histogram over [-B, B]: t = v * scale + off with
// scale = NBINS / 2B and off = B * scale (rounded once, by the fma); the bin is t clamped to
// [0, NBINS - 1] and truncated, the sub-bin inside a chosen bin b likewise from (t - b) NBINS
// (exact: t - b is in [0, 1) for entries of bin b, except in the clamped end bins, whose
// sub-bins are clamped too). The value kBins stands for "no bin": it lands in the pad word.
__device__ __forceinline__ float bin_pos(float v, float scale, float off) { return fmaf(v, scale, off); }
__device__ __forceinline__ int bin_of(float t) { return (int)__builtin_amdgcn_fmed3f(t, 0.f, (float)(kBins - 1)); }
__device__ __forceinline__ int sub_of(float t, int b) {
  return (int)__builtin_amdgcn_fmed3f((t - (float)b) * (float)kBins, 0.f, (float)(kBins - 1));
}

// 16-bit counts, two per word; bin kBins is the row's pad word
__device__ __forceinline__ void hist_inc(uint32_t* row_hist, int bin) {
  atomicAdd(&row_hist[bin >> 1], 1u << ((bin & 1) << 4));
}

// Wave-wide sum and exclusive scan of a non-negative value below 2^B per lane, bit-sliced through
// ballots (no data moves between lanes).
__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
template <int B>
__device__ __forceinline__ int wave_sum_b(uint32_t x) {
  int s = 0;
#pragma unroll
  for (int b = 0; b < B; ++b) s += __popcll(__ballot((x >> b) & 1u)) << b;
  return s;
}
template <int B>
__device__ __forceinline__ int wave_excl_scan_b(uint32_t x) {
  int s = 0;
#pragma unroll
  for (int b = 0; b < B; ++b) s += lanes_below(__ballot((x >> b) & 1u)) << b;
  return s;
}

// Per-row work runs on 16-lane segments (a DPP row), four rows per wave at once; sums and scans
// over a segment use DPP row rotations and shifts.
constexpr int kSeg = 16;                 // lanes per row
constexpr int kSegRows = 64 / kSeg;      // rows per wave at once
__device__ __forceinline__ int seg_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);  // row_ror:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false);  // row_ror:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false);  // row_ror:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false);  // row_ror:1
  return x;
}
__device__ __forceinline__ int seg_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1, zeros shifted in
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  return x;
}
// the value of the segment's lane src (a lane of the same segment)
__device__ __forceinline__ int seg_get(int x, int src) { return __shfl(x, src); }

// Each segment finds, in its row's histogram, the bin holding the want-th largest entry: returns
// the bin and, through above/count, the entries in higher bins and in the bin. Level a: lane s of
// the segment owns bins [kBins - 64 (s + 1), kBins - 64 s) (32 words, highest first); level b:
// the 64 bins of the lane holding the entry, 4 per lane. (Counts are at most nB <= 19968.)
__device__ int find_bin_seg(const uint32_t* row_hist, int want, int lane, int* above, int* count) {
  const int sl = lane & (kSeg - 1), seg0 = lane & ~(kSeg - 1);
  const unsigned long long segmask = 0xffffull << seg0;
  int s = 0;
  {
    const u32x4* p = reinterpret_cast<const u32x4*>(row_hist + kBins / 2 - 32 * (sl + 1));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const u32x4 w = p[k];
      s += (int)((w.x & 0xffffu) + (w.x >> 16) + (w.y & 0xffffu) + (w.y >> 16) + (w.z & 0xffffu) + (w.z >> 16) +
                 (w.w & 0xffffu) + (w.w >> 16));
    }
  }
  int inc = seg_incl_scan(s);
  unsigned long long hit = __ballot(inc - s < want && want <= inc) & segmask;
  const int o = hit ? (int)__builtin_ctzll(hit) : seg0;        // lane holding the entry
  const int before_o = seg_get(inc - s, o);
  // level b: bins kBins - 1 - 64 (o - seg0) - (4 sl + u), u = 0..3, in two words
  const int top = kBins - 1 - 64 * (o - seg0) - 4 * sl;
  const uint32_t w1 = row_hist[top >> 1], w0 = row_hist[(top >> 1) - 1];
  const int c[4] = {(int)(w1 >> 16), (int)(w1 & 0xffffu), (int)(w0 >> 16), (int)(w0 & 0xffffu)};
  const int s2 = c[0] + c[1] + c[2] + c[3];
  const int inc2 = seg_incl_scan(s2) + before_o;
  hit = __ballot(inc2 - s2 < want && want <= inc2) & segmask;
  const int o2 = hit ? (int)__builtin_ctzll(hit) : seg0;
  int bin = 0, ab = 0, cn = 0, acc = inc2 - s2;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (acc < want && want <= acc + c[u]) { bin = top - u; ab = acc; cn = c[u]; }
    acc += c[u];
  }
  *above = seg_get(ab, o2);
  *count = seg_get(cn, o2);
  return seg_get(bin, o2);
}

// order-preserving map of a double to uint64 (larger double -> larger key); -0 is folded to +0
__device__ __forceinline__ uint64_t order_key(double x) {
  x = x + 0.0;  // -0.0 + 0.0 = +0.0 under round-to-nearest
  const uint64_t u = __double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
// the same for float32: every finite float maps above 0
__device__ __forceinline__ uint32_t order_u32(float x) {
  const uint32_t u = __float_as_uint(x + 0.f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_u32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// OR of the values of lanes l and l ^ 32, in both
__device__ __forceinline__ uint32_t pair_or(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] | r[1];
}

// Writes the set bits of a row's bitmap (words [0, words)) in ascending order to dst, one wave;
// returns the number written (positions at or past cap are not written).
__device__ int64_t write_bits(const uint32_t* bits, int words, int32_t* dst, int64_t cap, int lane) {
  int64_t carry = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t m = w < words ? bits[w] : 0u;
    const int cnt = __popc(m);
    int64_t pos = carry + wave_excl_scan_b<6>((uint32_t)cnt);
    while (m) {
      const int bt = __builtin_ctz(m);
      if (pos < cap) dst[pos] = 32 * w + bt;
      ++pos;
      m &= m - 1;
    }
    carry += wave_sum_b<6>((uint32_t)cnt);
  }
  return carry;
}

// ----------------------------------------------------------------------------- top-k select

// The (batch-head, row chunk) of a selection workgroup. Consecutive workgroup ids are dealt to
// the 8 XCDs in turn; renumbered so that each XCD takes one contiguous range of (head, chunk)
// pairs, the workgroups of a head share one XCD's L2 and read its key operands from there.
struct WgTile {
  int64_t bh;
  int chunk;
};
__device__ __forceinline__ WgTile xcd_tile() {
  const int nrc = (int)gridDim.x;
  const int total = nrc * (int)gridDim.y;
  const int id = (int)blockIdx.x + nrc * (int)blockIdx.y;
  const int per = total / 8, rem = total % 8, x = id % 8, s = id / 8;
  const int lin = x < rem ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
  return WgTile{lin / nrc, lin % nrc};
}

constexpr int kAmbList = 256;  // entries of a workgroup decided on float64 scores
static_assert(kWaves * kSegRows * kSeg * 32 * 4 <= kRows * (kCap + 1) * 8, "staging must fit in the candidate lists");

// Per-row state of a selection workgroup, in LDS.
struct RowState {
  float scale[kRows], off[kRows], bsum[kRows];  // bin position t = v * scale + off over [-bsum, bsum]
  double e_v[kRows];                 // error bound E (v units)
  int bin1[kRows], bin2[kRows];      // chosen first-level bin, chosen sub-bin (-1: none)
  int above[kRows], count[kRows];    // entries above the chosen (sub)bin and inside it
  int status[kRows];                 // 0 resolving, 1 invalid row, 2 routed to the fallback
  float in_thr[kRows], cand_thr[kRows];  // classification thresholds (v units, rounded outward)
  int ncand[kRows];
  int need_a[kRows], amb0[kRows], namb[kRows];  // float64 decisions: the row's slice of the list
  int amb_total;
  int refine;
  uint32_t amb_e[kAmbList];          // (row << 16) | key block
  double amb_s[kAmbList];            // their float64 scores
};

// Per workgroup: 32 query blocks of one (batch, head).
//  1. histogram of every row's approximate scores (a second, finer pass over the chosen bin when
//     it holds more than kCap entries) -> the bin holding the keep-th largest;
//  2. classification pass: above the bin by more than 2E (plus the bin arithmetic's slack) ->
//     kept, written as bitmap words; within -> candidate (v, j) in the row's LDS list;
//  3. per row (one wave): the keep-th largest v among the candidates (t), candidates above t by
//     more than 2E kept, the ones within 2E of t listed for a float64 decision;
//  4. the listed entries' float64 scores, the whole workgroup at once; per row the best of them
//     by (score descending, index ascending) fill the remaining places;
//  5. the row's kept set written in ascending order. Rows that do not resolve (a bin that cannot
//     be split, overfull lists) are routed to the fallback kernel.
template <int D>
__global__ __launch_bounds__(kSelThreads, 2) void topk_select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ RowState st;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.n_blocks, keep = a.keep;
  const WgTile tile = xcd_tile();
  const int64_t bh = tile.bh;
  const int i0 = tile.chunk * kRows;
  const int words = (nb + 31) / 32;
  uint32_t* hist = dyn;                                        // [kRows][kHistStride]
  uint32_t* bits = dyn;                                        // [kRows][words]   (after the histograms)
  uint2* cand = reinterpret_cast<uint2*>(dyn + kRows * words);  // [kRows][kCap + 1]: (v bits, j), last slot discards

  int32_t* out_base = a.block_idx + (bh * nb + i0) * (int64_t)keep;
  if (keep == nb) {  // every block kept
    for (int r = wave; r < kRows; r += kWaves)
      if (i0 + r < nb)
        for (int j = lane; j < nb; j += 64) out_base[(int64_t)r * keep + j] = j;
    return;
  }
  if (tid < kRows) {
    const int i = i0 + tid;
    st.status[tid] = i < nb ? 0 : 1;
    st.bin2[tid] = -1;
    st.ncand[tid] = 0;
    st.namb[tid] = 0;
    float bs = 1.f;
    if (i < nb) {
      const RowBound rb = row_bound<D>(a, bh, i);
      st.e_v[tid] = rb.e_v;
      bs = __double2float_ru(rb.b_v);
    }
    const float sc = (float)kBins / (2.f * bs);
    st.bsum[tid] = bs;
    st.scale[tid] = sc;
    st.off[tid] = bs * sc;
  }
  if (tid == 0) {
    st.refine = 0;
    st.amb_total = 0;
  }
  for (int e = tid; e < kAmbList; e += kSelThreads) st.amb_e[e] = 0u;  // a harmless (row 0, key 0)
  QueryOperand<D> qo;
  qo.load(a, bh, tile.chunk, lane);
  for (int w = tid; w < kRows * kHistStride; w += kSelThreads) hist[w] = 0u;
  __syncthreads();

  // every entry a lane sees belongs to row r = lane % 32: its parameters stay in registers
  const int my_r = lane & 31;
  const bool my_live = st.status[my_r] == 0;
  const float my_scale = st.scale[my_r], my_off = st.off[my_r];
  uint32_t* my_hist = hist + my_r * kHistStride;
  auto no_done = [](int) {};

  // 1. level 1: histogram of every valid row
  // (rows past the end count garbage into their own, unread histograms)
  score_pass<D>(a, qo, bh, wave, lane, [&](int, int, float v, bool valid) {
    hist_inc(my_hist, valid ? bin_of(bin_pos(v, my_scale, my_off)) : kBins);
  }, no_done);
  __syncthreads();
  const int seg = lane / kSeg, sl = lane % kSeg;
  for (int r0 = wave * kSegRows; r0 < kRows; r0 += kWaves * kSegRows) {
    const int r = r0 + seg;
    int ab, cn;
    const int b = find_bin_seg(hist + r * kHistStride, keep, lane, &ab, &cn);
    if (sl == 0 && st.status[r] == 0) {
      st.bin1[r] = b;
      st.above[r] = ab;
      st.count[r] = cn;
      if (cn > kCap) st.refine = 1;
    }
  }
  __syncthreads();
  // level 2, only when some row's bin holds more entries than the candidate slots
  if (st.refine) {
    const bool my_refine = my_live && st.count[my_r] > kCap;
    const int my_bin1 = st.bin1[my_r];
    __syncthreads();
    for (int w = tid; w < kRows * kHistStride; w += kSelThreads) hist[w] = 0u;
    __syncthreads();
    score_pass<D>(a, qo, bh, wave, lane, [&](int, int, float v, bool valid) {
      const float t = bin_pos(v, my_scale, my_off);
      hist_inc(my_hist, valid && my_refine && bin_of(t) == my_bin1 ? sub_of(t, my_bin1) : kBins);
    }, no_done);
    __syncthreads();
    for (int r0 = wave * kSegRows; r0 < kRows; r0 += kWaves * kSegRows) {
      const int r = r0 + seg;
      const bool act = st.status[r] == 0 && st.count[r] > kCap;
      int ab, cn;
      const int b2 = find_bin_seg(hist + r * kHistStride, keep - st.above[r], lane, &ab, &cn);
      if (sl == 0 && act) {
        st.bin2[r] = b2;
        st.above[r] += ab;
        st.count[r] = cn;
        if (cn > kCap) st.status[r] = 2;
      }
    }
    __syncthreads();
  }
  // classification thresholds: the chosen (sub)bin spans t in [tlo, thi); back in v units with a
  // slack of 2^-20 B for the float32 bin arithmetic, then widened by 2 E and rounded outward
  if (tid < kRows && st.status[tid] == 0) {
    const int r = tid;
    const double b1 = st.bin1[r];
    const double tlo = st.bin2[r] < 0 ? b1 : b1 + st.bin2[r] / (double)kBins;
    const double thi = st.bin2[r] < 0 ? b1 + 1.0 : b1 + (st.bin2[r] + 1) / (double)kBins;
    const double sc = st.scale[r], off = st.off[r];
    const double slack = 0x1p-20 * (double)st.bsum[r];
    const double e2 = 2.0 * st.e_v[r];
    st.cand_thr[r] = tlo <= 0.0 ? -INFINITY : __double2float_rd((tlo - off) / sc - slack - e2);
    st.in_thr[r] = thi >= (double)kBins ? INFINITY : __double2float_ru((thi - off) / sc + slack + e2);
  }
  __syncthreads();
  // 2. classification: every bitmap word is written by the wave that scores its chunk (rows not
  // resolving here write their own, unread regions)
  {
    const float in_thr = st.in_thr[my_r], cand_thr = st.cand_thr[my_r];
    uint32_t* my_bits = bits + my_r * words;
    uint2* my_cand = cand + my_r * (kCap + 1);
    int* my_n = &st.ncand[my_r];
    uint32_t inm = 0u, cm = 0u;
    float cv[16];
    score_pass<D>(a, qo, bh, wave, lane, [&](int q, int j, float v, bool valid) {
      const bool in = valid && v > in_thr;
      const bool cd = valid && !(v > in_thr) && v >= cand_thr;
      inm |= (uint32_t)in << (j & 31);
      cm |= (uint32_t)cd << q;
      cv[q] = v;
    }, [&](int c) {
      my_bits[c] = pair_or(inm);
      const int base = atomicAdd(my_n, __popc(cm));
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int slot = base + __popc(cm & ((1u << q) - 1u));
        const bool put = ((cm >> q) & 1u) && slot < kCap;
        const int j = 32 * c + 8 * (q / 4) + 4 * (lane >> 5) + (q % 4);
        my_cand[put ? slot : kCap] = uint2{__float_as_uint(cv[q]), (uint32_t)j};
      }
      inm = 0u;
      cm = 0u;
    });
  }
  __syncthreads();

  // 3. per row (a segment): the pivot, the sure entries and the list for float64 decisions
  for (int r0 = wave * kSegRows; r0 < kRows; r0 += kWaves * kSegRows) {
    const int r = r0 + seg;
    const int status = st.status[r];
    const int n = st.ncand[r];
    bool fb = status == 2 || n > kCap;
    int nsure = 0;
    for (int w = sl; w < words; w += kSeg) nsure += __popc(bits[r * words + w]);
    nsure = seg_sum(nsure);
    const int need = keep - nsure;
    fb = fb || need < 1 || need > n;
    const bool go = status != 1 && !fb;
    const uint2* cr = cand + r * (kCap + 1);
    constexpr int U = (kCap + kSeg - 1) / kSeg;
    uint32_t key[U];
    float cvv[U];
    int cjj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = sl + kSeg * u;
      const bool present = go && c < n;
      const uint2 e = present ? cr[c] : uint2{0u, 0u};
      cvv[u] = __uint_as_float(e.x);
      cjj[u] = (int)e.y;
      key[u] = present ? order_u32(cvv[u]) : 0u;
    }
    // t: the need-th largest v, bit by bit. Every candidate lies in [cand_thr, in_thr], so the bits
    // above the highest one where the bracket's keys differ are the bracket's; the search runs over
    // the rest (the wave's widest), absent slots holding key 0.
    const uint32_t lo = order_u32(st.cand_thr[r]), hi = order_u32(st.in_thr[r]);
    const uint32_t diff = go ? lo ^ hi : 0u;
    const uint32_t dw = (uint32_t)__builtin_amdgcn_readlane((int)diff, 0) | (uint32_t)__builtin_amdgcn_readlane((int)diff, 16) |
                        (uint32_t)__builtin_amdgcn_readlane((int)diff, 32) | (uint32_t)__builtin_amdgcn_readlane((int)diff, 48);
    const int top = dw ? 31 - __builtin_clz(dw) : -1;
    uint32_t T = top < 0 ? lo : (top >= 31 ? 0u : (lo & ~((2u << top) - 1u)));
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t T2 = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) cnt += key[u] >= T2;
      if (seg_sum(cnt) >= need) T = T2;
    }
    const double t = from_order_u32(T), e2 = 2.0 * st.e_v[r];
    int nin = 0, nam = 0;
    bool am[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool present = go && sl + kSeg * u < n;
      const double v = cvv[u];
      const bool in = present && v - e2 > t;
      am[u] = present && !in && v + e2 >= t;
      if (in) atomicOr(&bits[r * words + (cjj[u] >> 5)], 1u << (cjj[u] & 31));
      nin += in;
      nam += am[u];
    }
    nin = seg_sum(nin);
    const int na = seg_sum(nam);
    const int need_a = need - nin;
    if (go) {
      if (need_a < 1 || need_a > na) {
        fb = true;
      } else if (need_a == na) {  // every listed entry is kept: no float64 decision needed
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (am[u]) atomicOr(&bits[r * words + (cjj[u] >> 5)], 1u << (cjj[u] & 31));
      } else {
        int start = 0;
        if (sl == 0) start = atomicAdd(&st.amb_total, na);
        start = seg_get(start, lane & ~(kSeg - 1));
        if (start + na > kAmbList) {
          fb = true;
        } else {
          int pos = start + seg_incl_scan(nam) - nam;
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (am[u]) st.amb_e[pos++] = ((uint32_t)r << 16) | (uint32_t)cjj[u];
          if (sl == 0) {
            st.need_a[r] = need_a;
            st.amb0[r] = start;
            st.namb[r] = na;
          }
        }
      }
    }
    if (fb && status != 1 && sl == 0) {
      st.status[r] = 2;
      const int slot = atomicAdd(a.fb_count, 1);
      a.fb_rows[slot] = (int32_t)(bh * nb + i0 + r);
    }
  }
  __syncthreads();

  // 4. the listed entries' float64 scores, four per wave at a time: lane l multiplies channels
  // 2l and 2l+1, a fixed shuffle tree adds the 64 products
  {
    const int total = st.amb_total < kAmbList ? st.amb_total : kAmbList;
    const double* qm_base = a.q_mean + (bh * nb + i0) * (int64_t)D;
    const double* km_base = a.k_mean + bh * nb * (int64_t)D;
    for (int e0 = 4 * wave; e0 < total; e0 += 4 * kWaves) {
      double p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = 0.0;
        const int e = e0 + u;
        if (e < total && 2 * lane < D) {
          const uint32_t ent = st.amb_e[e];
          const double2 x = *reinterpret_cast<const double2*>(qm_base + (int64_t)(ent >> 16) * D + 2 * lane);
          const double2 y = *reinterpret_cast<const double2*>(km_base + (int64_t)(ent & 0xffffu) * D + 2 * lane);
          p[u] = fma(x.y, y.y, x.x * y.x);
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] += __shfl_down(p[u], off);
      if (lane == 0)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (e0 + u < total) st.amb_s[e0 + u] = p[u];
    }
  }
  __syncthreads();

  // 5. per row (a segment): the best need_a listed entries by (score descending, index ascending),
  // then the ordered write, 16 bitmap words (at most 512 indices) at a time through a staging
  // area in the candidate lists' LDS (no longer needed), copied out with consecutive lanes on
  // consecutive indices
  int32_t* stage = reinterpret_cast<int32_t*>(cand) + (wave * kSegRows + seg) * (kSeg * 32);
  for (int r0 = wave * kSegRows; r0 < kRows; r0 += kWaves * kSegRows) {
    const int r = r0 + seg;
    const bool go = st.status[r] == 0;
    const int na = go ? st.namb[r] : 0, s0 = st.amb0[r], need_a = st.need_a[r];
    for (int c = sl; c < na; c += kSeg) {
      const double sc = st.amb_s[s0 + c];
      const int j = (int)(st.amb_e[s0 + c] & 0xffffu);
      int rk = 0;
      for (int c2 = 0; c2 < na; ++c2) {
        const double s2 = st.amb_s[s0 + c2];
        const int j2 = (int)(st.amb_e[s0 + c2] & 0xffffu);
        rk += (s2 > sc) || (s2 == sc && j2 < j);
      }
      if (rk < need_a) atomicOr(&bits[r * words + (j >> 5)], 1u << (j & 31));
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    int32_t* dst = out_base + (int64_t)r * keep;
    int carry = 0;
    for (int w0 = 0; w0 < words; w0 += kSeg) {
      const int w = w0 + sl;
      uint32_t m = go && w < words ? bits[r * words + w] : 0u;
      const int cnt = __popc(m);
      int pos = seg_incl_scan(cnt) - cnt;
      const int tot = seg_sum(cnt);
      while (m) {
        stage[pos++] = 32 * w + __builtin_ctz(m);
        m &= m - 1;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
      for (int p = sl; p < tot; p += kSeg)
        if (carry + p < keep) dst[carry + p] = stage[p];
      carry += tot;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
    }
  }
}

// --------------------------------------------------------------------------------- fallback

constexpr int kFbThreads = 256;

// block-wide exclusive prefix sum of one int per thread; returns the block total in *total
__device__ int block_exclusive_scan(int v, int* total, int* scratch /* >= 4 ints */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFbThreads / 64; ++w) {
    const int s = scratch[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// Writes, in ascending index order, every j with (keys[j] & mask) > thr plus the first k_rem
// indices with (keys[j] & mask) == thr (thr has no bits outside mask); each thread scans one
// contiguous index range, two block scans place the runs.
__device__ void ordered_compact(const uint64_t* keys, int nb, uint64_t thr, uint64_t mask, int k_rem, int32_t* dst,
                                int keep, int* scan_scratch) {
  const int tid = threadIdx.x;
  const int per = (nb + kFbThreads - 1) / kFbThreads;
  const int j0 = tid * per;
  const int j1 = j0 + per < nb ? j0 + per : nb;
  int n_eq = 0;
  for (int j = j0; j < j1; ++j) n_eq += (keys[j] & mask) == thr;
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, &tot, scan_scratch);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint64_t key = keys[j] & mask;
      if (key > thr) ++n_sel;
      else if (key == thr) { if (e < k_rem) ++n_sel; ++e; }
    }
  }
  const int pos0 = block_exclusive_scan(n_sel, &tot, scan_scratch);
  int e = eq_before, p = pos0;
  for (int j = j0; j < j1; ++j) {
    const uint64_t key = keys[j] & mask;
    bool take = false;
    if (key > thr) take = true;
    else if (key == thr) { take = e < k_rem; ++e; }
    if (take && p < keep) dst[p++] = j;
  }
}

// Rows the bracketing could not resolve (many exactly equal scores at the keep-th place): the
// row's float64 scores in LDS as order-preserving keys, then an MSB radix select of the keep-th
// largest key, 8 bits per pass (thread t owns bin 255 - t; a block prefix sum finds the digit;
// the select stops once the chosen bin holds exactly the keys still wanted), then the ordered
// compaction. A fixed grid walks the list of routed rows.
template <int D>
__global__ __launch_bounds__(kFbThreads) void fallback_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);
  __shared__ uint32_t hist[256];
  __shared__ int scan_scratch[4];
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_krem, sh_done;
  const int tid = threadIdx.x;
  const int nb = a.n_blocks;
  const int total = *a.fb_count;
  for (int e = blockIdx.x; e < total; e += gridDim.x) {
    const int64_t row = a.fb_rows[e];
    const int64_t bh = row / nb;
    const double* qm = a.q_mean + row * D;
    const double* km = a.k_mean + bh * nb * (int64_t)D;
    for (int j = tid; j < nb; j += kFbThreads) keys[j] = order_key(exact_score<D>(qm, km + (int64_t)j * D));
    __syncthreads();
    uint64_t prefix = 0, mask = 0;
    int k_rem = a.keep;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < nb; j += kFbThreads) {
        const uint64_t key = keys[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      const int d = 255 - tid;
      const int h = (int)hist[d];
      int tot;
      const int above = block_exclusive_scan(h, &tot, scan_scratch);
      if (above < k_rem && k_rem <= above + h) {
        sh_prefix = prefix | ((uint64_t)d << shift);
        sh_krem = k_rem - above;
        sh_done = h == k_rem - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      k_rem = sh_krem;
      mask |= (uint64_t)0xff << shift;
      if (sh_done) break;  // block-uniform
    }
    ordered_compact(keys, nb, prefix, mask, k_rem, a.block_idx + row * a.keep, a.keep, scan_scratch);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------- threshold mode

// Threshold mode keeps j iff s_ij >= m_i - tau sqrt(D), m_i = max_j s_ij (unscaled float64
// scores). Entries further than E from the threshold are decided on v, the others on their
// float64 score, so the count and fill kernels decide every entry identically.
struct ThrState {
  double e_v[kRows], to_v[kRows], thr_s[kRows], thr_v[kRows];
  int vmax[kRows];                // order-preserving int of the largest v
  unsigned long long smax[kRows]; // order key of the largest float64 score near the top
  int cnt[kRows];
  int valid[kRows];
};

__device__ __forceinline__ int order_int(float v) {
  const int u = __float_as_int(v + 0.f);
  return u >= 0 ? u : (u ^ 0x7fffffff);
}
__device__ __forceinline__ float from_order_int(int o) { return __int_as_float(o >= 0 ? o : (o ^ 0x7fffffff)); }
__device__ __forceinline__ double from_order_key(uint64_t k) {
  return __longlong_as_double((k & 0x8000000000000000ull) ? (long long)(k & 0x7fffffffffffffffull) : (long long)~k);
}

// 1 keep, 0 drop; decided on v when it is clear of the threshold by more than E (thr_v, e_v in v
// units), otherwise on the float64 score against thr_s
template <int D>
__device__ __forceinline__ int thr_keep(double thr_v, double e_v, double thr_s, float v, const double* qm,
                                        const double* km) {
  const double dv = v;
  if (dv - e_v > thr_v) return 1;
  if (dv + e_v < thr_v) return 0;
  return exact_score<D>(qm, km) >= thr_s ? 1 : 0;
}

template <int D>
__device__ void thr_setup(const SelectArgs& a, ThrState& ts, int64_t bh, int i0, int tid) {
  if (tid < kRows) {
    const int i = i0 + tid;
    ts.valid[tid] = i < a.n_blocks;
    ts.vmax[tid] = order_int(-INFINITY);
    ts.smax[tid] = 0ull;
    ts.cnt[tid] = 0;
    if (i < a.n_blocks) {
      const RowBound rb = row_bound<D>(a, bh, i);
      ts.e_v[tid] = rb.e_v;
      ts.to_v[tid] = rb.to_v;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kSelThreads, 2) void threshold_count_kernel(SelectArgs a) {
  __shared__ ThrState ts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.n_blocks;
  const WgTile tile = xcd_tile();
  const int64_t bh = tile.bh;
  const int i0 = tile.chunk * kRows;
  thr_setup<D>(a, ts, bh, i0, tid);
  QueryOperand<D> qo;
  qo.load(a, bh, tile.chunk, lane);
  __syncthreads();
  const double* qm_base = a.q_mean + (bh * nb + i0) * D;
  const double* km_base = a.k_mean + bh * nb * (int64_t)D;
  const int r = lane & 31;
  const bool live = ts.valid[r];
  // the largest v of each row (a per-lane maximum first)
  {
    float vm = -INFINITY;
    score_pass<D, false>(a, qo, bh, wave, lane, [&](int, int, float v, bool valid) { vm = fmaxf(vm, valid ? v : -INFINITY); },
                  [](int) {});
    if (live) atomicMax(&ts.vmax[r], order_int(vm));
  }
  __syncthreads();
  // the exact maximum is among the entries within 2E of the largest v
  {
    const double lim = (double)from_order_int(ts.vmax[r]) - 2.0 * ts.e_v[r];
    unsigned long long sm = 0ull;
    score_pass<D, false>(a, qo, bh, wave, lane, [&](int, int j, float v, bool valid) {
      if (live && valid && (double)v >= lim) {
        const uint64_t key = order_key(exact_score<D>(qm_base + (int64_t)r * D, km_base + (int64_t)j * D));
        sm = key > sm ? key : sm;
      }
    }, [](int) {});
    if (live) atomicMax(&ts.smax[r], sm);
  }
  __syncthreads();
  if (tid < kRows && ts.valid[tid]) {
    const double m = from_order_key(ts.smax[tid]);
    const double thr = m - a.tau_raw;
    ts.thr_s[tid] = thr;
    ts.thr_v[tid] = thr * ts.to_v[tid];
  }
  __syncthreads();
  {
    int cnt = 0;
    const double thr_v = ts.thr_v[r], e_v = ts.e_v[r], thr_s = ts.thr_s[r];
    const double* qm = qm_base + (int64_t)r * D;
    score_pass<D, false>(a, qo, bh, wave, lane, [&](int, int j, float v, bool valid) {
      if (live && valid) cnt += thr_keep<D>(thr_v, e_v, thr_s, v, qm, km_base + (int64_t)j * D);
    }, [](int) {});
    if (live) atomicAdd(&ts.cnt[r], cnt);
  }
  __syncthreads();
  if (tid < kRows && ts.valid[tid]) {
    const int64_t row = bh * nb + i0 + tid;
    a.row_cnt[row] = ts.cnt[tid];
    a.row_thr[row] = ts.thr_s[tid];
  }
}

template <int D>
__global__ __launch_bounds__(kSelThreads, 2) void threshold_fill_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t bits[];  // [kRows][words]
  __shared__ ThrState ts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.n_blocks;
  const int words = (nb + 31) / 32;
  const WgTile tile = xcd_tile();
  const int64_t bh = tile.bh;
  const int i0 = tile.chunk * kRows;
  thr_setup<D>(a, ts, bh, i0, tid);
  if (tid < kRows && ts.valid[tid]) {
    ts.thr_s[tid] = a.row_thr[bh * nb + i0 + tid];
    ts.thr_v[tid] = ts.thr_s[tid] * ts.to_v[tid];
  }
  QueryOperand<D> qo;
  qo.load(a, bh, tile.chunk, lane);
  for (int w = tid; w < kRows * words; w += kSelThreads) bits[w] = 0u;
  __syncthreads();
  const double* qm_base = a.q_mean + (bh * nb + i0) * D;
  const double* km_base = a.k_mean + bh * nb * (int64_t)D;
  {
    const int r = lane & 31;
    const double thr_v = ts.thr_v[r], e_v = ts.e_v[r], thr_s = ts.thr_s[r];
    const double* qm = qm_base + (int64_t)r * D;
    uint32_t* my_bits = bits + r * words;
    const bool live = ts.valid[r];
    score_pass<D, false>(a, qo, bh, wave, lane, [&](int, int j, float v, bool valid) {
      if (live && valid && thr_keep<D>(thr_v, e_v, thr_s, v, qm, km_base + (int64_t)j * D))
        atomicOr(&my_bits[j >> 5], 1u << (j & 31));
    }, [](int) {});
  }
  __syncthreads();
  for (int r = wave; r < kRows; r += kWaves) {
    if (!ts.valid[r]) continue;
    const int64_t row = bh * nb + i0 + r;
    const int64_t start = a.row_ptr[row];
    const int64_t room = a.col_capacity - start;
    write_bits(bits + r * words, words, a.col_idx + start, room > 0 ? room : 0, lane);
  }
}

// Exclusive scan of the per-row counts into row_ptr, in one workgroup. Each step covers
// kScanThreads * kScanPer rows: every thread loads kScanPer consecutive counts (all loads in
// flight at once), the thread totals are scanned across the workgroup (wave shuffles, then the
// wave totals through LDS), each thread writes its run, and a carry joins the steps.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;
__global__ __launch_bounds__(kScanThreads) void row_ptr_scan_kernel(SelectArgs a, int64_t rows) {
  __shared__ long long wave_tot[kScanThreads / 64];
  __shared__ long long s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < rows; base += (int64_t)kScanThreads * kScanPer) {
    const int64_t r0 = base + (int64_t)tid * kScanPer;
    long long v[kScanPer];
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) v[u] = r0 + u < rows ? a.row_cnt[r0 + u] : 0;
    long long tot = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) tot += v[u];
    long long inc = tot;  // inclusive scan of the thread totals inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    long long before = s_carry, all = s_carry;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const long long t = wave_tot[w];
      if (w < wave) before += t;
      all += t;
    }
    long long acc = before + inc - tot;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u)
      if (r0 + u < rows) {
        a.row_ptr[r0 + u] = acc;
        acc += v[u];
      }
    __syncthreads();  // every thread has read wave_tot and s_carry
    if (tid == 0) s_carry = all;
    __syncthreads();
  }
  if (tid == 0) a.row_ptr[rows] = s_carry;
}

// pooling grid: (block, head group) x 1 x (batch, tensor)
template <int D>
dim3 pool_grid(const SelectArgs& a) {
  const unsigned groups = (unsigned)((a.heads + kPoolThreads / (D / 8) - 1) / (kPoolThreads / (D / 8)));
  return dim3((unsigned)a.n_blocks * groups, 1, 2u * (unsigned)a.batch);
}

template <int D>
void launch_pool(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(pool_kernel<D>, pool_grid<D>(a), dim3(kPoolThreads), 0, stream, a);
  hipLaunchKernelGGL(key_stats_kernel, dim3((unsigned)(a.batch * a.heads)), dim3(256), 0, stream, a);
}

size_t topk_dyn_lds(int32_t nb) {
  const size_t words = ((size_t)nb + 31) / 32;
  const size_t hist = (size_t)kRows * kHistStride * 4;
  const size_t classify = (size_t)kRows * words * 4 + (size_t)kRows * (kCap + 1) * sizeof(uint2);
  return hist > classify ? hist : classify;
}

// the selection after the pooling kernel: key statistics, top-k, fallback
template <int D>
void launch_topk_pooled(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(key_stats_kernel, dim3((unsigned)(a.batch * a.heads)), dim3(256), 0, stream, a);
  const dim3 grid((unsigned)((a.n_blocks + kRows - 1) / kRows), (unsigned)(a.batch * a.heads));
  const size_t lds = topk_dyn_lds(a.n_blocks);
  // the dynamic-LDS limit plus the kernel's static LDS (RowState) must stay within a CU's 160 KB
  static_assert(sizeof(RowState) <= 8192, "per-row state outgrew its LDS share");
  allow_dynamic_lds(reinterpret_cast<const void*>(topk_select_kernel<D>), 160 * 1024 - 8192);
  hipLaunchKernelGGL(topk_select_kernel<D>, grid, dim3(kSelThreads), lds, stream, a);
  allow_dynamic_lds(reinterpret_cast<const void*>(fallback_kernel<D>), (int)kSelectRowLdsBytes);
  hipLaunchKernelGGL(fallback_kernel<D>, dim3(256), dim3(kFbThreads), (size_t)a.n_blocks * 8, stream, a);
}

template <int D>
void launch_topk(const SelectArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(pool_kernel<D>, pool_grid<D>(a), dim3(kPoolThreads), 0, stream, a);
  launch_topk_pooled<D>(a, stream);
}

template <int D>
void launch_thr_count(const SelectArgs& a, hipStream_t stream) {
  launch_pool<D>(a, stream);
  const dim3 grid((unsigned)((a.n_blocks + kRows - 1) / kRows), (unsigned)(a.batch * a.heads));
  hipLaunchKernelGGL(threshold_count_kernel<D>, grid, dim3(kSelThreads), 0, stream, a);
  const int64_t rows = (int64_t)a.batch * a.heads * a.n_blocks;
  hipLaunchKernelGGL(row_ptr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a, rows);
}

template <int D>
void launch_thr_fill(const SelectArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.n_blocks + kRows - 1) / kRows), (unsigned)(a.batch * a.heads));
  const size_t lds = (size_t)kRows * (((size_t)a.n_blocks + 31) / 32) * 4;
  allow_dynamic_lds(reinterpret_cast<const void*>(threshold_fill_kernel<D>), (int)kSelectRowLdsBytes);
  hipLaunchKernelGGL(threshold_fill_kernel<D>, grid, dim3(kSelThreads), lds, stream, a);
}

}  // namespace

void launch_subblock_select(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_topk<128>(a, stream);
  else launch_topk<64>(a, stream);
}

void launch_qk_norm_rope_pool(const NormRopeArgs& nr, const RopeTable& table, const SelectArgs& a,
                              hipStream_t stream) {
  if (a.head_dim == 128)
    hipLaunchKernelGGL(norm_rope_pool_kernel<128>, pool_grid<128>(a), dim3(kPoolThreads), 0, stream, nr, table, a);
  else
    hipLaunchKernelGGL(norm_rope_pool_kernel<64>, pool_grid<64>(a), dim3(kPoolThreads), 0, stream, nr, table, a);
}

void launch_subblock_select_pooled(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_topk_pooled<128>(a, stream);
  else launch_topk_pooled<64>(a, stream);
}

void launch_threshold_count(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_thr_count<128>(a, stream);
  else launch_thr_count<64>(a, stream);
}

void launch_threshold_fill(const SelectArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_thr_fill<128>(a, stream);
  else launch_thr_fill<64>(a, stream);
}

}  // namespace h3attn
