// FP8 (OCP e4m3) quantisation of the attention inputs for gfx950.
//
// Sources: "智東西…H3 Lightning" (hao.cnyes.com), section "02. 從50步壓到9步三層最佳化實現12倍提速"
// (SageAttention2 speeds up attention) and "VDN-MiniMax-H3：基于MiniMax H3的视频生成加速开源项目"
// (aipuzi.cn), sections "二、功能特色" / "三、技术细节" (FP8 quantised inference). The pages give no
// quantisation rule. Here every scale is a power of two, so x / s is exact and a code is the
// round-to-nearest-even e4m3 value of x / s (v_cvt_pk_fp8_f32); |x / s| <= 448 by construction.
//   q, k: one scale per (batch, head, 64-token block), the smallest power of two s with
//         amax <= 448 s;                                   qk_quant_kernel (one pass)
//   v:    one scale per (batch, head, channel) over all tokens; v_amax_kernel (per-chunk channel
//         maxima) -> v_scale_kernel (maximum over the chunks) -> v_quant_kernel, which transposes
//         each 64-key block to [channel][key slot] for the P.V product.
// All four are HBM-bound streams.
#include "device_util.h"
#include "kernels.h"

namespace h3attn {
namespace {

constexpr int kQThreads = 256;
// 64-token blocks per v_quant workgroup: two, so that each v8t row segment it writes is a whole
// 128-byte line (one block is only 64 bytes of a row)
constexpr int kVBlocks = 2;

// smallest e >= -60 with amax <= 448 * 2^e, for amax > 0 (448 = 0.875 * 2^9); the floor keeps
// the product of a query and a key scale a normal float32
__device__ __forceinline__ int pow2_exponent(float amax) {
  int ex;
  const float m = frexpf(amax, &ex);
  const int e = ex - 9 + (m > 0.875f ? 1 : 0);
  return e > -60 ? e : -60;
}

// 8 values (already divided by their power-of-two scale) -> 8 e4m3 bytes
__device__ __forceinline__ u32x2 to_e4m3x8(const float (&x)[8]) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// grid (heads * nB, 1, 2 * batch): blockIdx.x = blk * heads + h, blockIdx.z = 2 * b + (0: q, 1: k).
// With the head index fastest, the workgroups in flight together read and write whole token rows
// (all heads) instead of one head's 256-byte slice of many rows.
template <int D>
__global__ __launch_bounds__(kQThreads) void qk_quant_kernel(Fp8QuantArgs a) {
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int PER = 64 * CPR / kQThreads;  // chunks per thread
  __shared__ float red[kQThreads / 64];
  const int t = blockIdx.z & 1, b = blockIdx.z >> 1;
  const int h = (int)(blockIdx.x % (unsigned)a.heads);
  const int64_t blk = blockIdx.x / (unsigned)a.heads, N = a.n_tokens;
  const uint16_t* x = t ? a.k : a.q;
  uint8_t* x8 = t ? a.k8 : a.q8;
  float* scale = t ? a.k_scale : a.q_scale;
  const int64_t rs = (int64_t)a.heads * D;
  u32x4 v[PER];
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * kQThreads;
    const int64_t n = blk * 64 + c / CPR;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (n < N) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + ((int64_t)b * N + n) * rs + (int64_t)h * D + (c % CPR) * 8));
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[i][j])), fabsf(bf16_hi(v[i][j]))));
  }
  const float amax = block_max_256(mx, red);
  const int e = amax > 0.f ? pow2_exponent(amax) : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * kQThreads;
    const int64_t n = blk * 64 + c / CPR;
    if (n < N) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[2 * j] = ldexpf(bf16_lo(v[i][j]), -e);  // exact
        f[2 * j + 1] = ldexpf(bf16_hi(v[i][j]), -e);
      }
      __builtin_nontemporal_store(to_e4m3x8(f), reinterpret_cast<u32x2*>(x8 + ((int64_t)b * N + n) * rs + (int64_t)h * D + (c % CPR) * 8));
    }
  }
  if (threadIdx.x == 0) scale[((int64_t)b * a.heads + h) * a.n_blocks + blk] = ldexpf(1.0f, e);
}

// grid (n_chunks, heads, batch): channel maxima of |v| over one chunk of kFp8VChunk tokens
template <int D>
__global__ __launch_bounds__(kQThreads) void v_amax_kernel(Fp8QuantArgs a) {
  constexpr int CPR = D / 8;
  constexpr int TPP = kQThreads / CPR;  // tokens per pass
  __shared__ float red[TPP][D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int col = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  const int64_t N = a.n_tokens, rs = (int64_t)a.heads * D;
  const int64_t n0 = (int64_t)blockIdx.x * kFp8VChunk;
  const int64_t n1 = n0 + kFp8VChunk < N ? n0 + kFp8VChunk : N;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t n = n0 + r0; n < n1; n += TPP) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v + ((int64_t)b * N + n) * rs + (int64_t)h * D + col * 8));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[2 * j] = fmaxf(m[2 * j], fabsf(bf16_lo(v[j])));
      m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16_hi(v[j])));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[r0][col * 8 + j] = m[j];
  __syncthreads();
  if (threadIdx.x < D) {
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < TPP; ++r) mx = fmaxf(mx, red[r][threadIdx.x]);
    a.v_partial[(((int64_t)b * a.heads + h) * a.n_chunks + blockIdx.x) * D + threadIdx.x] = mx;
  }
}

// grid (heads, batch), 1024 threads: the channel scales; 1024 / D threads per channel take every
// (1024 / D)-th chunk, then one thread per channel takes the maximum of their maxima (exact in
// any order)
template <int D>
__global__ __launch_bounds__(1024) void v_scale_kernel(Fp8QuantArgs a) {
  constexpr int S = 1024 / D;
  __shared__ float red[S][D];
  const int ch = threadIdx.x % D, sl = threadIdx.x / D;
  const int64_t bh = (int64_t)blockIdx.y * a.heads + blockIdx.x;
  float mx = 0.f;
  for (int c = sl; c < a.n_chunks; c += S) mx = fmaxf(mx, a.v_partial[(bh * a.n_chunks + c) * D + ch]);
  red[sl][ch] = mx;
  __syncthreads();
  if (threadIdx.x >= D) return;
#pragma unroll
  for (int j = 1; j < S; ++j) mx = fmaxf(mx, red[j][ch]);
  const int e = mx > 0.f ? pow2_exponent(mx) : 0;
  a.v_exp[bh * D + ch] = e;
  a.v_scale[bh * D + ch] = ldexpf(1.0f, e);
}

// v8t layout: the P.V product takes P^T as its B operand straight from the score registers,
// where lane half hl holds, as bytes j = 16m + r (score sub-tile m, accumulator register r), the
// keys 32m + 8(r/4) + 4hl + r%4; the A operand (V^T) of lane half hl reads bytes [32hl, 32hl + 32)
// of a row. So within its block's 64 bytes of a v8t row, key kappa = 32m + 8a4 + 4hl + r
// (r < 4, a4 < 4) sits at slot 16 (2hl + m) + 4a4 + r: each 16-byte segment 2hl + m holds four
// runs of four consecutive keys.
//
// The NBLK blocks of a workgroup are staged in LDS as bf16, one 256-byte row (64 channel pairs)
// per key, with 16-byte writes. The dword of channel pair p of key row kappa sits at
// p ^ swz(kappa), swz taking bits 3, 4 and 5 from key-row bits 6, 2 and 5: the transpose reads
// 4 NBLK keys at a time that differ in exactly those bits, one per lane group, so each group
// lands in its own banks (a byte-wise transpose in LDS had been 16-way bank-conflicted).
__device__ __forceinline__ int vq_swizzle(int kappa) {
  return (((kappa >> 6) & 1) << 3) | (((kappa >> 2) & 1) << 4) | (((kappa >> 5) & 1) << 5);
}

template <int D, int NBLK>
__global__ __launch_bounds__(2 * D * NBLK) void v_quant_kernel(Fp8QuantArgs a) {
  constexpr int NT = 2 * D * NBLK;
  constexpr int CPR = D / 8;
  constexpr int PER = 64 * NBLK * CPR / NT;  // 4
  constexpr int PARTS = 4 * NBLK;            // 16-byte output segments per v8t row
  __shared__ __attribute__((aligned(16))) uint32_t tile[64 * NBLK * 64];
  const int b = blockIdx.z;
  const int h = (int)(blockIdx.x % (unsigned)a.heads);
  const int64_t blk0 = (int64_t)(blockIdx.x / (unsigned)a.heads) * NBLK;
  const int64_t N = a.n_tokens, rs = (int64_t)a.heads * D;
  const int64_t bh = (int64_t)b * a.heads + h;
  u32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * NT;
    const int64_t n = blk0 * 64 + c / CPR;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (n < N) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v + ((int64_t)b * N + n) * rs + (int64_t)h * D + (c % CPR) * 8));
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * NT;
    const int r = c / CPR, col = c % CPR;
    *reinterpret_cast<u32x4*>(&tile[r * 64 + ((4 * col) ^ vq_swizzle(r))]) = v[i];
  }
  __syncthreads();
  // one (channel pair, 16-byte segment) per thread; lanes PARTS p .. PARTS p + PARTS-1 write
  // consecutive segments of the same two v8t rows
  const int part = threadIdx.x % PARTS, pair = threadIdx.x / PARTS;
  const int bs = part >> 2, hl = (part >> 1) & 1, m = part & 1;  // segment = 4 bs + 2 hl + m
  if (blk0 + bs >= a.n_blocks) return;
  const int2 ex = *reinterpret_cast<const int2*>(a.v_exp + bh * D + 2 * pair);
  u32x4 o0, o1;
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) {
    float f0[4], f1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kappa = 64 * bs + 32 * m + 8 * a4 + 4 * hl + r;  // the key of slot 16 (2 hl + m) + 4 a4 + r
      const uint32_t w = tile[kappa * 64 + (pair ^ vq_swizzle(kappa))];
      f0[r] = ldexpf(bf16_lo(w), -ex.x);  // exact: the scales are powers of two
      f1[r] = ldexpf(bf16_hi(w), -ex.y);
    }
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f0[0], f0[1], 0, false);
    o0[a4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f0[2], f0[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f1[0], f1[1], 0, false);
    o1[a4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f1[2], f1[3], w1, true);
  }
  const int64_t np = (int64_t)a.n_blocks * 64;
  uint8_t* row = a.v8t + (bh * D + 2 * pair) * np + blk0 * 64 + part * 16;
  *reinterpret_cast<u32x4*>(row) = o0;
  *reinterpret_cast<u32x4*>(row + np) = o1;
}

template <int D>
void launch_all(const Fp8QuantArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(qk_quant_kernel<D>, dim3((unsigned)a.n_blocks * a.heads, 1, (unsigned)(2 * a.batch)),
                     dim3(kQThreads), 0, stream, a);
  hipLaunchKernelGGL(v_amax_kernel<D>, dim3((unsigned)a.n_chunks, (unsigned)a.heads, (unsigned)a.batch),
                     dim3(kQThreads), 0, stream, a);
  hipLaunchKernelGGL(v_scale_kernel<D>, dim3((unsigned)a.heads, (unsigned)a.batch), dim3(1024), 0, stream, a);
  hipLaunchKernelGGL((v_quant_kernel<D, kVBlocks>), dim3((unsigned)((a.n_blocks + kVBlocks - 1) / kVBlocks) * a.heads, 1, (unsigned)a.batch),
                     dim3(2 * D * kVBlocks), 0, stream, a);
}

}  // namespace

void launch_fp8_quantize(const Fp8QuantArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_all<128>(a, stream);
  else launch_all<64>(a, stream);
}

}  // namespace h3attn
