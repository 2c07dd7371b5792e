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
//         maxima) -> v_scale_kernel (fixed-order reduce) -> v_quant_kernel, which also transposes
//         each 64-key block to [channel][key slot] for the P.V product.
// All four are HBM-bound streams.
#include "device_util.h"
#include "kernels.h"

namespace h3attn {
namespace {

constexpr int kQThreads = 256;

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

// grid (nB, heads, 2 * batch): blockIdx.z = 2 * b + (0: q, 1: k)
template <int D>
__global__ __launch_bounds__(kQThreads) void qk_quant_kernel(Fp8QuantArgs a) {
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int PER = 64 * CPR / kQThreads;  // chunks per thread
  __shared__ float red[kQThreads / 64];
  const int t = blockIdx.z & 1, b = blockIdx.z >> 1, h = blockIdx.y;
  const int64_t blk = blockIdx.x, N = a.n_tokens;
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
    if (n < N) v[i] = *reinterpret_cast<const u32x4*>(x + ((int64_t)b * N + n) * rs + (int64_t)h * D + (c % CPR) * 8);
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
      *reinterpret_cast<u32x2*>(x8 + ((int64_t)b * N + n) * rs + (int64_t)h * D + (c % CPR) * 8) = to_e4m3x8(f);
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

// grid (heads, batch), D threads: the channel scales
template <int D>
__global__ __launch_bounds__(D) void v_scale_kernel(Fp8QuantArgs a) {
  const int64_t bh = (int64_t)blockIdx.y * a.heads + blockIdx.x;
  float mx = 0.f;
  for (int c = 0; c < a.n_chunks; ++c) mx = fmaxf(mx, a.v_partial[(bh * a.n_chunks + c) * D + threadIdx.x]);
  const int e = mx > 0.f ? pow2_exponent(mx) : 0;
  a.v_exp[bh * D + threadIdx.x] = e;
  a.v_scale[bh * D + threadIdx.x] = ldexpf(1.0f, e);
}

// slot of key kappa (0..63) inside its block's 64 bytes of a v8t row. The P.V product takes P^T
// as its B operand straight from the score registers: lane half hl holds, as bytes j = 16m + r
// (score sub-tile m, accumulator register r), the keys 32m + 8(r/4) + 4hl + r%4; the A operand
// (V^T) of lane half hl reads bytes [32hl, 32hl + 32) of a row, so key kappa goes to
// 32hl + 16m + 4(r/4) + r%4.
__device__ __forceinline__ int fp8_key_slot(int kappa) {
  const int m = kappa >> 5, a4 = (kappa >> 3) & 3, hl = (kappa >> 2) & 1, r = kappa & 3;
  return 32 * hl + 16 * m + 4 * a4 + r;
}

// grid (nB, heads, batch): quantise one 64-token block of v and write it transposed
template <int D>
__global__ __launch_bounds__(kQThreads) void v_quant_kernel(Fp8QuantArgs a) {
  constexpr int CPR = D / 8;
  constexpr int PER = 64 * CPR / kQThreads;
  __shared__ __attribute__((aligned(16))) uint8_t tile[D][64];
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t blk = blockIdx.x, N = a.n_tokens, rs = (int64_t)a.heads * D;
  const int64_t bh = (int64_t)b * a.heads + h;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = threadIdx.x + i * kQThreads;
    const int r = c / CPR, col = c % CPR;
    const int64_t n = blk * 64 + r;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (n < N) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v + ((int64_t)b * N + n) * rs + (int64_t)h * D + col * 8));
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // exact: the scales are powers of two
      f[2 * j] = ldexpf(bf16_lo(v[j]), -a.v_exp[bh * D + col * 8 + 2 * j]);
      f[2 * j + 1] = ldexpf(bf16_hi(v[j]), -a.v_exp[bh * D + col * 8 + 2 * j + 1]);
    }
    const u32x2 w = to_e4m3x8(f);
    const int slot = fp8_key_slot(r);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[col * 8 + j][slot] = (uint8_t)(w[j / 4] >> (8 * (j % 4)));
  }
  __syncthreads();
  const int64_t np = (int64_t)a.n_blocks * 64;
#pragma unroll
  for (int i = 0; i < D * 4 / kQThreads; ++i) {
    const int seg = threadIdx.x + i * kQThreads;
    const int d = seg >> 2, part = seg & 3;
    *reinterpret_cast<u32x4*>(a.v8t + (bh * D + d) * np + blk * 64 + part * 16) =
        *reinterpret_cast<const u32x4*>(&tile[d][part * 16]);
  }
}

template <int D>
void launch_all(const Fp8QuantArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(qk_quant_kernel<D>, dim3((unsigned)a.n_blocks, (unsigned)a.heads, (unsigned)(2 * a.batch)),
                     dim3(kQThreads), 0, stream, a);
  hipLaunchKernelGGL(v_amax_kernel<D>, dim3((unsigned)a.n_chunks, (unsigned)a.heads, (unsigned)a.batch),
                     dim3(kQThreads), 0, stream, a);
  hipLaunchKernelGGL(v_scale_kernel<D>, dim3((unsigned)a.heads, (unsigned)a.batch), dim3(D), 0, stream, a);
  hipLaunchKernelGGL(v_quant_kernel<D>, dim3((unsigned)a.n_blocks, (unsigned)a.heads, (unsigned)a.batch),
                     dim3(kQThreads), 0, stream, a);
}

}  // namespace

void launch_fp8_quantize(const Fp8QuantArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) launch_all<128>(a, stream);
  else launch_all<64>(a, stream);
}

}  // namespace h3attn
