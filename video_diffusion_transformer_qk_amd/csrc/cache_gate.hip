// Cache-DiT residual-change gate for gfx950: reduction kernel and host-side reuse policy.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section
// "6.24 倍里，真正有损的部分大约是三倍": Cache-DiT compares the residual change between adjacent
// denoising steps and, when it is small, reuses cached middle-block results; the conservative
// setting uses a tighter threshold and caches at most one step in a row, the stride setting a
// looser threshold and at most three.
//
// residual_partial_kernel: each workgroup reduces a contiguous range of 16-byte chunks of cur and
//   prev into (sum |cur - prev|, sum |prev|): float32 per thread (a few hundred terms), float64
//   across the workgroup, one pair per workgroup in the workspace. HBM-bound: both tensors are
//   read once with nontemporal loads.
// residual_final_kernel: one workgroup adds the per-workgroup pairs in a fixed order, so the
//   result is deterministic run to run.
#include <mutex>

#include "device_util.h"
#include "kernels.h"

namespace h3attn {
namespace {

constexpr int kRedThreads = 256;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(kRedThreads) void residual_partial_kernel(ResidualArgs a) {
  __shared__ double red[kRedThreads / 64];
  const int64_t chunks = a.n / 8;
  const int64_t c0 = (int64_t)blockIdx.x * a.chunks_per_block;
  const int64_t c1 = c0 + a.chunks_per_block < chunks ? c0 + a.chunks_per_block : chunks;
  float sd = 0.f, sp = 0.f;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += kRedThreads) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.cur + 8 * c));
    const u32x4 y = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.prev + 8 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sd += fabsf(bf16_lo(x[j]) - bf16_lo(y[j])) + fabsf(bf16_hi(x[j]) - bf16_hi(y[j]));
      sp += fabsf(bf16_lo(y[j])) + fabsf(bf16_hi(y[j]));
    }
  }
  // the tail of a length that is not a multiple of 8 goes to the last workgroup
  if (blockIdx.x == gridDim.x - 1) {
    for (int64_t e = chunks * 8 + threadIdx.x; e < a.n; e += kRedThreads) {
      const float x = __uint_as_float((uint32_t)a.cur[e] << 16), y = __uint_as_float((uint32_t)a.prev[e] << 16);
      sd += fabsf(x - y);
      sp += fabsf(y);
    }
  }
  const double d = block_sum_f64((double)sd, red);
  const double p = block_sum_f64((double)sp, red);
  if (threadIdx.x == 0) {
    a.partial[2 * blockIdx.x] = d;
    a.partial[2 * blockIdx.x + 1] = p;
  }
}

__global__ __launch_bounds__(kRedThreads) void residual_final_kernel(ResidualArgs a, int n_parts) {
  __shared__ double red[kRedThreads / 64];
  double d = 0.0, p = 0.0;
  for (int i = threadIdx.x; i < n_parts; i += kRedThreads) {
    d += a.partial[2 * i];
    p += a.partial[2 * i + 1];
  }
  d = block_sum_f64(d, red);
  p = block_sum_f64(p, red);
  if (threadIdx.x == 0) {
    a.result[0] = d;
    a.result[1] = p;
  }
}

// Partial sums of h3attn_residual_change_noalloc. Every GPU the library runs on holds its own copy
// until the process ends; calls on one GPU share it, so calls that overlap on one GPU race.
static __device__ __align__(256) double scratch[2 * kResidualNoAllocParts];

}  // namespace

double* residual_noalloc_scratch() {
  // one lookup per device, with that device current; the array's host-side name is not a device
  // address, so only the looked-up pointer is ever handed to kernels
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static double* ptr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = static_cast<double*>(p);
  }
  return ptr[dev];
}

int residual_parts(int64_t n) {
  const int64_t chunks = (n + 7) / 8;
  int64_t parts = (chunks + kResidualChunksPerBlock - 1) / kResidualChunksPerBlock;
  return (int)(parts < 1 ? 1 : parts);
}

void launch_residual_change(const ResidualArgs& a0, hipStream_t stream) {
  ResidualArgs a = a0;
  const int parts = residual_parts(a.n);
  a.chunks_per_block = kResidualChunksPerBlock;
  hipLaunchKernelGGL(residual_partial_kernel, dim3((unsigned)parts), dim3(kRedThreads), 0, stream, a);
  hipLaunchKernelGGL(residual_final_kernel, dim3(1), dim3(kRedThreads), 0, stream, a, parts);
}

}  // namespace h3attn
