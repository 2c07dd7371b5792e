// SubBlock key-block selection for gfx950: block pooling, block scores, per-row top-k.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section
// "6.24 倍里，真正有损的部分大约是三倍": queries and keys are cut into 64-token blocks, the key
// blocks that would contribute little are estimated and dropped, and the fraction dropped is
// the sparsity. The pages leave the estimator open; this library scores key block j for query
// block i by mean(q over block i) . mean(k over block j) and keeps the keep highest per row,
// equal scores ranking the lower key index first, indices written in ascending order.
//
// Exactness: block sums of bf16 values are exact in float64, and the 1/sqrt(D) scale is
// dropped (a positive factor does not change the order), so the GPU ranks by a float64 dot
// product of the same means the float64 definition uses; the top-k itself is an exact radix
// select over order-preserving 64-bit keys.
//
// Kernels:
//  pool_kernel   grid (heads * nB, 1, batch): 256 threads, 16-byte coalesced row reads (all
//                issued before the sums), fp64 sums reduced through LDS in a fixed order ->
//                means [B, H, nB, D] for q and k.
//  score_kernel  grid (ceil(nB/T), ceil(nB/T), B*H), T = 64 or 128: a T x T tile of Qm . Km^T on
//                the fp64 MFMA (v_mfma_f64_16x16x4f64), D staged through LDS in chunks of 32.
//  topk_kernel   grid (nB, heads, batch): one row of nB scores -> LDS keys -> 8-pass MSB radix
//                select of the keep-th largest key -> ordered compaction of the kept indices.
#include "device_util.h"
#include "kernels.h"
#include "launch_util.h"

namespace h3attn {
namespace {

constexpr int kPoolThreads = 256;

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(SelectArgs a) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int PAIRS = 2 * CH;        // (tensor, chunk) pairs
  constexpr int TL = kPoolThreads / PAIRS;  // token lanes
  __shared__ double red[TL][PAIRS][8];

  const int tid = threadIdx.x;
  const int pair = tid % PAIRS;
  const int tl = tid / PAIRS;
  const int tensor = pair / CH;
  const int chunk = pair % CH;
  const int head = (int)(blockIdx.x % (unsigned)a.heads), j = (int)(blockIdx.x / (unsigned)a.heads), b = blockIdx.z;
  const int64_t N = a.n_tokens;
  const int64_t row_stride = (int64_t)a.heads * D;
  const int64_t t0 = (int64_t)j * a.block_size;
  const int64_t t1 = t0 + a.block_size < N ? t0 + a.block_size : N;
  const uint16_t* src = (tensor == 0 ? a.q : a.k) + ((int64_t)b * N) * row_stride + (int64_t)head * D + chunk * 8;

  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int R = 64 / TL;  // rows per thread: blocks are 64 tokens (the entry points accept no other size)
  u32x4 w[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t t = t0 + tl + (int64_t)i * TL;
    w[i] = u32x4{0u, 0u, 0u, 0u};
    if (t < t1) w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + t * row_stride));
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (t0 + tl + (int64_t)i * TL >= t1) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_lo(w[i][e]);
      acc[2 * e + 1] += (double)bf16_hi(w[i][e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl][pair][e] = acc[e];
  __syncthreads();
  // tl == 0 lanes finish the sum in a fixed order and write the mean
  if (tl == 0) {
    const double cnt = (double)(t1 - t0);
    double* dst = (tensor == 0 ? a.q_mean : a.k_mean) + (((int64_t)b * a.heads + head) * a.n_blocks + j) * D + chunk * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double s = 0.0;
      for (int u = 0; u < TL; ++u) s += red[u][pair][e];
      dst[e] = s / cnt;
    }
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Qm . Km^T on the fp64 matrix cores. v_mfma_f64_16x16x4f64 takes A[i][k] from lane i + 16k and
// B[k][j] from lane j + 16k, and returns D[4r + l/16][l%16] in register r of lane l. A workgroup
// of 4 waves computes a TILE x TILE block of scores, each wave a (TILE/2)^2 quarter as
// (TILE/32)^2 16x16 tiles. Both operands are staged through LDS as [row][d] with a row stride of
// DC + 4 doubles, so the 16 rows x 4 k of an operand read fall in 2 passes over the 64 banks.
template <int D, int TILE, int DC>
__global__ __launch_bounds__(256) void score_kernel(SelectArgs a) {
  constexpr int LD = DC + 4;
  constexpr int RT = TILE / 32;  // 16x16 tiles per wave per dimension
  __shared__ __attribute__((aligned(16))) double qs[TILE * LD];
  __shared__ __attribute__((aligned(16))) double ks[TILE * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kq = lane >> 4;
  const int64_t bh = blockIdx.z;
  const int nb = a.n_blocks;
  const int i0 = blockIdx.y * TILE, j0 = blockIdx.x * TILE;
  const int rb = (wave >> 1) * (TILE / 2), cb = (wave & 1) * (TILE / 2);
  const double* qm = a.q_mean + bh * (int64_t)nb * D;
  const double* km = a.k_mean + bh * (int64_t)nb * D;
  f64x4 acc[RT][RT];
#pragma unroll
  for (int u = 0; u < RT; ++u)
#pragma unroll
    for (int w = 0; w < RT; ++w) acc[u][w] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int dc = 0; dc < D; dc += DC) {
    // stage TILE x DC of Qm and Km, 16 bytes per thread and step (rows past nb repeat the last)
#pragma unroll
    for (int e = tid; e < TILE * DC / 2; e += 256) {
      const int r = e / (DC / 2), c2 = e % (DC / 2);
      const int qi = i0 + r < nb ? i0 + r : nb - 1;
      const int kj = j0 + r < nb ? j0 + r : nb - 1;
      *reinterpret_cast<double2*>(&qs[r * LD + 2 * c2]) = *reinterpret_cast<const double2*>(qm + (int64_t)qi * D + dc + 2 * c2);
      *reinterpret_cast<double2*>(&ks[r * LD + 2 * c2]) = *reinterpret_cast<const double2*>(km + (int64_t)kj * D + dc + 2 * c2);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < DC / 4; ++kk) {
      double av[RT], bv[RT];
#pragma unroll
      for (int u = 0; u < RT; ++u) {
        av[u] = qs[(rb + 16 * u + l16) * LD + 4 * kk + kq];
        bv[u] = ks[(cb + 16 * u + l16) * LD + 4 * kk + kq];
      }
#pragma unroll
      for (int u = 0; u < RT; ++u)
#pragma unroll
        for (int w = 0; w < RT; ++w) acc[u][w] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u], bv[w], acc[u][w], 0, 0, 0);
    }
    __syncthreads();
  }
  double* out = a.scores + bh * (int64_t)nb * nb;
#pragma unroll
  for (int u = 0; u < RT; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + rb + 16 * u + 4 * r + kq;
      if (i >= nb) continue;
#pragma unroll
      for (int w = 0; w < RT; ++w) {
        const int j = j0 + cb + 16 * w + l16;
        if (j < nb) __builtin_nontemporal_store(acc[u][w][r], out + (int64_t)i * nb + j);
      }
    }
}

// order-preserving map of a double to uint64 (larger double -> larger key); -0 is folded to +0
__device__ __forceinline__ uint64_t order_key(double x) {
  x = x + 0.0;  // -0.0 + 0.0 = +0.0 under round-to-nearest
  const uint64_t u = __double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kTopkThreads = 256;
static_assert(kTopkThreads == 256, "one histogram bin per thread");

// Calls f(j, row[j]) for this thread's j = tid, tid + 256, ... < n, issuing 8 loads at a time so
// that a thread has several in flight (a plain loop waits for each load before the next).
template <typename F>
__device__ __forceinline__ void for_row(const double* row, int n, F f) {
  for (int j0 = threadIdx.x; j0 < n; j0 += 8 * kTopkThreads) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kTopkThreads;
      v[u] = j < n ? __builtin_nontemporal_load(row + j) : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * kTopkThreads;
      if (j < n) f(j, v[u]);
    }
  }
}

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
  for (int w = 0; w < kTopkThreads / 64; ++w) {
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
  const int per = (nb + kTopkThreads - 1) / kTopkThreads;
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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);
  __shared__ uint32_t hist[256];
  __shared__ int scan_scratch[4];
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_krem, sh_done;

  const int tid = threadIdx.x;
  const int nb = a.n_blocks;
  const int i = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int64_t row = ((int64_t)b * a.heads + head) * nb + i;
  const double* sc = a.scores + row * nb;
  for_row(sc, nb, [&](int j, double x) { keys[j] = order_key(x); });

  // Digit by digit from the top: the 8-bit digit of the keep-th largest key is the bin where the
  // count of keys in higher bins first reaches k_rem (thread t owns bin 255 - t, so a block
  // prefix sum gives every bin the count above it and exactly one thread finds the digit). The
  // select stops early once the chosen bin holds exactly the k_rem keys still wanted: all of
  // them are kept, so the remaining digits cannot change the kept set.
  uint64_t prefix = 0, mask = 0;
  int k_rem = a.keep;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nb; j += kTopkThreads) {
      const uint64_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int d = 255 - tid;
    const int h = (int)hist[d];
    int tot;
    const int above = block_exclusive_scan(h, &tot, scan_scratch);  // keys in the bins above d
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

  // keys whose top digits exceed the prefix are kept, plus k_rem of those equal to it
  ordered_compact(keys, nb, prefix, mask, k_rem, a.block_idx + row * a.keep, a.keep, scan_scratch);
}

// Threshold mode, pass 1: per row, the largest unscaled score m and the kept count
// #{j : s_j >= m - tau*sqrt(D)}; the threshold is stored so that pass 2 uses the same value.
__global__ __launch_bounds__(kTopkThreads) void threshold_count_kernel(SelectArgs a) {
  __shared__ double red[kTopkThreads / 64];
  __shared__ int cnt_red[kTopkThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = a.n_blocks;
  const int64_t row = ((int64_t)blockIdx.z * a.heads + blockIdx.y) * nb + blockIdx.x;
  // the row is read once, into LDS, and counted from there
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* sc = reinterpret_cast<double*>(smem);
  double m = -INFINITY;
  for_row(a.scores + row * nb, nb, [&](int j, double x) {
    sc[j] = x;
    m = fmax(m, x);
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / 64; ++w) m = fmax(m, red[w]);
  const double thr = m - a.tau_raw;
  int c = 0;
  for (int j = tid; j < nb; j += kTopkThreads) c += sc[j] >= thr;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if (lane == 0) cnt_red[wave] = c;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) tot += cnt_red[w];
    a.row_cnt[row] = tot;
    a.row_thr[row] = thr;
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

// Threshold mode, pass 2: ordered compaction of {j : s_j >= thr} into col_idx[row_ptr[row] ..].
// Writes past col_capacity are dropped (the caller sizes col_idx from row_ptr's last entry).
__global__ __launch_bounds__(kTopkThreads) void threshold_fill_kernel(SelectArgs a) {
  __shared__ int scan_scratch[4];
  const int tid = threadIdx.x;
  const int nb = a.n_blocks;
  const int64_t row = ((int64_t)blockIdx.z * a.heads + blockIdx.y) * nb + blockIdx.x;
  // the row is staged in LDS with coalesced loads; the ordered scans below walk contiguous runs
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  double* sc = reinterpret_cast<double*>(smem);
  for_row(a.scores + row * nb, nb, [&](int j, double x) { sc[j] = x; });
  __syncthreads();
  const double thr = a.row_thr[row];
  const int64_t start = a.row_ptr[row];
  const int per = (nb + kTopkThreads - 1) / kTopkThreads;
  const int j0 = tid * per;
  const int j1 = j0 + per < nb ? j0 + per : nb;
  int n_sel = 0;
  for (int j = j0; j < j1; ++j) n_sel += sc[j] >= thr;
  int tot;
  int64_t p = start + block_exclusive_scan(n_sel, &tot, scan_scratch);
  for (int j = j0; j < j1; ++j)
    if (sc[j] >= thr) {
      if (p < a.col_capacity) a.col_idx[p] = j;
      ++p;
    }
}

}  // namespace

static void launch_pool_and_scores(const SelectArgs& a, hipStream_t stream);

void launch_subblock_select(const SelectArgs& a, hipStream_t stream) {
  launch_pool_and_scores(a, stream);
  const dim3 g3((unsigned)a.n_blocks, (unsigned)a.heads, (unsigned)a.batch);
  const size_t lds = (size_t)a.n_blocks * sizeof(uint64_t);
  allow_dynamic_lds(reinterpret_cast<const void*>(topk_kernel), (int)kSelectRowLdsBytes);
  hipLaunchKernelGGL(topk_kernel, g3, dim3(kTopkThreads), lds, stream, a);
}

template <int TILE>
void launch_scores(const SelectArgs& a, hipStream_t stream) {
  const unsigned tiles = (unsigned)((a.n_blocks + TILE - 1) / TILE);
  const dim3 gs(tiles, tiles, (unsigned)(a.batch * a.heads));
  if (a.head_dim == 128) hipLaunchKernelGGL((score_kernel<128, TILE, 32>), gs, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((score_kernel<64, TILE, 32>), gs, dim3(256), 0, stream, a);
}

static void launch_pool_and_scores(const SelectArgs& a, hipStream_t stream) {
  const dim3 g3((unsigned)a.n_blocks * (unsigned)a.heads, 1, (unsigned)a.batch);
  if (a.head_dim == 128) hipLaunchKernelGGL(pool_kernel<128>, g3, dim3(kPoolThreads), 0, stream, a);
  else hipLaunchKernelGGL(pool_kernel<64>, g3, dim3(kPoolThreads), 0, stream, a);
  // 128 x 128 score tiles once there are enough of them (half the operand staging per score);
  // 64 x 64 for short rows, where 128-wide tiles leave most of the chip idle
  if (a.n_blocks >= 1024) launch_scores<128>(a, stream);
  else launch_scores<64>(a, stream);
}

void launch_threshold_count(const SelectArgs& a, hipStream_t stream) {
  launch_pool_and_scores(a, stream);
  const dim3 g3((unsigned)a.n_blocks, (unsigned)a.heads, (unsigned)a.batch);
  allow_dynamic_lds(reinterpret_cast<const void*>(threshold_count_kernel), (int)kSelectRowLdsBytes);
  hipLaunchKernelGGL(threshold_count_kernel, g3, dim3(kTopkThreads), (size_t)a.n_blocks * sizeof(double), stream, a);
  const int64_t rows = (int64_t)a.batch * a.heads * a.n_blocks;
  hipLaunchKernelGGL(row_ptr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a, rows);
}

void launch_threshold_fill(const SelectArgs& a, hipStream_t stream) {
  const dim3 g3((unsigned)a.n_blocks, (unsigned)a.heads, (unsigned)a.batch);
  const size_t lds = (size_t)a.n_blocks * sizeof(double);
  allow_dynamic_lds(reinterpret_cast<const void*>(threshold_fill_kernel), (int)kSelectRowLdsBytes);
  hipLaunchKernelGGL(threshold_fill_kernel, g3, dim3(kTopkThreads), lds, stream, a);
}

}  // namespace h3attn
