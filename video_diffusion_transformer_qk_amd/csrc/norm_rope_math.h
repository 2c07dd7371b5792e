// QK RMSNorm + 3D RoPE arithmetic of one 16-byte chunk (8 channels) of one head row, shared by the
// stand-alone kernel (qk_norm_rope.hip) and the kernel that also pools the result into SubBlock
// block means (subblock_select.hip), so that both write the same bits.
//
// Source: "MiniMax-H3 的 6.24 倍，不能直接算成六倍产能" (xiaodao.ai), section "先把近两倍的免费收益拿
// 走": QK RMSNorm and 3D RoPE as one fused pass.
#pragma once

#include "device_util.h"
#include "kernels.h"

namespace h3attn {

// Grid coordinates (t, h, w) of token n of a T x H x W latent (n = (t*H + h)*W + w).
__device__ __forceinline__ void rope_position(int64_t n, int32_t grid_h, int32_t grid_w, int64_t (&pos)[3]) {
  const int64_t hw = (int64_t)grid_h * grid_w;
  pos[0] = n / hw;
  pos[1] = (n / grid_w) % grid_h;
  pos[2] = n % grid_w;
}

// cos and sin of the rotation angle of channel pair `pair` at grid position pos: the angle
// position x rate in double, reduced to [-pi, pi] in double so the float sincos stays on its
// accurate short path.
__device__ __forceinline__ void rope_pair(const int64_t (&pos)[3], int pair, const RopeTable& tab, float& cs,
                                          float& sn) {
  const double ang = (double)pos[tab.axis[pair]] * tab.rate[pair];
  const double turns = rint(ang * 0.15915494309189535);  // 1/(2 pi)
  const float red = (float)fma(-turns, 6.283185307179586, ang);
  sincosf(red, &sn, &cs);
}

// RMSNorm of the row (the sum of squares reduced over the TPR = D/8 lanes that hold it, which
// must all be active), times the channel weights w, then the rotation of the chunk's four channel
// pairs by (cs[p], sn[p]); rounded to bf16.
template <int TPR>
__device__ __forceinline__ u32x4 norm_rope_chunk(const u32x4 x, const float (&w)[8], const float (&cs)[4],
                                                 const float (&sn)[4], float inv_d, float eps) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(x[j]); v[2 * j + 1] = bf16_hi(x[j]); }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, TPR);
  const float rs = rsqrtf(fmaf(ss, inv_d, eps));
  u32x4 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float y0 = v[2 * p] * rs * w[2 * p];
    const float y1 = v[2 * p + 1] * rs * w[2 * p + 1];
    const float z0 = fmaf(y0, cs[p], -y1 * sn[p]);
    const float z1 = fmaf(y0, sn[p], y1 * cs[p]);
    o[p] = pack_bf16x2(z0, z1);
  }
  return o;
}

}  // namespace h3attn
