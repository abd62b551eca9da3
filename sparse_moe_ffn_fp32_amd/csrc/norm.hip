// Pre-MoE RMSNorm of the decoder block: t = bf16(x / sqrt(mean(x^2) + eps)
// * scale) per token ("gpt-oss-20b" page, "Structure": RMSNorm_i_2 feeds
// MoE_i; rms_norm_eps from the raw config.json tables). The tiled expert
// GEMMs copy activation rows into LDS by DMA, so the normed rows are written
// once here (5,760 bytes per token) rather than recomputed by every reader.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kNormRowVec = kH / 8;                  // 360 16-byte vectors per row
constexpr int kNormPerLane = (kNormRowVec + 63) / 64;   // 6

// One wave per row, four rows per 256-thread block. The sum of squares is
// reduced in a fixed order (per lane, then a butterfly), so results are
// reproducible run to run.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ scale, float eps,
                                                      int T, uint16_t* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * kH);
  float v[kNormPerLane][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormPerLane; ++j) {
    const int i = lane + 64 * j;
    uint4 d = make_uint4(0u, 0u, 0u, 0u);
    if (i < kNormRowVec) d = xr[i];
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[j][2 * q] = bf16_bits_to_f32(dw[q] & 0xFFFFu);
      v[j][2 * q + 1] = bf16_bits_to_f32(dw[q] >> 16);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ss = fmaf(v[j][q], v[j][q], ss);
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) ss += __shfl_xor(ss, d, 64);
  const float inv = 1.0f / sqrtf(ss / (float)kH + eps);
  uint4* tr = reinterpret_cast<uint4*>(t + row * kH);
  const float4* sc = reinterpret_cast<const float4*>(scale);
#pragma unroll
  for (int j = 0; j < kNormPerLane; ++j) {
    const int i = lane + 64 * j;
    if (i >= kNormRowVec) break;
    const float4 s0 = sc[2 * i], s1 = sc[2 * i + 1];
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = f32_to_bf16_bits(v[j][2 * q] * inv * s[2 * q]) |
             (f32_to_bf16_bits(v[j][2 * q + 1] * inv * s[2 * q + 1]) << 16);
    tr[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* scale, float eps, int T, uint16_t* t,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, scale, eps,
                     T, t);
  return hipGetLastError();
}

}  // namespace moe
