// Pre-MoE RMSNorm of the decoder block: t = bf16(x / sqrt(mean(x^2) + eps)
// * scale) per token ("gpt-oss-20b" page, "Structure": RMSNorm_i_2 feeds
// MoE_i; rms_norm_eps from the raw config.json tables). The tiled expert
// GEMMs copy activation rows into LDS by DMA, so the normed rows are written
// once here (5,760 bytes per token) rather than recomputed by every reader.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// One wave per bf16 row of kH values, lane l holding 16-byte vectors l,
// l + 64, ...
constexpr int kNormRowVec = kH / 8;                      // 360 16-byte vectors per row
constexpr int kNormPerLane = (kNormRowVec + 63) / 64;    // 6

// the lane's raw vectors of a row (zero past the row's end)
__device__ __forceinline__ void norm_load_raw(const uint16_t* row, int lane,
                                              uint4 (&d)[kNormPerLane]) {
  const uint4* xr = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int j = 0; j < kNormPerLane; ++j) {
    const int i = lane + 64 * j;
    d[j] = make_uint4(0u, 0u, 0u, 0u);
    if (i < kNormRowVec) d[j] = xr[i];
  }
}

// 1 / sqrt(mean(x^2) + eps) of the row from the lane's raw vectors: the
// squares are summed per lane by bf16 dot-2 instructions (fp32 accumulate)
// into four partial sums, one per dword position, added in a fixed order,
// then a butterfly over the 64 lanes adds the lanes' sums; every lane gets
// the result.
__device__ __forceinline__ float norm_inv_rms(const uint4 (&d)[kNormPerLane], float eps) {
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kNormPerLane; ++j) {
    const uint32_t dw[4] = {d[j].x, d[j].y, d[j].z, d[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 v = __builtin_bit_cast(bf16x2, dw[q]);
      ss[q] = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss[q], false);
    }
  }
  float t = (ss[0] + ss[1]) + (ss[2] + ss[3]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) t += __shfl_xor(t, m, 64);
  return 1.0f / sqrtf(t / (float)kH + eps);
}

// One wave per row, four rows per 256-thread block. The sum of squares is
// reduced in a fixed order (per lane, then a butterfly), so results are
// reproducible run to run.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ scale, float eps,
                                                      int T, uint16_t* __restrict__ t,
                                                      float* __restrict__ inv_out) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  uint4 d[kNormPerLane];
  norm_load_raw(x + row * kH, lane, d);
  const float inv = norm_inv_rms(d, eps);
  if (inv_out && lane == 0) inv_out[row] = inv;
  uint4* tr = reinterpret_cast<uint4*>(t + row * kH);
  const float4* sc = reinterpret_cast<const float4*>(scale);
#pragma unroll
  for (int j = 0; j < kNormPerLane; ++j) {
    const int i = lane + 64 * j;
    if (i >= kNormRowVec) break;
    tr[i] = norm_apply8(d[j], inv, sc[2 * i], sc[2 * i + 1]);
  }
}

hipError_t launch_rmsnorm(const uint16_t* x, const float* scale, float eps, int T, uint16_t* t,
                          float* inv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, scale, eps,
                     T, t, inv);
  return hipGetLastError();
}

}  // namespace moe
