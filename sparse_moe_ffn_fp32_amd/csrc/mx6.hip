// Activation encoder of the block-scaled matrix-core path: bf16 rows ->
// two-piece MX FP6 (E2M3) records (layout in moe_device.h). The pieces are
// the OCP MX v1.0 conversion of each 32-value block and of its exact residual.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kVBlocks = kSteps * 4;   // 92: the 90 MX blocks of a row + 2 zero pads

// One thread per (row, MX block), blocks of a row consecutive across threads.
__global__ __launch_bounds__(256) void mx6_encode_kernel(const uint16_t* __restrict__ x,
                                                         long long units,
                                                         uint8_t* __restrict__ rec) {
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const long long row = u / kVBlocks;
  const int vb = (int)(u - row * kVBlocks);
  const int s = vb >> 2, g = vb & 3;
  uint32_t w1[6], w2[6], s1 = 127u, s2 = 127u;
#pragma unroll
  for (int i = 0; i < 6; ++i) w1[i] = w2[i] = 0u;
  if (vb < kKB) {
    float v[32];
    const uint4* src = reinterpret_cast<const uint4*>(x + row * kH + vb * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 d = src[q];
      const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = bf16_bits_to_f32(dw[i] & 0xFFFFu);
        v[8 * q + 2 * i + 1] = bf16_bits_to_f32(dw[i] >> 16);
      }
    }
    mx6x2_encode(v, w1, s1, w2, s2);
  }
  uint8_t* r = rec + (row * kSteps + s) * kRecBytes;
  *reinterpret_cast<uint4*>(r + g * 16) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
  *reinterpret_cast<uint4*>(r + (4 + g) * 16) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
  *reinterpret_cast<uint2*>(r + (8 + (g >> 1)) * 16 + (g & 1) * 8) = make_uint2(w1[4], w1[5]);
  *reinterpret_cast<uint2*>(r + (10 + (g >> 1)) * 16 + (g & 1) * 8) = make_uint2(w2[4], w2[5]);
  *reinterpret_cast<uint16_t*>(r + 12 * 16 + 2 * g) = (uint16_t)(s1 | (s2 << 8));
  if (g == 0) {
    *reinterpret_cast<uint2*>(r + 12 * 16 + 8) = make_uint2(0u, 0u);
#pragma unroll
    for (int i = 13; i < 16; ++i) *reinterpret_cast<uint4*>(r + i * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
}

hipError_t launch_mx6_encode(const uint16_t* x, int rows, uint8_t* rec, hipStream_t s) {
  const long long units = (long long)rows * kVBlocks;
  if (units == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  hipLaunchKernelGGL(mx6_encode_kernel, dim3(blocks), dim3(256), 0, s, x, units, rec);
  return hipGetLastError();
}

// Range of each expert's E8M0 scale bytes (the NaN byte 255 excluded), for
// the accuracy limit of the FP6-piece path: lohi[2e] = smallest byte,
// lohi[2e + 1] = largest (255 and 0 when the expert has none).
__global__ __launch_bounds__(256) void scale_range_init_kernel(int E, int32_t* __restrict__ lohi) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) {
    lohi[2 * e] = 255;
    lohi[2 * e + 1] = 0;
  }
}

__global__ __launch_bounds__(256) void scale_range_kernel(const uint8_t* __restrict__ scales,
                                                          long long per_expert,
                                                          int32_t* __restrict__ lohi) {
  const int e = blockIdx.y;
  const uint8_t* p = scales + (size_t)e * per_expert;
  int lo = 255, hi = 0;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < per_expert;
       i += (long long)gridDim.x * 256) {
    const int b = p[i];
    if (b != 255) {
      lo = min(lo, b);
      hi = max(hi, b);
    }
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    lo = min(lo, __shfl_xor(lo, d, 64));
    hi = max(hi, __shfl_xor(hi, d, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMin(&lohi[2 * e], lo);
    atomicMax(&lohi[2 * e + 1], hi);
  }
}

hipError_t launch_scale_range(const uint8_t* scales, int E, int N, int32_t* lohi, hipStream_t s) {
  hipLaunchKernelGGL(scale_range_init_kernel, dim3((E + 255) / 256), dim3(256), 0, s, E, lohi);
  hipLaunchKernelGGL(scale_range_kernel, dim3(16, E), dim3(256), 0, s, scales, (long long)N * kKB, lohi);
  return hipGetLastError();
}

}  // namespace moe
