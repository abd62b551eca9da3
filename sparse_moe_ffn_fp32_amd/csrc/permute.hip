// Stable expert permutation of the routed slots (one workgroup), and the
// weighted combine of per-slot expert outputs.
#include "moe_block_permute.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids,
                                                                int n, int E,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_rows) {
  __shared__ PermuteSmem sm;
  block_permute(ids, n, E, counts, offsets, sorted_rows, sm);
}

hipError_t launch_permute(const int32_t* ids, int n, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_rows, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, n, E, counts, offsets,
                     sorted_rows);
  return hipGetLastError();
}

// out[t, :] = sum_j w[t*k + j] * y[t*k + j, :]  (weighted sum of the selected
// experts' outputs; one thread per 4 output elements).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w, int T, int k,
                                                      float* __restrict__ out) {
  constexpr int C4 = kH / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * C4) return;
  const int t = (int)(idx / C4);
  const int c = (int)(idx % C4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wt = w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y)[((size_t)t * k + j) * C4 + c];
    acc.x += wt * v.x;
    acc.y += wt * v.y;
    acc.z += wt * v.z;
    acc.w += wt * v.w;
  }
  reinterpret_cast<float4*>(out)[(size_t)t * C4 + c] = acc;
}

hipError_t launch_combine(const float* y, const float* w, int T, int k, float* out, hipStream_t s) {
  const long long n4 = (long long)T * (kH / 4);
  const unsigned blocks = (unsigned)((n4 + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, y, w, T, k, out);
  return hipGetLastError();
}

}  // namespace moe
