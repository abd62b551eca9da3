// Expert histogram -> exclusive prefix sum -> stable scatter of the T*k routed
// slots into expert-sorted order. The pages do not describe this step; it is
// the grouping that lets the expert GEMMs run over contiguous row ranges.
//
// One workgroup of 16 waves. Ranks inside a wave come from ballots over the
// expert id bits (lanes with equal ids), ranks across waves from per-wave
// counts in LDS, so the order of slots within an expert is their input order
// and the result is deterministic.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids,
                                                                int n, int E,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted_rows) {
  __shared__ int hist[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < kMaxExperts; e += kPermThreads) hist[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();

  if (wave == 0) {
    int c[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = (e < E) ? hist[e] : 0;
      local += c[q];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < E) {
        counts[e] = c[q];
        offsets[e] = run;
        base[e] = run;
      }
      run += c[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n; c0 += kPermThreads) {
    for (int e = lane; e < kMaxExperts; e += 64) wcnt[wave][e] = 0;
    const int i = c0 + tid;
    int e = -1;
    if (i < n) e = ids[i];
    const bool valid = (e >= 0) && (e < E);
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const unsigned long long bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      sorted_rows[base[e] + pre + rank] = i;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kPermThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) s += wcnt[w][ee];
      base[ee] += s;
    }
    __syncthreads();
  }
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
