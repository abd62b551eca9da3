// Stable expert permutation of the routed slots (one workgroup up to 1024
// slots, histogram + scan + parallel scatter above), and the
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



// Parallel form of the same stable permutation when the router already
// counted its routed slots per block: route block b owns slots
// [b*spb, (b+1)*spb) (spb <= 256) and hist[b][e] counts them by expert.
// permute_scan_kernel (one workgroup) turns the histograms into counts,
// offsets and base[b][e] = offsets[e] + (slots of e in blocks before b), in
// place; permute_scatter_kernel (one workgroup per route block) ranks its
// slots within each expert and writes them. Slots go in ascending order
// within an expert, as in the single-workgroup version.
constexpr int kScanThreads = 1024;
constexpr int kScatterThreads = 256;
constexpr int kScanChunk = 32;   // histogram entries a scan thread loads at once

__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(int E, int32_t* __restrict__ hist,
                                                                    int nb,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets) {
  // thread (segment s, expert e): blocks [s*per, (s+1)*per) of expert e
  __shared__ int seg_sum[kScanThreads];
  __shared__ int excl_e[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int nseg = kScanThreads / E;   // E <= 256, so at least 4 segments
  const int e = tid % E, sgm = tid / E;
  const bool act = sgm < nseg;
  const int per = (nb + nseg - 1) / nseg;
  const int b0 = min(nb, sgm * per), b1 = min(nb, b0 + per);
  // the segment's counts in chunks of kScanChunk, each chunk's loads all in
  // flight at once (one memory round trip per chunk)
  int sum = 0;
  if (act) {
    for (int b = b0; b < b1; b += kScanChunk) {
      int v[kScanChunk];
#pragma unroll
      for (int j = 0; j < kScanChunk; ++j) v[j] = b + j < b1 ? hist[(size_t)(b + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanChunk; ++j) sum += v[j];
    }
  }
  seg_sum[tid] = act ? sum : 0;
  __syncthreads();
  if (tid < E) {
    int tot = 0;
    for (int q = 0; q < nseg; ++q) tot += seg_sum[q * E + tid];
    excl_e[tid] = tot;   // totals; scanned below
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan over experts: 4 per lane, then across the wave
    int c[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = tid * 4 + q;
      c[q] = ee < E ? excl_e[ee] : 0;
      local += c[q];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (tid >= d) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = tid * 4 + q;
      if (ee < E) {
        counts[ee] = c[q];
        offsets[ee] = run;
        excl_e[ee] = run;
      }
      run += c[q];
    }
    if (tid == 63) offsets[E] = incl;
  }
  __syncthreads();
  if (act) {
    int run = excl_e[e];
    for (int q = 0; q < sgm; ++q) run += seg_sum[q * E + e];
    for (int b = b0; b < b1; b += kScanChunk) {
      int v[kScanChunk];
#pragma unroll
      for (int j = 0; j < kScanChunk; ++j) v[j] = b + j < b1 ? hist[(size_t)(b + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanChunk; ++j) {
        if (b + j < b1) hist[(size_t)(b + j) * E + e] = run;
        run += v[j];
      }
    }
  }
}

__global__ __launch_bounds__(kScatterThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int n, int E, const int32_t* __restrict__ base, int spb,
    int32_t* __restrict__ sorted_rows) {
  __shared__ int wcnt[kScatterThreads / 64][kMaxExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = lane; e < kMaxExperts; e += 64) wcnt[wave][e] = 0;
  const int i = blockIdx.x * spb + tid;
  int e = -1;
  if (tid < spb && i < n) e = ids[i];
  const bool valid = e >= 0 && e < E;
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = valid && ((e >> bit) & 1);
    const unsigned long long bal = __ballot(on);
    peers &= on ? bal : ~bal;
  }
  const int rank = __popcll(peers & ((1ull << lane) - 1ull));
  if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int p = base[(size_t)blockIdx.x * E + e] + rank;
    for (int w = 0; w < wave; ++w) p += wcnt[w][e];
    sorted_rows[p] = i;
  }
}

// Expert histogram of each block's spb consecutive slots (the standalone
// permutation's first pass; the router writes the same table as it goes).
__global__ __launch_bounds__(kScatterThreads) void permute_hist_kernel(const int32_t* __restrict__ ids,
                                                                       int n, int E, int spb,
                                                                       int32_t* __restrict__ hist) {
  __shared__ int h[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < kMaxExperts; e += kScatterThreads) h[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * spb + tid;
  if (tid < spb && i < n) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kScatterThreads) hist[(size_t)blockIdx.x * E + e] = h[e];
}

hipError_t launch_permute_blocks(const int32_t* ids, int n, int E, int32_t* hist, int nb, int spb,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                                 hipStream_t s) {
  if (spb > kScatterThreads || E > kMaxExperts) return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, E, hist, nb, counts,
                     offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(kScatterThreads), 0, s, ids, n, E, hist,
                     spb, sorted_rows);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int n, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_rows, int32_t* hist, hipStream_t s) {
  if (n <= kPermThreads || !hist) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, s, ids, n, E, counts, offsets,
                       sorted_rows);
    return hipGetLastError();
  }
  // slots in blocks of 32 tokens, as the router's histograms
  const int spb = 32 * k;
  const int nb = (n + spb - 1) / spb;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(kScatterThreads), 0, s, ids, n, E, spb, hist);
  return launch_permute_blocks(ids, n, E, hist, nb, spb, counts, offsets, sorted_rows, s);
}

// out[t, :] = sum_j w[t*k + j] * y[t*k + j, :]  (weighted sum of the selected
// experts' outputs; one thread per 4 output elements).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w, int T, int k,
                                                      const uint16_t* __restrict__ resid,
                                                      float* __restrict__ out) {
  constexpr int C4 = kH / 4;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * C4) return;
  const int t = (int)(idx / C4);
  const int c = (int)(idx % C4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (resid) {
    const uint2 r = reinterpret_cast<const uint2*>(resid)[idx];
    acc = make_float4(bf16_bits_to_f32(r.x & 0xFFFFu), bf16_bits_to_f32(r.x >> 16),
                      bf16_bits_to_f32(r.y & 0xFFFFu), bf16_bits_to_f32(r.y >> 16));
  }
  for (int j = 0; j < k; ++j) {
    const float wt = w[(size_t)t * k + j];
    // y is read once: non-temporal loads keep it from evicting the caches
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y) + ((size_t)t * k + j) * C4 + c);
    acc.x += wt * v[0];
    acc.y += wt * v[1];
    acc.z += wt * v[2];
    acc.w += wt * v[3];
  }
  reinterpret_cast<float4*>(out)[(size_t)t * C4 + c] = acc;
}

hipError_t launch_combine(const float* y, const float* w, int T, int k, const uint16_t* resid,
                          float* out, hipStream_t s) {
  const long long n4 = (long long)T * (kH / 4);
  const unsigned blocks = (unsigned)((n4 + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, y, w, T, k, resid, out);
  return hipGetLastError();
}

}  // namespace moe
