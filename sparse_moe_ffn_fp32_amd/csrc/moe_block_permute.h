// One-workgroup stable counting sort of routed slots by expert id.
//
// Expert histogram -> exclusive prefix sum -> stable scatter. The pages do
// not describe this step; it is the grouping that lets the expert GEMMs run
// over contiguous row ranges. Ranks inside a wave come from ballots over the
// expert-id bits (lanes with equal ids), ranks across waves from per-wave
// counts in LDS, so slots keep their input order within an expert and the
// result is deterministic.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

struct PermuteSmem {
  int hist[kMaxExperts];
  int base[kMaxExperts];
  int wcnt[kPermWaves][kMaxExperts];
};

// Called by all 1024 threads of the block. `ids` (n entries) may live in
// global memory or LDS; entries outside [0, E) are ignored.
__device__ __forceinline__ void block_permute(const int32_t* ids, int n, int E,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ sorted_rows, PermuteSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < kMaxExperts; e += kPermThreads) sm.hist[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPermThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&sm.hist[e], 1);
  }
  __syncthreads();

  if (wave == 0) {
    int c[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      c[q] = (e < E) ? sm.hist[e] : 0;
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
        sm.base[e] = run;
      }
      run += c[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();

  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n; c0 += kPermThreads) {
    for (int e = lane; e < kMaxExperts; e += 64) sm.wcnt[wave][e] = 0;
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
    if (valid && rank == 0) sm.wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += sm.wcnt[w][e];
      sorted_rows[sm.base[e] + pre + rank] = i;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kPermThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) s += sm.wcnt[w][ee];
      sm.base[ee] += s;
    }
    __syncthreads();
  }
}

}  // namespace moe
