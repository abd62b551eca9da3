// Router GEMM + top-k + softmax over the selected logits.
//
// logits[t, e] = sum_h x[t, h] Wr[e, h] + br[e]  (gpt-oss-120b techniques map,
// "Checked in its code" table, row "Auxiliary-loss-free load balancing": the
// router is a linear layer with a bias; row "Mixture of experts": top-k over
// the router logits, then softmax over the selected ones).
//
// fp32 router on bf16 matrix cores: x is bf16, and each fp32 weight is split
// exactly into three bf16 pieces (hi + mid + lo, 8 significant bits each).
// Every product x * piece is exact in fp32 and the matrix core accumulates in
// fp32, so the result is an fp32-accumulated dot product of the fp32 weights.
// A wave computes a 32-token x 32*MT-expert tile of 32x32x16 MFMAs over a K
// range, with a register prefetch ring over its K steps.
//
// Two schedules, chosen by T (both deterministic, fixed summation order):
//  * few tokens (T <= 128, T*E <= 4096): the K dimension is cut into 20 chunks, one wave
//    per (32-token tile, chunk) writes partial logits to scratch; a second
//    launch adds the 20 partials in chunk order, adds the bias and selects
//    the top k: blocks of 256/E tokens when no permutation is wanted, or a
//    single 1024-thread block that also builds the expert permutation.
//  * many tokens: a block per 32 tokens, its waves split K and add their
//    partial tiles in wave order through LDS, then select the top k and
//    count the block's routed slots per expert for the parallel permutation.
#include "moe_block_permute.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteChunks = 20;                  // K chunks of the few-token schedule
constexpr int kRouteChunkSteps = kH / 16 / kRouteChunks;  // 9 MFMA steps of 16 K
constexpr int kRouteSmallT = 128;
constexpr int kRouteMaxPairs = 4 * 1024;   // T * E of the few-token schedule (LDS logits)
static_assert(kRouteChunkSteps * 16 * kRouteChunks == kH, "chunks must tile K");

static bool few_tokens(int T, int E) { return T <= kRouteSmallT && T * E <= kRouteMaxPairs; }

size_t route_scratch_bytes(int T, int E) {
  // few tokens: K-chunk partial logits; many: per-32-token-block expert histograms
  return few_tokens(T, E) ? (size_t)kRouteChunks * T * E * sizeof(float)
                          : (size_t)((T + 31) / 32) * E * sizeof(int32_t);
}

__device__ __forceinline__ void split3_bf16(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t uh = u & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(uh);          // exact: at most 16 significant bits
  const uint32_t um = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(um);         // exact: at most 8 significant bits
  hi = uh >> 16;
  mid = um >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// 8 fp32 weights -> three bf16x8 fragments
__device__ __forceinline__ void split_frag(const float4& a, const float4& b, bf16x8& fh, bf16x8& fm,
                                           bf16x8& fl) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) split3_bf16(v[i], h[i], m[i], l[i]);
  uint4 ph, pm, pl;
  ph.x = h[0] | (h[1] << 16); ph.y = h[2] | (h[3] << 16); ph.z = h[4] | (h[5] << 16); ph.w = h[6] | (h[7] << 16);
  pm.x = m[0] | (m[1] << 16); pm.y = m[2] | (m[3] << 16); pm.z = m[4] | (m[5] << 16); pm.w = m[6] | (m[7] << 16);
  pl.x = l[0] | (l[1] << 16); pl.y = l[2] | (l[3] << 16); pl.z = l[4] | (l[5] << 16); pl.w = l[6] | (l[7] << 16);
  fh = u4_as_bf16x8(ph);
  fm = u4_as_bf16x8(pm);
  fl = u4_as_bf16x8(pl);
}

template <int MT>
struct RStage {
  uint4 xv;
  float4 w[MT][2];
};

// Operand loader of one wave: tokens tok0 + (lane & 31), experts 32mt +
// (lane & 31), K from k0 in steps of 16 (lane half hh takes 8 of them).
template <int MT>
struct RouteLoader {
  const uint16_t* xrow;
  bool tok_ok;
  const float* wrow[MT];
  bool e_ok[MT];

  __device__ __forceinline__ void init(const uint16_t* x, const float* Wr, int T, int E, int tok,
                                       int k0, int lane) {
    // padded tokens / experts read a clamped valid row: their results are
    // never used, and the loads stay unconditional
    const int n = lane & 31;
    const int hh = lane >> 5;
    tok_ok = tok < T;
    xrow = x + (size_t)min(tok, T - 1) * kH + k0 + 8 * hh;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int e = mt * 32 + n;
      e_ok[mt] = e < E;
      wrow[mt] = Wr + (size_t)min(e, E - 1) * kH + k0 + 8 * hh;
    }
  }
  __device__ __forceinline__ void load(RStage<MT>& st, int s) const {
    st.xv = *reinterpret_cast<const uint4*>(xrow + 16 * s);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      st.w[mt][0] = *reinterpret_cast<const float4*>(wrow[mt] + 16 * s);
      st.w[mt][1] = *reinterpret_cast<const float4*>(wrow[mt] + 16 * s + 4);
    }
  }
};

template <int MT>
__device__ __forceinline__ void route_mma(const RStage<MT>& st, f32x16 (&acc)[MT]) {
  const bf16x8 xb = u4_as_bf16x8(st.xv);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    bf16x8 fh, fm, fl;
    split_frag(st.w[mt][0], st.w[mt][1], fh, fm, fl);
    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, xb, acc[mt], 0, 0, 0);
    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fm, xb, acc[mt], 0, 0, 0);
    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh, xb, acc[mt], 0, 0, 0);
  }
}

template <int MT>
constexpr int route_depth() {
  return MT <= 1 ? 8 : MT <= 2 ? 6 : MT <= 4 ? 4 : 2;
}

// K loop over NSTEPS steps with a register prefetch ring: fully unrolled for
// short K ranges (exact load counting), a rolled ring otherwise (the long
// unroll would spill).
template <int MT, int NSTEPS>
__device__ __forceinline__ void route_kloop(const RouteLoader<MT>& L, f32x16 (&acc)[MT]) {
  constexpr int D = route_depth<MT>() < NSTEPS ? route_depth<MT>() : NSTEPS;
  RStage<MT> st[D];
#pragma unroll
  for (int q = 0; q < D; ++q) L.load(st[q], q);
  // scheduling barriers keep the ring's loads where they are written: left
  // free, the scheduler sinks them next to their use and only about one
  // step stays in flight
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NSTEPS <= 16) {
#pragma unroll
    for (int s = 0; s < NSTEPS; ++s) {
      route_mma<MT>(st[s % D], acc);
      if (s + D < NSTEPS) L.load(st[s % D], s + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int s0 = 0; s0 < NSTEPS; s0 += D) {
#pragma unroll
      for (int q = 0; q < D; ++q) {
        const int s = s0 + q;
        if (s < NSTEPS) {
          route_mma<MT>(st[q], acc);
          if (s + D < NSTEPS) L.load(st[q], s + D);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Insert (cv, ci) into the descending list (bv, bi) of length k <= KM; branch-free.
template <int KM>
__device__ __forceinline__ void topk_insert(float (&bv)[KM], int (&bi)[KM], int k, float cv, int ci) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const bool b = better(cv, ci, bv[j], bi[j]);
      const float tv = b ? bv[j] : cv;
      const int ti = b ? bi[j] : ci;
      bv[j] = b ? cv : bv[j];
      bi[j] = b ? ci : bi[j];
      cv = tv;
      ci = ti;
    }
  }
}

// Top-k (descending, ties -> lower expert id) and softmax over the selected
// logits of one token, by LPT consecutive lanes: lane `sub` scans experts
// sub, sub + LPT, ... (logit of expert e at lg[e * e_stride]), then the lanes
// merge their lists in log2(LPT) butterfly steps. All lanes of the wave must
// call it. When `active`, lanes sub < k write slot sub of ids_t / w_t (and
// lds_ids_t if non-null).
template <int LPT, int KM>
__device__ __forceinline__ void lanes_topk_km(const float* lg, int e_stride, int E, int k,
                                              bool active, int32_t* ids_t, float* w_t,
                                              int32_t* lds_ids_t) {
  const int sub = threadIdx.x & (LPT - 1);
  float bv[KM];
  int bi[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    bv[j] = -INFINITY;
    bi[j] = 0x7FFFFFFF;
  }
  if (active)
    for (int e = sub; e < E; e += LPT) topk_insert<KM>(bv, bi, k, lg[e * e_stride], e);
#pragma unroll
  for (int d = 1; d < LPT; d <<= 1) {
    float pv[KM];
    int pi[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      pv[j] = __shfl_xor(bv[j], d, 64);
      pi[j] = __shfl_xor(bi[j], d, 64);
    }
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) topk_insert<KM>(bv, bi, k, pv[j], pi[j]);
  }
  if (!active) return;
  float ex[KM];
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    ex[j] = (j < k) ? __expf(bv[j] - bv[0]) : 0.f;
    z += ex[j];
  }
  const float inv = 1.0f / z;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k && sub == j) {
      ids_t[j] = bi[j];
      w_t[j] = ex[j] * inv;
      if (lds_ids_t) lds_ids_t[j] = bi[j];
    }
  }
}

template <int LPT>
__device__ __forceinline__ void lanes_topk(const float* lg, int e_stride, int E, int k, bool active,
                                           int32_t* ids_t, float* w_t, int32_t* lds_ids_t) {
  if (k == 1) lanes_topk_km<LPT, 1>(lg, e_stride, E, k, active, ids_t, w_t, lds_ids_t);
  else if (k == 2) lanes_topk_km<LPT, 2>(lg, e_stride, E, k, active, ids_t, w_t, lds_ids_t);
  else if (k <= 4) lanes_topk_km<LPT, 4>(lg, e_stride, E, k, active, ids_t, w_t, lds_ids_t);
  else lanes_topk_km<LPT, 8>(lg, e_stride, E, k, active, ids_t, w_t, lds_ids_t);
}

constexpr int kTopkLanes = 8;   // lanes per token in the top-k

// ---------------------------------------------------------------- many tokens
template <int MT, int WK>
__global__ __launch_bounds__(WK * 64) void route_kernel(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ Wr,
                                                        const float* __restrict__ br, int T, int E,
                                                        int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ wts,
                                                        float* __restrict__ logits,
                                                        int32_t* __restrict__ block_hist) {
  constexpr int KW = kH / WK;      // K range of one wave
  constexpr int KSTEPS = KW / 16;  // MFMA steps of one wave
  constexpr int LDR = 33;          // padded row of the reduction buffer
  static_assert(KW % 16 == 0, "K split must be a multiple of 16");
  extern __shared__ float red[];   // [MT * 32][LDR]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 32;
  const int n = lane & 31;
  const int hh = lane >> 5;

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
  RouteLoader<MT> L;
  L.init(x, Wr, T, E, tok0 + n, wave * KW, lane);
  route_kloop<MT, KSTEPS>(L, acc);

  // Fixed-order split-K reduction: red[e][token] = sum over waves 0..WK-1.
  // 32x32 result layout: lane holds column n (token), rows 8q + 4hh + j.
  for (int w = 0; w < WK; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float* p = &red[(mt * 32 + 8 * q + 4 * hh + j) * LDR + n];
            *p = (w == 0) ? acc[mt][4 * q + j] : (*p + acc[mt][4 * q + j]);
          }
    }
    __syncthreads();
  }

  // bias, optional logits output
  for (int i = threadIdx.x; i < 32 * E; i += WK * 64) {
    const int e = i / 32, tt = i % 32;
    const float v = red[e * LDR + tt] + br[e];
    red[e * LDR + tt] = v;
    if (logits && tok0 + tt < T) logits[(size_t)(tok0 + tt) * E + e] = v;
  }
  __syncthreads();
  // top-k: 8 lanes per token, the first 256 threads cover the 32 tokens
  if (threadIdx.x < 32 * kTopkLanes) {
    const int tt = threadIdx.x / kTopkLanes;
    const int t = tok0 + tt;
    lanes_topk<kTopkLanes>(red + tt, LDR, E, k, t < T, ids + (size_t)t * k, wts + (size_t)t * k,
                           nullptr);
  }
  if (block_hist) {
    // expert histogram of this block's routed slots, for the parallel permutation
    int* hist = reinterpret_cast<int*>(red);   // the logits tile is no longer needed
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += WK * 64) hist[e] = 0;
    __syncthreads();
    const int nslots = (min(T, tok0 + 32) - tok0) * k;
    for (int i = threadIdx.x; i < nslots; i += WK * 64) atomicAdd(&hist[ids[(size_t)tok0 * k + i]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += WK * 64) block_hist[(size_t)blockIdx.x * E + e] = hist[e];
  }
}

// ---------------------------------------------------------------- few tokens
template <int MT>
__global__ __launch_bounds__(64) void route_partial_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ Wr, int T,
                                                           int E, float* __restrict__ partial) {
  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tok = blockIdx.x * 32 + n;
  const int kc = blockIdx.y;
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
  RouteLoader<MT> L;
  L.init(x, Wr, T, E, tok, kc * kRouteChunkSteps * 16, lane);
  route_kloop<MT, kRouteChunkSteps>(L, acc);
  if (tok < T) {
    float* prow = partial + ((size_t)kc * T + tok) * E;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = mt * 32 + 8 * q + 4 * hh + j;
          if (e < E) prow[e] = acc[mt][4 * q + j];
        }
  }
}

// One 1024-thread block: logits = bias + sum of the chunk partials in chunk
// order (one thread per (token, expert) pair, all partial loads in flight at
// once), then the top k of each token by rank, the softmax, and the expert
// permutation of the T*k slots.
template <int PAIRS>
__global__ __launch_bounds__(kPermThreads) void route_finish_kernel(
    const float* __restrict__ partial, const float* __restrict__ br, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows) {
  __shared__ PermuteSmem sm;
  __shared__ int lds_ids[kRouteSmallT * kMaxTopK];
  __shared__ float lg[kRouteMaxPairs + kMaxExperts];   // [E][T + 1]
  __shared__ float sel_v[kRouteSmallT * kMaxTopK];
  const int tid = threadIdx.x;
  const int TE = T * E;
  const int ldt = T + 1;   // padded expert-major stride: a token's lanes hit distinct banks
  float bias[PAIRS];
#pragma unroll
  for (int j = 0; j < PAIRS; ++j) bias[j] = br[min(tid + j * kPermThreads, TE - 1) % E];
  float acc[PAIRS];
#pragma unroll
  for (int j = 0; j < PAIRS; ++j) acc[j] = 0.f;
#pragma unroll
  for (int c = 0; c < kRouteChunks; ++c) {
#pragma unroll
    for (int j = 0; j < PAIRS; ++j) {
      const int i = min(tid + j * kPermThreads, TE - 1);
      acc[j] += partial[(size_t)c * TE + i];
    }
  }
#pragma unroll
  for (int j = 0; j < PAIRS; ++j) {
    const int i = tid + j * kPermThreads;
    if (i < TE) {
      const int t = i / E, e = i - (i / E) * E;
      const float v = acc[j] + bias[j];
      lg[e * ldt + t] = v;
      if (logits) logits[i] = v;
    }
  }
  __syncthreads();
  // Top-k by rank: the thread of (token t, expert e) counts the experts that
  // beat e (larger logit, or equal logit and lower id); e is selected at
  // position `rank` when rank < k. No cross-lane traffic; the logits of a
  // token are LDS broadcasts.
#pragma unroll
  for (int j = 0; j < PAIRS; ++j) {
    const int i = tid + j * kPermThreads;
    if (i < TE) {
      const int t = i / E, e = i - (i / E) * E;
      const float v = lg[e * ldt + t];
      int rank = 0;
      for (int e2 = 0; e2 < E; ++e2) rank += better(lg[e2 * ldt + t], e2, v, e) ? 1 : 0;
      if (rank < k) {
        sel_v[t * k + rank] = v;
        lds_ids[t * k + rank] = e;
      }
    }
  }
  __syncthreads();
  // softmax over the selected logits (position 0 holds the largest)
  for (int i = tid; i < T * k; i += kPermThreads) {
    const int t = i / k;
    const float m = sel_v[t * k];
    float z = 0.f;
    for (int j = 0; j < k; ++j) z += __expf(sel_v[t * k + j] - m);
    ids[i] = lds_ids[i];
    wts[i] = __expf(sel_v[i] - m) / z;
  }
  __syncthreads();
  block_permute(lds_ids, T * k, E, counts, offsets, sorted_rows, sm);
}

// The same sums, top-k and softmax as route_finish_kernel without the
// permutation, spread over blocks of 256 / E tokens each (one thread per
// (token, expert) pair), so that the partial-logit loads of a decode batch
// run on many CUs instead of one. Arithmetic in the same order: identical
// expert choices and weights.
__global__ __launch_bounds__(256) void route_finish_tiles_kernel(
    const float* __restrict__ partial, const float* __restrict__ br, int T, int E, int k, int tb,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits) {
  __shared__ float lg[256];
  __shared__ float sel_v[256];
  __shared__ int sel_e[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * tb;
  const int nt = min(tb, T - t0);
  const int TE = T * E;
  const int np = nt * E;
  float v = 0.f;
  if (tid < np) {
    const int i = t0 * E + tid;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kRouteChunks; ++c) acc += partial[(size_t)c * TE + i];
    v = acc + br[tid % E];
    lg[tid] = v;
    if (logits) logits[i] = v;
  }
  __syncthreads();
  if (tid < np) {
    const int tl = tid / E, e = tid - tl * E;
    const float* row = lg + tl * E;
    int rank = 0;
    for (int e2 = 0; e2 < E; ++e2) rank += better(row[e2], e2, v, e) ? 1 : 0;
    if (rank < k) {
      sel_v[tl * k + rank] = v;
      sel_e[tl * k + rank] = e;
    }
  }
  __syncthreads();
  if (tid < nt * k) {
    const int tl = tid / k;
    const float m = sel_v[tl * k];
    float z = 0.f;
    for (int j = 0; j < k; ++j) z += __expf(sel_v[tl * k + j] - m);
    ids[t0 * k + tid] = sel_e[tid];
    wts[t0 * k + tid] = __expf(sel_v[tid] - m) / z;
  }
}

static void launch_finish(const float* scratch, const float* br, int T, int E, int k, int32_t* ids,
                          float* w, float* logits, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_rows, hipStream_t s) {
  const int pairs = (T * E + kPermThreads - 1) / kPermThreads;
#define MOE_FINISH(P)                                                                             \
  hipLaunchKernelGGL((route_finish_kernel<P>), dim3(1), dim3(kPermThreads), 0, s, scratch,          \
                     br, T, E, k, ids, w, logits, counts, offsets, sorted_rows)
  if (pairs <= 1) MOE_FINISH(1);
  else if (pairs <= 2) MOE_FINISH(2);
  else MOE_FINISH(4);
#undef MOE_FINISH
}

// ---------------------------------------------------------------- launch
template <int MT>
static hipError_t launch_route_mt(const uint16_t* x, const float* Wr, const float* br, int T, int E,
                                  int k, int32_t* ids, float* w, float* logits,
                                  float* scratch, int32_t* counts, int32_t* offsets,
                                  int32_t* sorted_rows, hipStream_t s) {
  if (few_tokens(T, E)) {
    const dim3 grid((T + 31) / 32, kRouteChunks);
    hipLaunchKernelGGL((route_partial_kernel<MT>), grid, dim3(64), 0, s, x, Wr, T, E, scratch);
    if (counts) {
      launch_finish(scratch, br, T, E, k, ids, w, logits, counts, offsets, sorted_rows, s);
    } else {
      const int tb = 256 / E;   // tokens per block; E <= 256
      hipLaunchKernelGGL(route_finish_tiles_kernel, dim3((T + tb - 1) / tb), dim3(256), 0, s, scratch,
                         br, T, E, k, tb, ids, w, logits);
    }
    return hipGetLastError();
  }
  const int blocks = (T + 31) / 32;
  const size_t lds = (size_t)MT * 32 * 33 * sizeof(float);
  static_assert(32 * 33 >= kMaxExperts, "the reduction tile doubles as the histogram");
  int32_t* hist = reinterpret_cast<int32_t*>(scratch);   // [blocks][E] routed-slot histograms
  // 12 waves split K when few blocks would run; only for one expert tile,
  // where the 768-thread register budget holds the prefetch ring.
  if constexpr (MT == 1) {
    if (blocks < 256) {
      hipLaunchKernelGGL((route_kernel<1, 12>), dim3(blocks), dim3(12 * 64), lds, s, x, Wr, br, T, E,
                         k, ids, w, logits, counts ? hist : nullptr);
    } else {
      hipLaunchKernelGGL((route_kernel<1, 4>), dim3(blocks), dim3(4 * 64), lds, s, x, Wr, br, T, E,
                         k, ids, w, logits, counts ? hist : nullptr);
    }
  } else {
    hipLaunchKernelGGL((route_kernel<MT, 4>), dim3(blocks), dim3(4 * 64), lds, s, x, Wr, br, T, E, k,
                       ids, w, logits, counts ? hist : nullptr);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !counts) return err;
  return launch_permute_blocks(ids, T * k, E, hist, blocks, 32 * k, counts, offsets, sorted_rows, s);
}

hipError_t launch_route(const uint16_t* x, const float* Wr, const float* br, int T, int E, int k,
                        int32_t* ids, float* w, float* logits, float* scratch,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_rows, hipStream_t s) {
  switch ((E + 31) / 32) {
    case 1: return launch_route_mt<1>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 2: return launch_route_mt<2>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 3: return launch_route_mt<3>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 4: return launch_route_mt<4>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 5: return launch_route_mt<5>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 6: return launch_route_mt<6>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 7: return launch_route_mt<7>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    case 8: return launch_route_mt<8>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets, sorted_rows, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
