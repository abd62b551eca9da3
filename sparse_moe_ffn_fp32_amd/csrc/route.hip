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
// A wave computes 32-token x 32*MT-expert tiles of 32x32x16 MFMAs over a K
// range, with a register prefetch ring over its K steps.
//
// Two schedules, chosen by T (both deterministic, fixed summation order):
//  * few tokens (T <= 128, T*E <= 4096): the K dimension is cut into 20 chunks, one wave
//    per (32-token tile, chunk) writes partial logits to scratch; a second
//    launch adds the 20 partials in chunk order, adds the bias and selects
//    the top k: blocks of 256/E tokens when no permutation is wanted, or a
//    single 1024-thread block that also builds the expert permutation.
//  * many tokens: one launch splits the weights into their bf16 pieces, in
//    MFMA operand order; then a block per 32 or 64 tokens, its waves split K
//    and add their partial tiles in wave order through LDS, then select the
//    top k and count the routed slots per expert of each 32-token group for
//    the parallel permutation.
// The decoder block's pre-MoE RMSNorm folds into either schedule (RouteNorm):
// the weights are scaled by the norm scale and each token's logits by its
// inverse RMS, which the few-token schedule forms from its own sums of
// squares.
#include "moe_block_permute.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRouteSteps = kH / 16;             // MFMA steps of 16 K
constexpr int kRouteChunks = 20;                  // K chunks of the few-token schedule
constexpr int kRouteChunkSteps = kH / 16 / kRouteChunks;  // 9 MFMA steps of 16 K
constexpr int kRouteSmallT = 128;
constexpr int kRouteMaxPairs = 4 * 1024;   // T * E of the few-token schedule (LDS logits)
static_assert(kRouteChunkSteps * 16 * kRouteChunks == kH, "chunks must tile K");

static bool few_tokens(int T, int E) { return T <= kRouteSmallT && T * E <= kRouteMaxPairs; }
bool route_few_tokens(int T, int E) { return few_tokens(T, E); }

size_t route_split_bytes(int E);

size_t route_scratch_bytes(int T, int E) {
  // few tokens: K-chunk partial logits (and the decoder block's chunk sums of
  // squares); many: the split weights, then the
  // per-32-token-group expert histograms
  return few_tokens(T, E) ? (size_t)kRouteChunks * T * (E + 1) * sizeof(float)   // + sums of squares
                          : route_split_bytes(E) + (size_t)((T + 31) / 32) * E * sizeof(int32_t);
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
  float4 sc[2];   // NORM: the norm scale of the step's 8 K values
};

// Operand loader of one wave: tokens tok0 + (lane & 31), experts 32mt +
// (lane & 31), K from k0 in steps of 16 (lane half hh takes 8 of them).
// NORM: also the norm scale of the same K values (the router of the decoder
// block takes Wr[e, h] * scale[h] as its weights; the comment above
// route_partial_kernel gives the algebra).
template <int MT, bool NORM = false>
struct RouteLoader {
  const uint16_t* xrow;
  bool tok_ok;
  const float* wrow[MT];
  const float* srow;
  bool e_ok[MT];

  __device__ __forceinline__ void init(const uint16_t* x, const float* Wr, const float* scale, int T,
                                       int E, int tok, int k0, int lane) {
    // padded tokens / experts read a clamped valid row: their results are
    // never used, and the loads stay unconditional
    const int n = lane & 31;
    const int hh = lane >> 5;
    tok_ok = tok < T;
    xrow = x + (size_t)min(tok, T - 1) * kH + k0 + 8 * hh;
    srow = NORM ? scale + k0 + 8 * hh : nullptr;
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
    if (NORM) {
      st.sc[0] = *reinterpret_cast<const float4*>(srow + 16 * s);
      st.sc[1] = *reinterpret_cast<const float4*>(srow + 16 * s + 4);
    }
  }
};

__device__ __forceinline__ float4 mul4(const float4 a, const float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

// NORM: the weights are multiplied by the norm scale (rounded to fp32) before
// the exact split, and `ss` accumulates the squares of the lane's 8 inputs.
template <int MT, bool NORM = false>
__device__ __forceinline__ void route_mma(const RStage<MT>& st, f32x16 (&acc)[MT], float& ss) {
  const bf16x8 xb = u4_as_bf16x8(st.xv);
  if (NORM) {
    const uint32_t dw[4] = {st.xv.x, st.xv.y, st.xv.z, st.xv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 v = __builtin_bit_cast(bf16x2, dw[q]);
      ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    bf16x8 fh, fm, fl;
    if (NORM)
      split_frag(mul4(st.w[mt][0], st.sc[0]), mul4(st.w[mt][1], st.sc[1]), fh, fm, fl);
    else
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

// K loop over NSTEPS steps with a register prefetch ring, fully unrolled
// (exact load counting).
template <int MT, int NSTEPS, bool NORM = false>
__device__ __forceinline__ void route_kloop(const RouteLoader<MT, NORM>& L, f32x16 (&acc)[MT],
                                            float& ss) {
  static_assert(NSTEPS <= 16, "a longer unroll would spill");
  constexpr int D = route_depth<MT>() < NSTEPS ? route_depth<MT>() : NSTEPS;
  RStage<MT> st[D];
#pragma unroll
  for (int q = 0; q < D; ++q) L.load(st[q], q);
  // scheduling barriers keep the ring's loads where they are written: left
  // free, the scheduler sinks them next to their use and only about one
  // step stays in flight
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < NSTEPS; ++s) {
    route_mma<MT, NORM>(st[s % D], acc, ss);
    if (s + D < NSTEPS) L.load(st[s % D], s + D);
    __builtin_amdgcn_sched_barrier(0);
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
constexpr int kRouteTwoTileBlocks = 256;   // blocks of 64 tokens that fill the chip

// ---------------------------------------------------------------- many tokens
// The fp32 router weights are split once per call into their three bf16
// pieces, stored in MFMA operand order: fragment (s, mt, p) is 64 lanes x 8
// bf16 (1 KiB), lane (n, hh) holding piece p (lo, mid, hi) of
// Wr[32 mt + n][16 s + 8 hh .. + 7]; experts past E are zero. The tile
// kernel then streams whole fragments (one coalesced 1 KiB load each) with no
// arithmetic besides the MFMAs.
// Expert tiles of the split weights: E rounded up to 32, and for the
// expert-tiled kernel further to a whole number of tiles per wave.
constexpr int route_tiles_padded(int MT) { return MT <= 4 ? MT : MT <= 6 ? 6 : 8; }

size_t route_split_bytes(int E) {
  return (size_t)kRouteSteps * route_tiles_padded((E + 31) / 32) * 3 * 1024;
}

// MT = padded expert tiles of the layout; tiles past E are zero. With
// `scale` (the decoder block's norm scale) the pieces are those of
// Wr[e, h] * scale[h] rounded to fp32.
__global__ __launch_bounds__(256) void route_split_kernel(const float* __restrict__ Wr,
                                                          const float* __restrict__ scale, int E,
                                                          int MT, uint4* __restrict__ Wp) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= kRouteSteps * MT * 64) return;
  const int lane = idx & 63;
  const int mt = (idx >> 6) % MT;
  const int s = (idx >> 6) / MT;
  const int e = mt * 32 + (lane & 31);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  if (e < E) {
    const float* src = Wr + (size_t)e * kH + 16 * s + 8 * (lane >> 5);
    a = *reinterpret_cast<const float4*>(src);
    b = *reinterpret_cast<const float4*>(src + 4);
    if (scale) {
      const float* sc = scale + 16 * s + 8 * (lane >> 5);
      a = mul4(a, *reinterpret_cast<const float4*>(sc));
      b = mul4(b, *reinterpret_cast<const float4*>(sc + 4));
    }
  }
  bf16x8 fh, fm, fl;
  split_frag(a, b, fh, fm, fl);
  uint4* dst = Wp + (size_t)((s * MT + mt) * 3) * 64 + lane;
  dst[0] = __builtin_bit_cast(uint4, fl);
  dst[64] = __builtin_bit_cast(uint4, fm);
  dst[128] = __builtin_bit_cast(uint4, fh);
}

// K-split router (E <= 64): a block of KS waves owns 32*NTW tokens; wave w
// computes all 32*MT experts of those tokens over the K range
// [w*2880/KS, (w+1)*2880/KS), holding NTW token tiles so that every weight
// fragment it loads feeds NTW MFMAs. The K loop is fully unrolled over a
// D-deep register ring (exact load accounting). The KS partial tiles meet in
// LDS and are added in wave order, then the bias, the top k and the routed-slot
// histograms of the block's 32-token groups.
template <int MT, int NTW, int KS>
struct RouteTileCfg {
  static constexpr int kSteps = kRouteSteps / KS;   // K steps of one wave
  static constexpr int kTB = 32 * NTW;              // tokens per block
  // partial-tile row: rows 4 apart (the two lane halves) land 32 banks apart
  // when it fits the LDS, else 16
  static constexpr int kLdr = kTB + (MT > 4 ? 4 : 8);
  static constexpr int kStageRegs = 4 * NTW + 12 * MT;
  // ring depth from the register budget: up to 224 VGPRs beside the
  // accumulators (which the compiler moves to AGPRs) at one wave per SIMD,
  // 168 in all at the three waves per SIMD of 12 K splits
  static constexpr int kRingRegs = KS > 4 ? 168 - 16 * NTW * MT - 32 : 224;
  static constexpr int kDepth = kRingRegs / kStageRegs > 8 ? 8
                                : kRingRegs / kStageRegs < 2 ? 2 : kRingRegs / kStageRegs;
  static constexpr int kRedFloats = KS * MT * 32 * kLdr;
  static_assert(kSteps * KS == kRouteSteps, "the K split must divide the K steps");
  static_assert(kRedFloats * 4 + kTB * kMaxTopK * 4 <= 160 * 1024, "LDS");
};

template <int MT, int NTW>
struct RTStage {
  uint4 xv[NTW];
  uint4 f[MT][3];
};

template <int MT, int NTW, int KS>
__global__ __launch_bounds__(KS * 64) void route_ksplit_kernel(
    const uint16_t* __restrict__ x, const uint4* __restrict__ Wp, const float* __restrict__ br,
    const float* __restrict__ inv, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, float* __restrict__ logits, int32_t* __restrict__ block_hist) {
  using C = RouteTileCfg<MT, NTW, KS>;
  constexpr int D = C::kDepth;
  constexpr int LDR = C::kLdr;
  constexpr int TB = C::kTB;
  __shared__ float red[C::kRedFloats];           // [KS][MT*32][LDR] partial logits
  __shared__ int32_t sel[TB * kMaxTopK];         // the block's chosen experts

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tok0 = blockIdx.x * TB;

  // padded tokens read a clamped valid row; their results are never used
  const uint16_t* xr[NTW];
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw)
    xr[tw] = x + (size_t)min(tok0 + 32 * tw + n, T - 1) * kH + wave * (C::kSteps * 16) + 8 * hh;
  const uint4* wp = Wp + (size_t)wave * C::kSteps * MT * 3 * 64 + lane;

  f32x16 acc[NTW][MT];
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[tw][mt] = f32x16{};

  RTStage<MT, NTW> st[D];
  auto load = [&](RTStage<MT, NTW>& S, int s) __attribute__((always_inline)) {
    // opaque step offsets: each step computes its own addresses instead of
    // the compiler keeping every step's pointers live
    int xo = 16 * s, wo = s * MT * 3 * 64;
    asm volatile("" : "+s"(xo), "+s"(wo));
#pragma unroll
    for (int tw = 0; tw < NTW; ++tw) S.xv[tw] = *reinterpret_cast<const uint4*>(xr[tw] + xo);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int p = 0; p < 3; ++p) S.f[mt][p] = wp[wo + (mt * 3 + p) * 64];
  };
  static_for<D>([&](auto Q) __attribute__((always_inline)) { load(st[Q], Q); });
  __builtin_amdgcn_sched_barrier(0);
  static_for<C::kSteps>([&](auto S) __attribute__((always_inline)) {
    constexpr int s = S;
    RTStage<MT, NTW>& cur = st[s % D];
    // pieces lo, mid, hi in turn; the NTW*MT accumulators in between keep
    // dependent MFMAs apart
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[tw][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              u4_as_bf16x8(cur.f[mt][p]), u4_as_bf16x8(cur.xv[tw]), acc[tw][mt], 0, 0, 0);
    if constexpr (s + D < C::kSteps) load(cur, s + D);
    __builtin_amdgcn_sched_barrier(0);
  });

  // partial tiles: red[wave][e][t]; 32x32 result layout: lane holds column n
  // (token), rows 8q + 4hh + j (experts)
  float* mine = red + (size_t)wave * MT * 32 * LDR;
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          mine[(mt * 32 + 8 * q + 4 * hh + j) * LDR + 32 * tw + n] = acc[tw][mt][4 * q + j];
  __syncthreads();
  // logits = partials added in wave order, then the bias; into slice 0
  for (int i = threadIdx.x; i < E * TB; i += KS * 64) {
    const int e = i / TB, t = i - (i / TB) * TB;
    float v = red[e * LDR + t];
#pragma unroll
    for (int w = 1; w < KS; ++w) v += red[(size_t)w * MT * 32 * LDR + e * LDR + t];
    if (inv) v *= inv[min(tok0 + t, T - 1)];   // the decoder block's norm
    v += br[e];
    red[e * LDR + t] = v;
    if (logits && tok0 + t < T) logits[(size_t)(tok0 + t) * E + e] = v;
  }
  __syncthreads();
  // top k: kTopkLanes lanes per token (the count of such lanes is a multiple
  // of 64, so every wave takes part in a round as a whole)
  for (int base = 0; base < TB * kTopkLanes; base += KS * 64) {
    const int i = base + threadIdx.x;
    if (i < TB * kTopkLanes) {
      const int tt = i / kTopkLanes;
      const int t = tok0 + tt;
      lanes_topk<kTopkLanes>(red + tt, LDR, E, k, t < T, ids + (size_t)t * k, wts + (size_t)t * k,
                             sel + tt * k);
    }
  }
  if (block_hist) {
    // expert histograms of the block's 32-token groups, for the parallel
    // permutation (the partial tiles are no longer needed)
    int* hist = reinterpret_cast<int*>(red);   // [NTW][E]
    __syncthreads();   // the top k has read its logits and written sel
    for (int i = threadIdx.x; i < NTW * E; i += KS * 64) hist[i] = 0;
    __syncthreads();
    const int nslots = (min(T, tok0 + TB) - tok0) * k;
    for (int i = threadIdx.x; i < nslots; i += KS * 64) atomicAdd(&hist[(i / (32 * k)) * E + sel[i]], 1);
    __syncthreads();
    const int groups = (T + 31) / 32;
    for (int i = threadIdx.x; i < NTW * E; i += KS * 64) {
      const int g = blockIdx.x * NTW + i / E;
      if (g < groups) block_hist[(size_t)g * E + i % E] = hist[i];
    }
  }
}

// Expert-tiled router (E > 64): a block of W waves owns 32*NTW tokens; wave
// w computes expert tiles [w*MTW, (w+1)*MTW) of them over all of K, so no
// partial sums cross waves and each logit is one fixed-order accumulation
// plus the bias. The block's activation rows pass through a two-slot LDS
// ring of 64-K groups (whole 128-byte lines per row, loaded two groups ahead
// into registers and shared by all waves); each wave streams only its own
// tiles' weight fragments through a register ring. One barrier per group.
template <int MTW, int W, int NTW>
struct RouteWideCfg {
  static constexpr int kTB = 32 * NTW;               // tokens per block
  static constexpr int kGroups = kH / 64;            // 45 groups of 4 K steps
  static constexpr int kPieces = kTB * 8;            // 16-byte pieces of a group
  static constexpr int kXLoads = (kPieces + W * 64 - 1) / (W * 64);
  static constexpr int kMTP = W * MTW;               // padded expert tiles
  static constexpr int kLdr = kTB + 8;               // logit row: lane halves 32 banks apart
  static constexpr int kStageRegs = 12 * MTW;
  static constexpr int kDepth = 96 / kStageRegs > 8 ? 8 : 96 / kStageRegs;
  static_assert(kGroups * 64 == kH, "groups must tile K");
};

// LDS byte offset of 16-byte piece p of row r in a group slot (rows of 128
// bytes; pieces XOR-swizzled by r/2 so that a 32-row fragment read is free of
// bank conflicts)
__device__ __forceinline__ int route_xs_off(int r, int p) { return r * 128 + ((p ^ ((r >> 1) & 7)) << 4); }

template <int MTW, int W, int NTW>
__global__ __launch_bounds__(W * 64) void route_tile_kernel(
    const uint16_t* __restrict__ x, const uint4* __restrict__ Wp, const float* __restrict__ br,
    const float* __restrict__ inv, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, float* __restrict__ logits, int32_t* __restrict__ block_hist) {
  using C = RouteWideCfg<MTW, W, NTW>;
  constexpr int D = C::kDepth;
  constexpr int TB = C::kTB;
  constexpr int LDR = C::kLdr;
  constexpr int MTP = C::kMTP;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TB * 128];   // activation group ring
  __shared__ float lg[MTP * 32 * LDR];                               // [expert][token] logits
  __shared__ int32_t sel[TB * kMaxTopK];                             // the block's chosen experts

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tok0 = blockIdx.x * TB;

  // activation pieces this thread stages: piece q = tid + i*W*64 of a group,
  // row q/8 (token, clamped to a valid row: padded tokens' results are never
  // used), 16-byte piece q%8; threads past the last piece load a valid
  // duplicate and skip the store
  const uint16_t* xsrc[C::kXLoads];
  int xdst[C::kXLoads];
#pragma unroll
  for (int i = 0; i < C::kXLoads; ++i) {
    const int q = tid + i * W * 64;
    const int qc = min(q, C::kPieces - 1);
    const int r = qc >> 3, p = qc & 7;
    xsrc[i] = x + (size_t)min(tok0 + r, T - 1) * kH + 8 * p;
    xdst[i] = q < C::kPieces ? route_xs_off(r, p) : -1;
  }
  // (compile-time indices throughout, so that the staging registers stay
  // registers and are never placed in memory)
  u32x4 xra[C::kXLoads], xrb[C::kXLoads];   // staging registers of alternate groups
  auto load_group = [&](u32x4 (&R)[C::kXLoads], int g) __attribute__((always_inline)) {
    int go = 64 * g;
    asm volatile("" : "+s"(go));
    static_for<C::kXLoads>([&](auto I) __attribute__((always_inline)) {
      R[I] = *reinterpret_cast<const u32x4*>(xsrc[I] + go);
    });
  };
  auto store_group = [&](const u32x4 (&R)[C::kXLoads], int slot) __attribute__((always_inline)) {
    static_for<C::kXLoads>([&](auto I) __attribute__((always_inline)) {
      if (xdst[I] >= 0) *reinterpret_cast<u32x4*>(&xs[slot][xdst[I]]) = R[I];
    });
  };
  // fragment of token tile tw, K step j of a group: row 32 tw + n, piece 2j + hh
  auto read_frags = [&](uint4 (&F)[NTW], int slot, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int tw = 0; tw < NTW; ++tw)
      F[tw] = *reinterpret_cast<const uint4*>(&xs[slot][route_xs_off(32 * tw + n, 2 * j + hh)]);
  };

  // this wave's weight fragments: tiles wave*MTW .. + MTW of every step
  const uint4* wp = Wp + (size_t)wave * MTW * 3 * 64 + lane;
  uint4 ring[D][MTW][3];
  auto load_w = [&](uint4 (&S)[MTW][3], int s) __attribute__((always_inline)) {
    int wo = s * MTP * 3 * 64;
    asm volatile("" : "+s"(wo));
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int p = 0; p < 3; ++p) S[m][p] = wp[wo + (m * 3 + p) * 64];
  };

  f32x16 acc[NTW][MTW];
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
    for (int m = 0; m < MTW; ++m) acc[tw][m] = f32x16{};

  // group barrier: this thread's LDS writes done, then the workgroup barrier
  // (no wait on the weight loads in flight)
  auto group_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");        // no LDS access moves across it
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: groups 0 and 1 into registers, group 0 into slot 0, group 2
  // into registers; the weight ring's first D steps
  load_group(xra, 0);
  load_group(xrb, 1);
  static_for<D>([&](auto Q) __attribute__((always_inline)) { load_w(ring[Q], Q); });
  store_group(xra, 0);
  load_group(xra, 2);
  group_sync();
  uint4 xf[2][NTW];
  read_frags(xf[0], 0, 0);

  static_for<C::kGroups>([&](auto G) __attribute__((always_inline)) {
    constexpr int g = G;
    // group g+1 into the other slot (its last readers passed the previous
    // barrier), and its registers refilled with group g+3
    auto& xr = [&]() -> auto& { if constexpr ((g + 1) & 1) return xrb; else return xra; }();
    if constexpr (g + 1 < C::kGroups) store_group(xr, (g + 1) & 1);
    if constexpr (g + 3 < C::kGroups) load_group(xr, g + 3);
    static_for<4>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = J;
      constexpr int s = 4 * g + j;
      const uint4 (&cur)[NTW] = xf[s & 1];
      // pieces lo, mid, hi in turn; the NTW*MTW accumulators in between
      // keep dependent MFMAs apart
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int tw = 0; tw < NTW; ++tw)
#pragma unroll
          for (int m = 0; m < MTW; ++m)
            acc[tw][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                u4_as_bf16x8(ring[s % D][m][p]), u4_as_bf16x8(cur[tw]), acc[tw][m], 0, 0, 0);
      if constexpr (s + D < kRouteSteps) load_w(ring[s % D], s + D);
      if constexpr (j < 3) {
        read_frags(xf[(s + 1) & 1], g & 1, j + 1);
      } else if constexpr (g + 1 < C::kGroups) {
        group_sync();   // group g+1 is in its slot; everyone is done with slot g&1
        read_frags(xf[(s + 1) & 1], (g + 1) & 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });

  // logits (+ bias) into LDS; 32x32 result layout: lane holds column n
  // (token), rows 8q + 4hh + j (experts)
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw) {
    // the decoder block's norm: the token's inverse RMS
    const float iv = inv ? inv[min(tok0 + 32 * tw + n, T - 1)] : 1.f;
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 32 * (wave * MTW + m) + 8 * q + 4 * hh + j;
          const float a = inv ? acc[tw][m][4 * q + j] * iv : acc[tw][m][4 * q + j];
          lg[e * LDR + 32 * tw + n] = a + (e < E ? br[e] : 0.f);
        }
  }
  __syncthreads();
  if (logits) {
    for (int i = tid; i < E * TB; i += W * 64) {
      const int e = i / TB, t = i - (i / TB) * TB;
      if (tok0 + t < T) logits[(size_t)(tok0 + t) * E + e] = lg[e * LDR + t];
    }
  }
  // top k: kTopkLanes lanes per token (a multiple of 64 lanes per round, so
  // every wave takes part in a round as a whole)
  for (int base = 0; base < TB * kTopkLanes; base += W * 64) {
    const int i = base + tid;
    if (i < TB * kTopkLanes) {
      const int tt = i / kTopkLanes;
      const int t = tok0 + tt;
      lanes_topk<kTopkLanes>(lg + tt, LDR, E, k, t < T, ids + (size_t)t * k, wts + (size_t)t * k,
                             sel + tt * k);
    }
  }
  if (block_hist) {
    // expert histograms of the block's 32-token groups, for the parallel
    // permutation (the logits are no longer needed)
    int* hist = reinterpret_cast<int*>(lg);   // [NTW][E]
    __syncthreads();   // the top k has read its logits and written sel
    for (int i = tid; i < NTW * E; i += W * 64) hist[i] = 0;
    __syncthreads();
    const int nslots = (min(T, tok0 + TB) - tok0) * k;
    for (int i = tid; i < nslots; i += W * 64) atomicAdd(&hist[(i / (32 * k)) * E + sel[i]], 1);
    __syncthreads();
    const int groups = (T + 31) / 32;
    for (int i = tid; i < NTW * E; i += W * 64) {
      const int g = blockIdx.x * NTW + i / E;
      if (g < groups) block_hist[(size_t)g * E + i % E] = hist[i];
    }
  }
}

// ---------------------------------------------------------------- few tokens
// RMSNorm folded in (NORM, the decoder block, "gpt-oss-20b" page,
// "Structure": RMSNorm_i_2 feeds MoE_i): the router's input is t = x * inv *
// scale with inv = 1 / sqrt(mean(x^2) + eps) per token, so t . Wr[e] =
// inv * (x . (Wr[e] * scale)). The chunk waves multiply x by the scaled
// weights and also write their tokens' chunk sums of x^2 (ss, [chunk][T]);
// the finish kernels add those in chunk order, form inv and scale the logits
// by it. No kernel waits for a token's whole row before its products.
template <int MT, bool NORM>
__global__ __launch_bounds__(64) void route_partial_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ Wr,
                                                           const float* __restrict__ scale, int T,
                                                           int E, float* __restrict__ partial,
                                                           float* __restrict__ ss_partial) {
  const int lane = threadIdx.x;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tok = blockIdx.x * 32 + n;
  const int kc = blockIdx.y;
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
  float ss = 0.f;
  RouteLoader<MT, NORM> L;
  L.init(x, Wr, scale, T, E, tok, kc * kRouteChunkSteps * 16, lane);
  route_kloop<MT, kRouteChunkSteps, NORM>(L, acc, ss);
  if (NORM) ss += __shfl_xor(ss, 32, 64);   // the two K halves of the token, lane order fixed
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
    if (NORM && ss_partial && hh == 0) ss_partial[(size_t)kc * T + tok] = ss;
  }
}

// The norm's inverse RMS of token t from the chunk sums of squares, added in
// chunk order.
__device__ __forceinline__ float route_inv_rms(const float* __restrict__ ss_partial, int T, int t,
                                               float eps) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kRouteChunks; ++c) ss += ss_partial[(size_t)c * T + t];
  return 1.0f / sqrtf(ss / (float)kH + eps);
}

// Norm arguments of the finish kernels: with `ss` the inverse RMS is formed
// from the chunk sums; without `ss` but with `inv` it is read from there;
// with neither the logits are not scaled.
struct RouteFinishNorm {
  const float* ss;
  float eps;
  const float* inv;
  __device__ __forceinline__ float get(int T, int t) const {
    if (ss) return route_inv_rms(ss, T, t, eps);
    return inv ? inv[t] : 1.f;
  }
};

// One 1024-thread block: logits = bias + sum of the chunk partials in chunk
// order (one thread per (token, expert) pair, all partial loads in flight at
// once), then the top k of each token by rank, the softmax, and the expert
// permutation of the T*k slots.
template <int PAIRS>
__global__ __launch_bounds__(kPermThreads) void route_finish_kernel(
    const float* __restrict__ partial, const float* __restrict__ br, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
    RouteFinishNorm nrm) {
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
      const float v = (nrm.ss || nrm.inv) ? acc[j] * nrm.get(T, t) + bias[j] : acc[j] + bias[j];
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

// The decoder block's normed rows t = bf16(x * inv * scale) from the chunk
// sums of squares, one wave per row (the norm kernel's arithmetic, with the
// router's inverse RMS).
__device__ __forceinline__ void route_write_normed_row(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ scale,
                                                       const RouteFinishNorm& nrm, int T, int row,
                                                       uint16_t* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const float inv = nrm.get(T, row);
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * kH);
  uint4* tr = reinterpret_cast<uint4*>(t + (size_t)row * kH);
  const float4* sc = reinterpret_cast<const float4*>(scale);
#pragma unroll
  for (int j = 0; j < (kH / 8 + 63) / 64; ++j) {
    const int i = lane + 64 * j;
    if (i < kH / 8) tr[i] = norm_apply8(xr[i], inv, sc[2 * i], sc[2 * i + 1]);
  }
}

// The same sums, top-k and softmax as route_finish_kernel without the
// permutation, spread over blocks of 256 / E tokens each (one thread per
// (token, expert) pair), so that the partial-logit loads of a decode batch
// run on many CUs instead of one. Arithmetic in the same order: identical
// expert choices and weights. With `t_out` (the decoder block), blocks from
// `nfin` on write the normed rows instead, four per block, so the block needs
// no separate norm launch.
__global__ __launch_bounds__(256) void route_finish_tiles_kernel(
    const float* __restrict__ partial, const float* __restrict__ br, int T, int E, int k, int tb,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ logits,
    RouteFinishNorm nrm, int nfin, const uint16_t* __restrict__ x, const float* __restrict__ nscale,
    uint16_t* __restrict__ t_out) {
  if ((int)blockIdx.x >= nfin) {
    const int row = ((int)blockIdx.x - nfin) * 4 + (int)(threadIdx.x >> 6);
    if (row < T) route_write_normed_row(x, nscale, nrm, T, row, t_out);
    return;
  }
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
    if (nrm.ss || nrm.inv) acc *= nrm.get(T, t0 + tid / E);
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
                          int32_t* sorted_rows, const RouteFinishNorm& fn, hipStream_t s) {
  const int pairs = (T * E + kPermThreads - 1) / kPermThreads;
#define MOE_FINISH(P)                                                                             \
  hipLaunchKernelGGL((route_finish_kernel<P>), dim3(1), dim3(kPermThreads), 0, s, scratch,          \
                     br, T, E, k, ids, w, logits, counts, offsets, sorted_rows, fn)
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
                                  int32_t* sorted_rows, const RouteNorm* norm, hipStream_t s) {
  if (few_tokens(T, E)) {
    const dim3 grid((T + 31) / 32, kRouteChunks);
    // the chunk sums of squares follow the partial logits
    float* ss = norm && !norm->inv_ready ? scratch + (size_t)kRouteChunks * T * E : nullptr;
    if (norm)
      hipLaunchKernelGGL((route_partial_kernel<MT, true>), grid, dim3(64), 0, s, x, Wr, norm->scale, T, E,
                         scratch, ss);
    else
      hipLaunchKernelGGL((route_partial_kernel<MT, false>), grid, dim3(64), 0, s, x, Wr, nullptr, T, E,
                         scratch, nullptr);
    const RouteFinishNorm fn{ss, norm ? norm->eps : 0.f, norm ? norm->inv : nullptr};
    uint16_t* t_out = ss ? norm->t_out : nullptr;   // the normed rows, from the router's sums
    if (counts) {
      if (t_out) return hipErrorInvalidValue;
      launch_finish(scratch, br, T, E, k, ids, w, logits, counts, offsets, sorted_rows, fn, s);
    } else {
      const int tb = 256 / E;   // tokens per block; E <= 256
      const int nfin = (T + tb - 1) / tb;
      const int nwrite = t_out ? (T + 3) / 4 : 0;
      hipLaunchKernelGGL(route_finish_tiles_kernel, dim3(nfin + nwrite), dim3(256), 0, s, scratch, br,
                         T, E, k, tb, ids, w, logits, fn, nfin, x, norm ? norm->scale : nullptr, t_out);
    }
    return hipGetLastError();
  }
  // many tokens: the norm's inverse RMS comes from the norm kernel
  if (norm && (!norm->inv_ready || !norm->inv)) return hipErrorInvalidValue;
  const float* nscale = norm ? norm->scale : nullptr;
  const float* ninv = norm ? norm->inv : nullptr;
  // split weights first (16-byte aligned: a multiple of 1 KiB), then the histograms
  constexpr int MTP = route_tiles_padded(MT);
  uint4* wp = reinterpret_cast<uint4*>(scratch);
  int32_t* hist = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(scratch) + route_split_bytes(E));
  hipLaunchKernelGGL(route_split_kernel, dim3((kRouteSteps * MTP * 64 + 255) / 256), dim3(256), 0, s,
                     Wr, nscale, E, MTP, wp);
  int32_t* bh = counts ? hist : nullptr;
  if constexpr (MT <= 2) {
    // few expert tiles: waves split K (little work per wave and step)
    hipLaunchKernelGGL((route_ksplit_kernel<MT, 1, 12>), dim3((T + 31) / 32), dim3(12 * 64), 0, s, x,
                       wp, br, ninv, T, E, k, ids, w, logits, bh);
  } else {
    // a wave per one or two expert tiles; two token tiles per wave (half the
    // weight traffic per token) once 64-token blocks alone fill the chip
    constexpr int MTW = MT <= 4 ? 1 : 2;
    constexpr int WV = MTP / MTW;
    if ((T + 63) / 64 >= kRouteTwoTileBlocks)
      hipLaunchKernelGGL((route_tile_kernel<MTW, WV, 2>), dim3((T + 63) / 64), dim3(WV * 64), 0, s, x,
                         wp, br, ninv, T, E, k, ids, w, logits, bh);
    else
      hipLaunchKernelGGL((route_tile_kernel<MTW, WV, 1>), dim3((T + 31) / 32), dim3(WV * 64), 0, s, x,
                         wp, br, ninv, T, E, k, ids, w, logits, bh);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !counts) return err;
  return launch_permute_blocks(ids, T * k, E, hist, (T + 31) / 32, 32 * k, counts, offsets,
                               sorted_rows, s);
}

hipError_t launch_route(const uint16_t* x, const float* Wr, const float* br, int T, int E, int k,
                        int32_t* ids, float* w, float* logits, float* scratch,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                        const RouteNorm* norm, hipStream_t s) {
#define MOE_ROUTE(M)                                                                                \
  case M:                                                                                           \
    return launch_route_mt<M>(x, Wr, br, T, E, k, ids, w, logits, scratch, counts, offsets,         \
                              sorted_rows, norm, s)
  switch ((E + 31) / 32) {
    MOE_ROUTE(1);
    MOE_ROUTE(2);
    MOE_ROUTE(3);
    MOE_ROUTE(4);
    MOE_ROUTE(5);
    MOE_ROUTE(6);
    MOE_ROUTE(7);
    MOE_ROUTE(8);
    default: return hipErrorInvalidValue;
  }
#undef MOE_ROUTE
}

}  // namespace moe
