// Router GEMM + in-register top-k + softmax over the selected logits.
//
// logits[t, e] = sum_h x[t, h] Wr[e, h] + br[e]  (gpt-oss-120b techniques map,
// "Checked in its code" table, row "Auxiliary-loss-free load balancing": the
// router is a linear layer with a bias; row "Mixture of experts": top-k over
// the router logits, then softmax over the selected ones).
//
// fp32 router on bf16 matrix cores: x is bf16, and each fp32 weight is split
// exactly into three bf16 pieces (hi + mid + lo, 8 significant bits each).
// Every product x * piece is exact in fp32, and the matrix core accumulates in
// fp32, so the result is an fp32-accumulated dot product of the fp32 weights.
// Block = 32 tokens; its waves split K and their partial sums are added in a
// fixed wave order through LDS (deterministic).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

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

struct Cand {
  float v;
  int id;
};

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// MT = ceil(E / 32) expert tiles, WK = waves splitting K.
template <int MT, int WK>
__global__ __launch_bounds__(WK * 64) void route_kernel(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ Wr,
                                                        const float* __restrict__ br, int T, int E,
                                                        int k, int32_t* __restrict__ ids,
                                                        float* __restrict__ wts,
                                                        float* __restrict__ logits,
                                                        float* __restrict__ zero_out) {
  constexpr int KW = kH / WK;      // K range of one wave
  constexpr int KSTEPS = KW / 16;  // 16-deep MFMA steps per wave
  constexpr int LDR = 33;          // padded row of the reduction buffer
  static_assert(KW % 16 == 0, "K split must be a multiple of 16");
  extern __shared__ float red[];   // [MT * 32][LDR]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * 32;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int tok = tok0 + n;
  const bool tok_ok = tok < T;

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};

  const uint16_t* xrow = x + (size_t)(tok_ok ? tok : 0) * kH + wave * KW + 8 * hh;
  const float* wrow[MT];
  bool e_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int e = mt * 32 + n;
    e_ok[mt] = e < E;
    wrow[mt] = Wr + (size_t)(e_ok[mt] ? e : 0) * kH + wave * KW + 8 * hh;
  }

#pragma unroll 3
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 xv = make_uint4(0, 0, 0, 0);
    if (tok_ok) xv = *reinterpret_cast<const uint4*>(xrow + 16 * s);
    const bf16x8 xb = u4_as_bf16x8(xv);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (e_ok[mt]) {
        a = *reinterpret_cast<const float4*>(wrow[mt] + 16 * s);
        b = *reinterpret_cast<const float4*>(wrow[mt] + 16 * s + 4);
      }
      bf16x8 fh, fm, fl;
      split_frag(a, b, fh, fm, fl);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, xb, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fm, xb, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh, xb, acc[mt], 0, 0, 0);
    }
  }

  // Fixed-order split-K reduction: red[e][token] = sum over waves 0..WK-1.
  // Result layout of the 32x32 tile: lane holds column n (token) and rows
  // 8q + 4*hh + j (experts) in element 4q + j.
  for (int w = 0; w < WK; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = mt * 32 + 8 * q + 4 * hh + j;
            float* p = &red[m * LDR + n];
            *p = (w == 0) ? acc[mt][4 * q + j] : (*p + acc[mt][4 * q + j]);
          }
    }
    __syncthreads();
  }

  // Top-k, one wave per token: lane holds experts lane + 64q.
  for (int tt = wave; tt < 32; tt += WK) {
    const int t = tok0 + tt;
    if (t >= T) break;
    float v[4];
    int id[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        v[q] = red[e * LDR + tt] + br[e];
        id[q] = e;
        if (logits) logits[(size_t)t * E + e] = v[q];
      } else {
        v[q] = -INFINITY;
        id[q] = 0x7FFFFFFF;
      }
    }
    float sel_v[kMaxTopK];
    int sel_i[kMaxTopK];
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
      if (r < k) {
        float bv = v[0];
        int bi = id[0];
#pragma unroll
        for (int q = 1; q < 4; ++q)
          if (better(v[q], id[q], bv, bi)) { bv = v[q]; bi = id[q]; }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
          const float ov = __shfl_xor(bv, d, 64);
          const int oi = __shfl_xor(bi, d, 64);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        sel_v[r] = bv;
        sel_i[r] = bi;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (id[q] == bi) { v[q] = -INFINITY; id[q] = 0x7FFFFFFF; }
      }
    }
    // softmax over the k selected logits (sel_v[0] is the largest)
    float z = 0.f;
    float ex[kMaxTopK];
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
      ex[r] = (r < k) ? __expf(sel_v[r] - sel_v[0]) : 0.f;
      z += ex[r];
    }
    const float inv = 1.0f / z;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
      if (r < k && lane == r) {
        ids[(size_t)t * k + r] = sel_i[r];
        wts[(size_t)t * k + r] = ex[r] * inv;
      }
    }
  }

  // Optionally clear this block's rows of the layer output (the fused down
  // projection accumulates into it).
  if (zero_out) {
    const int rows = min(32, T - tok0);
    float4* o = reinterpret_cast<float4*>(zero_out + (size_t)tok0 * kH);
    const int n4 = rows * (kH / 4);
    for (int i = threadIdx.x; i < n4; i += WK * 64) o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int MT, int WK>
static hipError_t launch_route_t(const uint16_t* x, const float* Wr, const float* br, int T, int E,
                                 int k, int32_t* ids, float* w, float* logits, float* zero_out,
                                 hipStream_t s) {
  const int blocks = (T + 31) / 32;
  const size_t lds = (size_t)MT * 32 * 33 * sizeof(float);
  hipLaunchKernelGGL((route_kernel<MT, WK>), dim3(blocks), dim3(WK * 64), lds, s, x, Wr, br, T, E,
                     k, ids, w, logits, zero_out);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, const float* Wr, const float* br, int T, int E, int k,
                        int32_t* ids, float* w, float* logits, float* zero_out, hipStream_t s) {
  const int mt = (E + 31) / 32;
  const int blocks = (T + 31) / 32;
  // Few token blocks: split K over 12 waves to spread the work; many: 4 waves.
  const bool wide = blocks < 256 && mt <= 4;
#define MOE_ROUTE_CASE(M)                                                                   \
  case M:                                                                                   \
    return wide ? launch_route_t<(M <= 4 ? M : 4), 12>(x, Wr, br, T, E, k, ids, w, logits, \
                                                       zero_out, s)                         \
                : launch_route_t<M, 4>(x, Wr, br, T, E, k, ids, w, logits, zero_out, s);
  switch (mt) {
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(3)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(5)
    MOE_ROUTE_CASE(6)
    MOE_ROUTE_CASE(7)
    MOE_ROUTE_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_CASE
}

}  // namespace moe
