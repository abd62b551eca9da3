// Grouped expert GEMMs over MXFP4 weights with fused epilogues.
//
// Gate/up: gu = x W13[e]^T + b13[e], then the gpt-oss gated unit
//   h = (clamp(up, -7, 7) + 1) * min(gate, 7) * sigmoid(1.702 * min(gate, 7))
// (gpt-oss-120b techniques map, "Checked in its code", row "SwiGLU
// feed-forward"; swiglu_limit = 7 from the raw config.json tables).
// Down: y = h W2[e]^T + b2[e], either stored per routed slot or multiplied
// by the routing weight and added into the token's output row (the weighted
// sum over the selected experts, row "Mixture of experts").
//
// Weights are MXFP4 (techniques map, "inference & serving": MXFP4 weight
// quantization / tensor packing): a lane loads one whole 32-element block (16
// code bytes, one 128-bit load) plus its E8M0 byte and converts it to bf16 in
// registers with v_cvt_scalef32_pk_bf16_fp4, which is exact for the scale
// range the library supports. Products run on bf16 matrix cores with fp32
// accumulation. The K index assignment inside a matrix-core step is free as
// long as both operands agree: a lane's 32 weight values (one block) meet the
// 32 activation values of the same K range.
//
// Two schedules:
//  * weight-streaming ("skinny"), for few rows per expert (decode): one wave
//    owns 64 weight rows of one expert and <= 16 of its tokens, streams the
//    rows' blocks with a 3-step register prefetch and reads its activations
//    straight from global memory (L2-resident). 16x16x32 bf16 MFMA with the
//    weights as the 16-row operand.
//  * tiled ("wide"), for many rows per expert (prefill): a 256-thread block
//    owns 256 weight rows x 128 tokens; the gathered activation tile goes
//    through a double-buffered LDS ring (64 K per step), weights go straight
//    to registers. 32x32x16 bf16 MFMA.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ------------------------------------------------------------------ skinny
constexpr int kSkRows = 64;    // weight rows per wave (four 16-row tiles)
constexpr int kSkBT = 16;      // tokens per tile
constexpr int kSkSteps = 23;   // ceil(90 blocks / 4 lane groups)
constexpr int kSkDepth = 3;    // prefetch depth in steps

struct SkStage {
  uint4 w[4];
  uint32_t sc[4];
  uint4 xv[4];
};

template <int EPI>
__global__ __launch_bounds__(64) void ffn_skinny_kernel(FfnArgs a) {
  const int lane = threadIdx.x;
  int e, rb, re;
  if (!find_tile(a.offsets, a.E, kSkBT, blockIdx.y, e, rb, re)) return;
  const int row_base = blockIdx.x * kSkRows;
  const int r = lane & 15;   // weight row in a 16-row tile / token column
  const int g = lane >> 4;   // lane group: owns MX block 4s + g in step s
  const int p = rb + r;
  const bool tok_ok = p < re;
  const int slot = tok_ok ? a.sorted_rows[p] : 0;
  const int arow = a.gather ? slot / a.k : p;
  const uint16_t* xp = a.act + (size_t)(tok_ok ? arow : 0) * kH;
  const size_t wrow0 = (size_t)e * a.N + row_base + r;
  const uint8_t* cp = a.codes + wrow0 * kRowCodeBytes;
  const uint8_t* sp = a.scales + wrow0 * kRowScaleBytes;

  auto issue = [&](SkStage& st, int s) {
    const int kb = 4 * s + g;
    const bool k_ok = kb < kKB;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      st.w[mt] = make_uint4(0, 0, 0, 0);
      st.sc[mt] = 127;
      if (k_ok) {
        st.w[mt] = *reinterpret_cast<const uint4*>(cp + (size_t)mt * 16 * kRowCodeBytes + kb * 16);
        st.sc[mt] = sp[(size_t)mt * 16 * kRowScaleBytes + kb];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.xv[i] = make_uint4(0, 0, 0, 0);
      if (k_ok && tok_ok) st.xv[i] = *reinterpret_cast<const uint4*>(xp + kb * 32 + 8 * i);
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const SkStage& st) {
    float sf[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sf[mt] = e8m0_to_f32(st.sc[mt]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 xb = u4_as_bf16x8(st.xv[i]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t wd = i == 0 ? st.w[mt].x : i == 1 ? st.w[mt].y : i == 2 ? st.w[mt].z : st.w[mt].w;
        const bf16x8 wb = fp4x8_to_bf16x8(wd, sf[mt]);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb, acc[mt], 0, 0, 0);
      }
    }
  };

  SkStage st[kSkDepth];
#pragma unroll
  for (int q = 0; q < kSkDepth; ++q) issue(st[q], q);
  for (int s0 = 0; s0 < kSkSteps; s0 += kSkDepth) {
#pragma unroll
    for (int q = 0; q < kSkDepth; ++q) {
      const int s = s0 + q;
      if (s < kSkSteps) {
        compute(st[q]);
        if (s + kSkDepth < kSkSteps) issue(st[q], s + kSkDepth);
      }
    }
  }

  // 16x16 result: lane holds token column r and weight rows 4g + j.
  const uint16_t* bias = a.bias + (size_t)e * a.N;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int R0 = row_base + 16 * mt + 4 * g;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[mt][j] + bf16_bits_to_f32(bias[R0 + j]);
    if (!tok_ok) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      const uint32_t h0 = f32_to_bf16_bits(swiglu_pair(v[0], v[1]));
      const uint32_t h1 = f32_to_bf16_bits(swiglu_pair(v[2], v[3]));
      *reinterpret_cast<uint32_t*>(a.h_out + (size_t)p * kI + R0 / 2) = h0 | (h1 << 16);
    } else if constexpr (EPI == EPI_COMBINE) {
      const float wt = a.topk_w[slot];
      float* o = a.out + (size_t)(slot / a.k) * kH + R0;
#pragma unroll
      for (int j = 0; j < 4; ++j) unsafeAtomicAdd(o + j, wt * v[j]);
    } else {
      *reinterpret_cast<float4*>(a.y_out + (size_t)slot * kH + R0) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------------ wide
constexpr int kWdBT = 128;      // tokens per tile
constexpr int kWdRows = 256;    // weight rows per block (4 waves x 64)
constexpr int kWdSteps = 45;    // K = 2880 in steps of 64 (two MX blocks)
constexpr int kXsStride = 72;   // bf16 per LDS activation row (64 + 8 pad)

template <int EPI, bool W_AS_B>
__global__ __launch_bounds__(256) void ffn_wide_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kWdBT * kXsStride];
  __shared__ int slot_of[kWdBT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int e, rb, re;
  if (!find_tile(a.offsets, a.E, kWdBT, blockIdx.y, e, rb, re)) return;
  const int row_w = blockIdx.x * kWdRows + wave * 64;
  const bool w_ok = row_w < a.N;
  if (tid < kWdBT) {
    const int p = rb + tid;
    slot_of[tid] = p < re ? a.sorted_rows[p] : -1;
  }

  // activation loader: chunk c = tid + 256q -> token (tid >> 3) + 32q, 16-byte piece tid & 7
  const int piece = tid & 7;
  const uint16_t* gptr[4];
  bool gok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tt = (tid >> 3) + 32 * q;
    const int p = rb + tt;
    gok[q] = p < re;
    int row = 0;
    if (gok[q]) row = a.gather ? a.sorted_rows[p] / a.k : p;
    gptr[q] = a.act + (size_t)row * kH + piece * 8;
  }
  uint4 xr[4];
  auto load_x = [&](int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xr[q] = make_uint4(0, 0, 0, 0);
      if (gok[q]) xr[q] = *reinterpret_cast<const uint4*>(gptr[q] + s * 64);
    }
  };
  auto store_x = [&](int stage) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tt = (tid >> 3) + 32 * q;
      *reinterpret_cast<uint4*>(&xs[stage][tt * kXsStride + piece * 8]) = xr[q];
    }
  };

  // weight rows of this wave: tile mt covers rows row_w + 32mt + (lane & 31)
  const int r32 = lane & 31;
  const int hh = lane >> 5;   // lane half: owns MX block 2s + hh in step s
  const size_t wrow0 = (size_t)e * a.N + (w_ok ? row_w : 0) + r32;
  const uint8_t* cp = a.codes + wrow0 * kRowCodeBytes;
  const uint8_t* sp = a.scales + wrow0 * kRowScaleBytes;
  uint4 wq[2][2];
  uint32_t wsc[2][2];
  auto load_w = [&](int buf, int s) {
    const int kb = 2 * s + hh;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      wq[buf][mt] = *reinterpret_cast<const uint4*>(cp + (size_t)mt * 32 * kRowCodeBytes + kb * 16);
      wsc[buf][mt] = sp[(size_t)mt * 32 * kRowScaleBytes + kb];
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};

  auto compute = [&](int stage, int buf) {
    const uint16_t* xsb = xs[stage];
    float sf[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) sf[mt] = e8m0_to_f32(wsc[buf][mt]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 xf[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        xf[nt] = *reinterpret_cast<const bf16x8*>(&xsb[(32 * nt + r32) * kXsStride + 32 * hh + 8 * i]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint4 w4 = wq[buf][mt];
        const uint32_t wd = i == 0 ? w4.x : i == 1 ? w4.y : i == 2 ? w4.z : w4.w;
        const bf16x8 wf = fp4x8_to_bf16x8(wd, sf[mt]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if constexpr (W_AS_B)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[nt], wf, acc[mt][nt], 0, 0, 0);
          else
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
  };

  load_x(0);
  store_x(0);
  load_x(1);
  if (w_ok) {
    load_w(0, 0);
    load_w(1, 1);
  }
  __syncthreads();
  for (int s0 = 0; s0 < kWdSteps; s0 += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int s = s0 + q;
      if (s < kWdSteps) {
        if (s + 1 < kWdSteps) store_x(q ^ 1);
        if (s + 2 < kWdSteps) load_x(s + 2);
        if (w_ok) {
          compute(q, q);
          if (s + 2 < kWdSteps) load_w(q, s + 2);
        }
        __syncthreads();
      }
    }
  }
  if (!w_ok) return;

  const uint16_t* bias = a.bias + (size_t)e * a.N;
  if constexpr (!W_AS_B) {
    // D[weight row][token]: lane holds token column r32, rows 8q + 4hh + j
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int R0 = row_w + 32 * mt + 8 * q + 4 * hh;
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = bf16_bits_to_f32(bias[R0 + j]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int p = rb + 32 * nt + r32;
          if (p >= re) continue;
          const f32x16& c = acc[mt][nt];
          const uint32_t h0 = f32_to_bf16_bits(swiglu_pair(c[4 * q] + b[0], c[4 * q + 1] + b[1]));
          const uint32_t h1 = f32_to_bf16_bits(swiglu_pair(c[4 * q + 2] + b[2], c[4 * q + 3] + b[3]));
          *reinterpret_cast<uint32_t*>(a.h_out + (size_t)p * kI + R0 / 2) = h0 | (h1 << 16);
        }
      }
    }
  } else {
    // D[token][weight row]: lane holds weight row (output feature) r32,
    // tokens 8q + 4hh + j of the 32-token tile
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int f = row_w + 32 * mt + r32;
      const float bf = bf16_bits_to_f32(bias[f]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int slot = slot_of[32 * nt + 8 * q + 4 * hh + j];
            if (slot < 0) continue;
            const float v = acc[mt][nt][4 * q + j] + bf;
            if constexpr (EPI == EPI_COMBINE) {
              unsafeAtomicAdd(a.out + (size_t)(slot / a.k) * kH + f, a.topk_w[slot] * v);
            } else {
              a.y_out[(size_t)slot * kH + f] = v;
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
constexpr int kSkinnyMaxMeanRows = 24;

hipError_t launch_ffn(const FfnArgs& a, Epilogue epi, int n_rows, hipStream_t s) {
  const bool skinny = (long long)n_rows <= (long long)kSkinnyMaxMeanRows * a.E;
  if (skinny) {
    const int tiles = (n_rows + kSkBT - 1) / kSkBT + min(a.E, n_rows);
    const dim3 grid(a.N / kSkRows, tiles);
    switch (epi) {
      case EPI_SWIGLU: hipLaunchKernelGGL(ffn_skinny_kernel<EPI_SWIGLU>, grid, dim3(64), 0, s, a); break;
      case EPI_COMBINE: hipLaunchKernelGGL(ffn_skinny_kernel<EPI_COMBINE>, grid, dim3(64), 0, s, a); break;
      default: hipLaunchKernelGGL(ffn_skinny_kernel<EPI_STORE_Y>, grid, dim3(64), 0, s, a); break;
    }
  } else {
    const int tiles = (n_rows + kWdBT - 1) / kWdBT + min(a.E, n_rows);
    const dim3 grid((a.N + kWdRows - 1) / kWdRows, tiles);
    switch (epi) {
      case EPI_SWIGLU: hipLaunchKernelGGL((ffn_wide_kernel<EPI_SWIGLU, false>), grid, dim3(256), 0, s, a); break;
      case EPI_COMBINE: hipLaunchKernelGGL((ffn_wide_kernel<EPI_COMBINE, true>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((ffn_wide_kernel<EPI_STORE_Y, true>), grid, dim3(256), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
