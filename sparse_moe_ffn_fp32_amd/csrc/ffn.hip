// Grouped expert GEMMs over packed MXFP4 weights with fused epilogues.
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
// quantization, MXFP4 tensor packing) in the library's packed order (see
// moe_pack_weights in moe.h): inside each group of 64 rows, the bytes come in
// the order the matrix-core lanes consume them, so every weight load of a wave
// is contiguous 256-byte runs or better (16 code bytes per lane). Each lane
// converts its 32 codes of one MX block to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp4, exact for the supported scales); the
// activation operand supplies the same K values, so each MFMA sums over a
// permutation of K that both operands share.
//
// Two schedules:
//  * weight-streaming ("skinny", few rows per expert: decode). A workgroup
//    of three waves owns three 64-row groups of one expert and its tokens,
//    16 at a time, on 16x16x32 MFMAs (weights the 16-row operand); each wave
//    streams its group's code bytes front to back (non-temporal loads,
//    3-step register prefetch), and the workgroup loads each K step's
//    activation tile once into an LDS ring that all three waves read. In the
//    layer's own schedule the waves find their expert's slots in the routing
//    ids; through the standalone entry points they read offsets / sorted_rows.
//  * tiled (many rows per expert: prefill), ffn_tile_kernel. A block of 8
//    waves owns 512 weight rows (one 64-row group per wave) x 128 tokens of
//    one expert, each wave a 64 x 128 tile of 32x32x16 bf16 MFMAs; the
//    gathered activation rows go global -> LDS by DMA through a 4-stage ring
//    (three K steps ahead), the weights straight to registers (two steps
//    ahead). The work (column block, token tile) is split over the 8 XCDs in
//    equal contiguous ranges. Its block-scaled variant (ffn_wide6_kernel, 4
//    waves x 64 tokens) reads the activations as two-piece MX FP6 records and
//    feeds them, with the packed FP4 weights unconverted, to the FP4 x FP6
//    matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
#include "moe_device.h"
#include "moe_launch.h"


namespace moe {

// ------------------------------------------------------------------ packing
// canonical [E, N, 1440] codes + [E, N, 90] scales -> packed order (a byte
// permutation inside every 64-row group). One thread per (row, MX block).
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   long long units, uint8_t* __restrict__ pcodes,
                                                   uint8_t* __restrict__ pscales) {
  const long long u = (long long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int kb = (int)(u % kKB);
  const long long row = u / kKB;         // e * N + n
  const long long grp = row >> 6;
  const int rin = (int)(row & 63);
  const int m = rin >> 4, r = rin & 15;
  const int s = kb >> 2, g = kb & 3;
  const int l = 16 * g + r;
  const long long dst = grp * kGroupCodeBytes + (long long)s * kStepCodeBytes +
                        m * (s < kFullSteps ? 1024 : 512) + l * 16;
  *reinterpret_cast<uint4*>(pcodes + dst) = *reinterpret_cast<const uint4*>(codes + u * 16);
  pscales[grp * kGroupScaleBytes + s * 256 + l * 4 + m] = scales[u];
}

hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int E, int N,
                       uint8_t* pcodes, uint8_t* pscales, hipStream_t s) {
  const long long units = (long long)E * N * kKB;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, codes, scales, units, pcodes, pscales);
  return hipGetLastError();
}

// Weight fragment loader of one wave over one packed 64-row group. Loads are
// unconditional (branch-free, so the compiler can count outstanding loads
// exactly): in the half last step, lanes 32..63 re-read lanes 0..31's bytes
// and their codes are replaced by zeros.
struct GroupStream {
  const uint8_t* cg;   // codes of the group + lane * 16
  const uint8_t* sg;   // scales of the group + lane * 4
  bool half_ok;        // lane group g < 2: valid in the last (half) step

  __device__ __forceinline__ void init(const FfnArgs& a, int e, int G, int lane) {
    const size_t grp = (size_t)e * (a.N >> 6) + G;
    const int l_last = lane & 31;
    cg = a.codes + grp * kGroupCodeBytes;
    sg = a.scales + grp * kGroupScaleBytes;
    half_ok = (lane >> 4) < 2;
    lane_c = lane * 16;
    lane_c_last = l_last * 16;
    lane_s = lane * 4;
    lane_s_last = l_last * 4;
  }
  int lane_c, lane_c_last, lane_s, lane_s_last;

  // four 16-row tiles of step s (s is a compile-time constant after
  // unrolling). NT marks the loads non-temporal: a stream read once (the
  // weight-streaming schedule) then keeps the caches for the activations.
  template <bool NT = false>
  __device__ __forceinline__ void load(int s, uint4 (&w)[4], uint32_t& sc) const {
    const bool last = s >= kFullSteps;
    const int tstride = last ? 512 : 1024;
    const uint8_t* c = cg + s * kStepCodeBytes + (last ? lane_c_last : lane_c);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(sg + s * 256 + (last ? lane_s_last : lane_s));
    if constexpr (NT) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c + mt * tstride));
        w[mt] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      sc = __builtin_nontemporal_load(sp);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) w[mt] = *reinterpret_cast<const uint4*>(c + mt * tstride);
      sc = *sp;
    }
    if (last) {
      const uint32_t keep = half_ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        w[mt].x &= keep; w[mt].y &= keep; w[mt].z &= keep; w[mt].w &= keep;
      }
    }
  }
};

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ------------------------------------------------------------------ skinny
constexpr int kSkDepth = 3;    // prefetch depth in K steps
constexpr int kSkTwoTilesMeanRows = 10;   // mean rows per expert above which a pass covers 32 tokens
constexpr int kSkWaves = 3;    // waves per workgroup: one expert, the activation tile shared
constexpr int kSkThreads = 64 * kSkWaves;

// One pass over the weights serves NT 16-token column tiles.
template <int NT>
struct SkShape {
  static constexpr int BT = 16 * NT;                  // tokens per pass
  static constexpr int XStage = BT * 256;             // activation tile of one K step (128 bf16 per row)
  static constexpr int Pieces = XStage / 16;          // its 16-byte pieces
  static constexpr int PPT = (Pieces + kSkThreads - 1) / kSkThreads;   // pieces per thread
};

struct SkStage {
  uint4 w[4];    // four 16-row tiles of the wave's group
  uint32_t sc;   // their four scale bytes
};

// Position of the n-th set bit (n < popcount) of a 64-bit mask.
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1ull));
    if (n >= c) {
      n -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}

// Expert e's slots straight from the routing ids: `below` = slots of lower
// experts (e's first position in the stable expert order), `count` = e's
// slots, and for lane r the slots of ranks rank0 + (r & 15) and rank0 + 16 +
// (r & 15) among e's slots in slot order (-1 past the end). One pass of
// coalesced loads, no dependent lookups; every lane of the wave must call it.
__device__ __forceinline__ void scan_expert_slots(const int32_t* ids, int n, int e, int rank0,
                                                  int& below, int& count, int& slot_r,
                                                  int& slot_r16) {
  const int lane = threadIdx.x & 63;
  const int tr = rank0 + (lane & 15);
  const int tr16 = tr + 16;
  below = 0;
  count = 0;
  slot_r = -1;
  slot_r16 = -1;
#pragma unroll 4
  for (int c = 0; c < n; c += 64) {
    const int i = c + lane;
    const int id = i < n ? ids[i] : 0x7FFFFFFF;
    const unsigned long long eq = __ballot(id == e);
    below += __popcll(__ballot(id < e));
    const int in = __popcll(eq);
    if (tr >= count && tr < count + in) slot_r = c + nth_set_bit(eq, tr - count);
    if (tr16 >= count && tr16 < count + in) slot_r16 = c + nth_set_bit(eq, tr16 - count);
    count += in;
  }
}

// One workgroup: kSkWaves waves, each streaming one 64-row group of expert
// e, over the expert's tokens 16 * NT at a time. The weight stream needs no
// routing data, so a wave only waits for the expert's row range and its first
// row lookups before the stream starts; a dependent load issued behind the
// chip-wide weight traffic would wait for the whole in-flight volume. The
// weights are read once and loaded non-temporally.
// The activations of a K step (16 * NT token rows x 256 bytes) are loaded
// once per workgroup, 16-byte pieces spread over the threads, written to a
// 3-slot LDS ring (pieces XOR-swizzled by row) and read back in the
// matrix-core layout by every wave: per-wave activation loads, though L2
// hits, cost the weight stream a sixth of its rate.
template <int EPI, int NT>
__global__ __launch_bounds__(kSkThreads) void ffn_skinny_kernel(FfnArgs a) {
  using Sh = SkShape<NT>;
  constexpr int MT = 4;
  constexpr int PPT = Sh::PPT;
  // the ring, then a spare area for the pieces a thread has beyond the tile
  // (it loads its first piece again and writes it there, so the code has no
  // branch; never read)
  __shared__ __attribute__((aligned(16))) uint8_t xs[kSkDepth * Sh::XStage + kSkThreads * 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.y;
  const int G0 = blockIdx.x * kSkWaves + wave;   // the wave's 64-row group
  const int r = lane & 15;   // weight row in a 16-row tile / token column
  const int g = lane >> 4;   // lane group: MX block 4s + g of step s
  // activation pieces of this thread: piece c = (token row c >> 4, 16-byte
  // piece c & 15 of the row's 256 bytes of the step)
  int pc[PPT], pw[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int c = tid + i * kSkThreads;
    const bool in = c < Sh::Pieces;
    pc[i] = in ? c : tid;
    pw[i] = in ? (c >> 4) * 256 + (((c & 15) ^ (c >> 4)) & 15) * 16 : -1;   // at most one spare per thread
  }

  int e_begin, e_end, slot_first = -1, slot_first16 = -1;
  if (a.ids) {
    int below, count;
    scan_expert_slots(a.ids, a.n_slots, e, 0, below, count, slot_first, slot_first16);
    e_begin = below;
    e_end = below + count;
  } else {
    e_begin = a.offsets[e];
    e_end = a.offsets[e + 1];
  }
  if (e_end <= e_begin) return;   // the whole workgroup: one expert
  // biases of this lane's output rows (consumed by the epilogue)
  const uint16_t* bias = a.bias + (size_t)e * a.N + G0 * 64 + 4 * g;
  uint2 braw[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) braw[mt] = *reinterpret_cast<const uint2*>(bias + 16 * mt);

  for (int rb = e_begin; rb < e_end; rb += Sh::BT) {
    const int re = min(e_end, rb + Sh::BT);
    // column r of tile nt holds the token of position rb + 16 nt + r; padded
    // columns take the pass's first slot and their outputs are dropped
    int slot[NT];
    bool tok_ok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tok_ok[nt] = rb + 16 * nt + r < re;
    if (a.ids) {
      int sr = slot_first, sr16 = slot_first16;
      if (rb != e_begin) {
        int b2, c2;
        scan_expert_slots(a.ids, a.n_slots, e, rb - e_begin, b2, c2, sr, sr16);
      }
      const int first = __shfl(sr, 0, 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) slot[nt] = tok_ok[nt] ? (nt == 0 ? sr : sr16) : first;
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) slot[nt] = a.sorted_rows[tok_ok[nt] ? rb + 16 * nt + r : rb];
    }
    // the routing weights are fetched with the row lookups, not behind the stream
    float wt[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wt[nt] = EPI == EPI_COMBINE ? a.topk_w[slot[nt]] : 0.f;
    // activation rows of this thread's pieces (token row c >> 4 of the pass)
    const uint16_t* xp[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int tr = pc[i] >> 4;
      int sl = __shfl(slot[0], tr & 15, 64);
      if (NT > 1) {
        const int sl16 = __shfl(slot[NT - 1], tr & 15, 64);
        sl = tr < 16 ? sl : sl16;
      }
      const int arow = a.gather ? sl / a.k : (rb + tr < re ? rb + tr : rb);
      xp[i] = a.act + (size_t)arow * kH + (pc[i] & 15) * 8;
    }
    // slot >= 0 always; the compiler cannot know it, so the weight addresses
    // depend on the row lookup and the stream starts after it returns
    GroupStream ws;
    ws.init(a, e + (slot[0] < 0 ? 1 : 0), G0, lane);

    // s is a compile-time constant after unrolling; the K tail (blocks >= 90)
    // re-reads the row's last 8 values, whose weights are zero there
    auto issue = [&](SkStage& st, u32x4 (&xr)[PPT], int s) __attribute__((always_inline)) {
      ws.template load<true>(s, st.w, st.sc);
      const int k0 = s * 128;
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        xr[i] = *reinterpret_cast<const u32x4*>(xp[i] + min(k0, kH - 8 - (pc[i] & 15) * 8));
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const SkStage& st, const uint8_t* xsb) __attribute__((always_inline)) {
      float sf[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sf[mt] = e8m0_to_f32((st.sc >> (8 * mt)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8 xb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          xb[nt] = *reinterpret_cast<const bf16x8*>(xsb + (16 * nt + r) * 256 + (((4 * g + i) ^ r) & 15) * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 wb = fp4x8_to_bf16x8(dword_of(st.w[mt], i), sf[mt]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb, xb[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    };

    // fully unrolled K loop with a kSkDepth-step register prefetch ring; per
    // step: write this thread's activation pieces into the step's LDS slot,
    // wait for the LDS writes, barrier, then every wave computes from LDS and
    // refills the ring slot. A slot is rewritten kSkDepth steps after it was
    // read, and its readers have passed the barrier in between.
    SkStage st[kSkDepth];
    u32x4 xr[kSkDepth][PPT];
#pragma unroll
    for (int q = 0; q < kSkDepth; ++q) issue(st[q], xr[q], q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int q = s % kSkDepth;
      const int xo = q * Sh::XStage;
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        *reinterpret_cast<u32x4*>(xs + (pw[i] >= 0 ? xo + pw[i] : kSkDepth * Sh::XStage + tid * 16)) = xr[q][i];
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this thread's LDS writes are done
      __builtin_amdgcn_s_barrier();
      compute(st[q], xs + xo);
      if (s + kSkDepth < kSteps) issue(st[q], xr[q], s + kSkDepth);
      __builtin_amdgcn_sched_barrier(0);
    }

    // 16x16 results: lane holds token column r of tile nt and weight rows
    // 4g + j of each weight tile mt.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!tok_ok[nt]) continue;
      const int p = rb + 16 * nt + r;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int R0 = G0 * 64 + 16 * mt + 4 * g;
        const float v0 = acc[mt][nt][0] + bf16_bits_to_f32(braw[mt].x & 0xFFFFu);
        const float v1 = acc[mt][nt][1] + bf16_bits_to_f32(braw[mt].x >> 16);
        const float v2 = acc[mt][nt][2] + bf16_bits_to_f32(braw[mt].y & 0xFFFFu);
        const float v3 = acc[mt][nt][3] + bf16_bits_to_f32(braw[mt].y >> 16);
        if constexpr (EPI == EPI_SWIGLU) {
          *reinterpret_cast<uint32_t*>(a.h_out + (size_t)p * kI + R0 / 2) =
              f32x2_to_bf16x2_bits(swiglu_pair(v0, v1), swiglu_pair(v2, v3));
        } else if constexpr (EPI == EPI_COMBINE) {
          float* o = a.out + (size_t)(slot[nt] / a.k) * kH + R0;
          unsafeAtomicAdd(o + 0, wt[nt] * v0);
          unsafeAtomicAdd(o + 1, wt[nt] * v1);
          unsafeAtomicAdd(o + 2, wt[nt] * v2);
          unsafeAtomicAdd(o + 3, wt[nt] * v3);
        } else {
          *reinterpret_cast<float4*>(a.y_out + (size_t)slot[nt] * kH + R0) = make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
}

// Grid (workgroups of kSkWaves groups, expert): 30 workgroups per expert for
// the gate/up GEMM (90 groups), 15 for the down GEMM (45). Two token tiles
// per pass once most experts have more than 16 rows.
template <int EPI>
static hipError_t launch_skinny(const FfnArgs& a, int n_rows, hipStream_t s) {
  const int groups = a.N >> 6;
  if (groups % kSkWaves != 0) return hipErrorInvalidValue;   // every wave owns one group
  const dim3 grid(groups / kSkWaves, a.E);
  if ((long long)n_rows > (long long)kSkTwoTilesMeanRows * a.E)
    hipLaunchKernelGGL((ffn_skinny_kernel<EPI, 2>), grid, dim3(kSkThreads), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_skinny_kernel<EPI, 1>), grid, dim3(kSkThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ wide

constexpr int kTileChunk = 8;   // token tiles that share a pass over the weight columns
constexpr int kXcds = 8;

// Work order of the tiled kernel. Workgroups are dealt to the 8 XCDs
// round-robin in launch order, and each XCD has its own L2, so the linear
// block id is first turned into an order in which every XCD runs one
// contiguous range of the work. Within that order, kTileChunk consecutive
// token tiles go with each weight column block in turn (tiles fastest): the
// tiles of a chunk read the same weights close together in time on one L2.
template <int CH = kTileChunk>
__device__ __forceinline__ void wide_work_item(int gx, int gy, int& wx, int& ty) {
  const int nb = gx * gy;
  const int b = blockIdx.x;
  const int q = nb / kXcds, r = nb % kXcds, xcd = b % kXcds, idx = b / kXcds;
  const int L = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
  const int per = gx * CH;
  const int chunk = L / per, rem = L - chunk * per;
  const int cy = min(CH, gy - chunk * CH);
  wx = rem / cy;
  ty = chunk * CH + (rem - wx * cy);
}
constexpr int kWdNT = 4;           // 16-token column tiles per wave
constexpr int kWdBT = 16 * kWdNT;   // tokens per tile
constexpr int kWdGroups = 4;   // 64-row groups per block, one per wave
constexpr int kXRow = 256;     // bytes per token row of an LDS activation stage (128 K)
constexpr int kXStage = kWdBT * kXRow;   // 16 KiB
constexpr int kXLoads = kWdBT / 16;   // 1 KiB LDS DMA instructions per wave per stage

// One lane's FP6 activation operand from an LDS stage of MX6 records (record
// layout in moe_device.h; 16-byte pieces swizzled by token & 15 like the bf16
// rows): the 24 code bytes of MX block g of one piece for token 16 nt + r.
struct X6Half {
  uint4 lo;
  uint2 hi;
  __device__ __forceinline__ void read(const uint8_t* xsb, int nt, int piece, int r, int g) {
    const uint8_t* xr = xsb + (16 * nt + r) * kXRow;
    lo = *reinterpret_cast<const uint4*>(xr + ((4 * piece + g) ^ r) * 16);
    hi = *reinterpret_cast<const uint2*>(xr + ((8 + 2 * piece + (g >> 1)) ^ r) * 16 + (g & 1) * 8);
  }
  // both pieces' scale bytes of block g (piece 1 in bits 0..7, piece 2 in 8..15)
  __device__ __forceinline__ static uint32_t read_scales(const uint8_t* xsb, int nt, int r, int g) {
    return *reinterpret_cast<const uint16_t*>(xsb + (16 * nt + r) * kXRow + (12 ^ r) * 16 + 2 * g);
  }
  __device__ __forceinline__ i32x8 operand() const {
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, 0, 0};
  }
};

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The block-scaled tiled kernel (activations as two-piece MX FP6 records).
// Block = 4 waves = four 64-row groups x 64 tokens. The records go straight
// from global memory into a 2-stage LDS ring (global_load_lds, 16 bytes per
// lane, no staging registers); within a 256-byte token row the 16-byte
// pieces are XOR-swizzled by (token & 15). Weights stream to registers
// (2-step ring). Per K step: wait for this step's loads, barrier, issue the
// next activation stage, compute, refill the weights.
template <int EPI, bool W_AS_B>
__device__ __forceinline__ void wide6_body(const FfnArgs& a) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs[2 * kXStage];
  __shared__ int slot_of[kWdBT];
  __shared__ uint16_t bias_s[kWdGroups * 64];
  static_assert(kWdGroups * 64 == 256, "one bias per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int e, rb, re;
  int wx, ty;
  const int gx = ((a.N >> 6) + kWdGroups - 1) / kWdGroups;
  wide_work_item(gx, gridDim.x / gx, wx, ty);
  if (!find_tile(a.offsets, a.E, kWdBT, ty, e, rb, re)) return;
  const int G = wx * kWdGroups + wave;
  const bool w_ok = G < (a.N >> 6);
  if (tid < kWdBT) {
    const int p = rb + tid;
    slot_of[tid] = p < re ? a.sorted_rows[p] : -1;
  }
  // the block's 256 output-row biases go to LDS now; loaded in the epilogue
  // they would wait behind the tail of the weight stream
  {
    const int row = wx * kWdGroups * 64 + tid;
    bias_s[tid] = row < a.N ? a.bias[(size_t)e * a.N + row] : 0;
  }

  // Activation loads: wave w, instruction j fills LDS rows 4*(4w+j) .. +3
  // (1 KiB); lane i takes token t = 4*(4w+j) + (i >> 4) and LDS piece
  // q = i & 15, which holds record piece q ^ (t & 15). Padded tokens read the
  // tile's first row (outputs dropped). A record holds a whole K step, so
  // there is no tail handling.
  const int q_lds = lane & 15;
  const uint8_t* xbase = a.act6;
  size_t xoff[kXLoads];
#pragma unroll
  for (int j = 0; j < kXLoads; ++j) {
    const int t = 4 * (kXLoads * wave + j) + (lane >> 4);
    const int p = rb + t < re ? rb + t : rb;
    const int row = a.gather ? a.sorted_rows[p] / a.k : p;
    xoff[j] = (size_t)row * kRowRecBytes + (q_lds ^ (t & 15)) * 16;
  }
  auto load_x = [&](uint8_t* dst, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) {
      const uint8_t* src = xbase + xoff[j] + s * kRecBytes;
      __builtin_amdgcn_global_load_lds(
          (const void*)src,
          (__attribute__((address_space(3))) void*)(dst + (kXLoads * wave + j) * 1024), 16, 0, 0);
    }
  };

  GroupStream wsrc;
  wsrc.init(a, e, w_ok ? G : 0, lane);
  uint4 wq[2][4];
  uint32_t wsc[2];
  const int r = lane & 15;
  const int g = lane >> 4;

  f32x4 acc[4][kWdNT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kWdNT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* xsb, int buf) __attribute__((always_inline)) {
    {
      // Block-scaled FP4 x FP6 (16x16x128): the packed weight lane holds one
      // whole MX block, which is the instruction's operand as it stands; its
      // scale is byte mt of the step's scale dword (the instruction reads
      // byte 0 of the scale operand). Two MFMAs per tile pair, one per piece.
      // One (token tile, piece) operand is read from LDS while the previous
      // one computes; scheduling barriers and register-tied empty asm keep
      // that order (otherwise every tile's operands are loaded up front and
      // the registers of three waves per SIMD overflow).
      int wsa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) wsa[mt] = (int)(wsc[buf] >> (8 * mt));
      X6Half hb[2];
      uint32_t scb[2];
      hb[0].read(xsb, 0, 0, r, g);
      scb[0] = X6Half::read_scales(xsb, 0, r, g);
#pragma unroll
      for (int q = 0; q < 2 * kWdNT; ++q) {
        const int nt = q >> 1, piece = q & 1;
        if (q + 1 < 2 * kWdNT) {
          hb[(q + 1) & 1].read(xsb, (q + 1) >> 1, (q + 1) & 1, r, g);
          if (((q + 1) & 1) == 0) scb[((q + 1) >> 1) & 1] = X6Half::read_scales(xsb, (q + 1) >> 1, r, g);
        }
        asm volatile("" ::: "memory");   // no LDS read moves across operands
        __builtin_amdgcn_sched_barrier(0);
        const i32x8 xp = hb[q & 1].operand();
        const int xsc = (int)(scb[nt & 1] >> (8 * piece));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 wv = wq[buf][mt];
          const i32x8 wa = {(int)wv.x, (int)wv.y, (int)wv.z, (int)wv.w, 0, 0, 0, 0};
          if constexpr (W_AS_B)
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                xp, wa, acc[mt][nt], kFmtE2M3, kFmtFp4, 0, xsc, 0, wsa[mt]);
          else
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wa, xp, acc[mt][nt], kFmtFp4, kFmtE2M3, 0, wsa[mt], 0, xsc);
        }
        // pins this operand's matrix-core work before the next LDS reads
        asm volatile("" : "+v"(acc[0][nt]), "+v"(acc[1][nt]), "+v"(acc[2][nt]), "+v"(acc[3][nt]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Load issue order: W(0), W(1), X(0); then per step s: [X(s+1)] ... [W(s+2)].
  // Before computing step s the loads still allowed in flight are those
  // issued after X(s) and W(s): W(s+1) (5 loads per wave, or none when the
  // wave holds no rows).
  if (w_ok) {
    wsrc.load(0, wq[0], wsc[0]);
    wsrc.load(1, wq[1], wsc[1]);
  }
  load_x(xs, 0);
  for (int s0 = 0; s0 < kSteps; s0 += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int s = s0 + q;
      if (s < kSteps) {
        if (s == 0 || !w_ok || s + 1 >= kSteps) wait_vmcnt<0>();
        else wait_vmcnt<5>();
        __builtin_amdgcn_s_barrier();
        if (s + 1 < kSteps) load_x(xs + (q ^ 1) * kXStage, s + 1);
        if (w_ok) {
          compute(xs + q * kXStage, q);
          if (s + 2 < kSteps) wsrc.load(s + 2, wq[q], wsc[q]);
        }
      }
    }
  }
  if constexpr (!W_AS_B && EPI == EPI_SWIGLU) {
    if (a.h6_out) {
      // h as two-piece MX FP6 records: this wave's 32 h features of a token
      // (group G of 64 interleaved gate/up rows) are MX block G of that
      // token's h row, i.e. block G % 4 of the record of K step G / 4. The
      // wave's bf16 h values go token-major through its own 4 KiB of LDS
      // stage 1 (idle since the last step's barrier; LDS operations of a wave
      // complete in order), then lane t encodes token t's block, the same
      // rounding to bf16 first as the separate encoder. The waves past the
      // last group (G = 90, 91) write the zero blocks that pad the last step.
      const int t = lane;
      const int p = rb + t;
      const int st = G >> 2, gb = G & 3;
      uint8_t* rec = a.h6_out + (size_t)p * kRowRecBytes + st * kRecBytes;
      uint32_t w1[6], w2[6], s1 = 127u, s2 = 127u;
#pragma unroll
      for (int i = 0; i < 6; ++i) w1[i] = w2[i] = 0u;
      if (w_ok) {
        uint8_t* hs = xs + kXStage + wave * (kWdBT * 64);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          float b[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) b[j] = bf16_bits_to_f32(bias_s[wave * 64 + 16 * mt + 4 * g + j]);
#pragma unroll
          for (int nt = 0; nt < kWdNT; ++nt) {
            const f32x4& c = acc[mt][nt];
            *reinterpret_cast<uint32_t*>(hs + (16 * nt + r) * 64 + (8 * mt + 2 * g) * 2) =
                f32x2_to_bf16x2_bits(swiglu_pair(c[0] + b[0], c[1] + b[1]), swiglu_pair(c[2] + b[2], c[3] + b[3]));
          }
        }
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 d = *reinterpret_cast<const uint4*>(hs + t * 64 + q * 16);
          const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = bf16_bits_to_f32(dw[i] & 0xFFFFu);
            v[8 * q + 2 * i + 1] = bf16_bits_to_f32(dw[i] >> 16);
          }
        }
        mx6x2_encode(v, w1, s1, w2, s2);
      }
      if (p < re) {
        *reinterpret_cast<uint4*>(rec + gb * 16) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        *reinterpret_cast<uint4*>(rec + (4 + gb) * 16) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        *reinterpret_cast<uint2*>(rec + (8 + (gb >> 1)) * 16 + (gb & 1) * 8) = make_uint2(w1[4], w1[5]);
        *reinterpret_cast<uint2*>(rec + (10 + (gb >> 1)) * 16 + (gb & 1) * 8) = make_uint2(w2[4], w2[5]);
        *reinterpret_cast<uint16_t*>(rec + 12 * 16 + 2 * gb) = (uint16_t)(s1 | (s2 << 8));
      }
      return;
    }
  }
  if (!w_ok) return;

  if constexpr (!W_AS_B) {
    // D[weight row][token]: lane holds token column r, rows 4g + j of tile mt
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int R0 = G * 64 + 16 * mt + 4 * g;
      float b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = bf16_bits_to_f32(bias_s[wave * 64 + 16 * mt + 4 * g + j]);
#pragma unroll
      for (int nt = 0; nt < kWdNT; ++nt) {
        const int p = rb + 16 * nt + r;
        if (p >= re) continue;
        const f32x4& c = acc[mt][nt];
        *reinterpret_cast<uint32_t*>(a.h_out + (size_t)p * kI + R0 / 2) =
            f32x2_to_bf16x2_bits(swiglu_pair(c[0] + b[0], c[1] + b[1]), swiglu_pair(c[2] + b[2], c[3] + b[3]));
      }
    }
  } else {
    // D[token][weight row]: lane holds weight row (output feature) r of tile
    // mt, tokens 4g + j of column tile nt
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int f = G * 64 + 16 * mt + r;
      const float bf = bf16_bits_to_f32(bias_s[wave * 64 + 16 * mt + r]);
#pragma unroll
      for (int nt = 0; nt < kWdNT; ++nt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int slot = slot_of[16 * nt + 4 * g + j];
          if (slot < 0) continue;
          const float v = acc[mt][nt][j] + bf;
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

// The FP6 fragments of four token tiles would otherwise all be loaded ahead
// of the matrix-core work, leaving room for two waves per SIMD; three keep
// the load latency covered.
template <int EPI, bool W_AS_B>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void ffn_wide6_kernel(FfnArgs a) {
  wide6_body<EPI, W_AS_B>(a);
}

// ------------------------------------------------------------------ tiled, bf16
// The many-rows-per-expert schedule of the bf16 path. Block = 8 waves = eight
// 64-row weight groups (512 rows) x 128 tokens of one expert, two waves per
// SIMD; each wave owns a 64 x 128 output tile of 32x32x16 bf16 MFMAs (2
// weight tiles x 4 token tiles, 128 accumulator registers), so every
// dequantised weight fragment feeds four MFMAs and every activation fragment
// read from LDS feeds two, and each activation stage serves 512 weight rows.
//
// Weights: straight to registers from the packed order. For a 32-row tile mt
// and K half h of the instruction, lane 32h + c loads row 32mt + c = 16-row
// tile m = 2mt + (c >> 4), packed lane 16g + (c & 15), MX block g = 2jb + h of
// the step (jb = 0, 1): four 256-byte runs per load. Dword i of that load
// (codes 8i .. 8i + 7 of the block) is the lane's 8-value K slice of MFMA
// (jb, i); the activation operand supplies the same K for its token.
// Activations: gathered rows go global -> LDS by DMA into a 4-stage ring of
// 128 rows x 256 bytes (128 K); the 16-byte pieces of a row are XOR-swizzled
// by (row & 15), so the 32-row operand reads (row c, piece 4(2jb + h) + i)
// hit 64 distinct banks in every LDS cycle (measured conflict-free).
// A tile with at most 64 tokens (an expert's last) runs only its first two
// token tiles.
// The last column block of a projection holds fewer than 8 groups (N = 5,760:
// 2 of 8; N = 2,880: 5 of 8). With one group per wave its busiest SIMD
// would carry a full block's work, so there the token tiles are split across
// waves (tl_wave_role): each wave then takes one group and one or more
// consecutive 32-token tiles, which evens out the SIMDs (waves w and w + 4
// share one).
constexpr int kTlBT = 128;                       // tokens per tile
constexpr int kTlWaves = 8;                      // waves per block, one 64-row group each
constexpr int kTlThreads = 64 * kTlWaves;
constexpr int kTlRows = 64 * kTlWaves;           // weight rows per block (512)
constexpr int kTlStage = kTlBT * kXRow;          // 32 KiB per activation stage
constexpr int kTlStages = 4;                     // activation ring depth (3 steps ahead)
constexpr int kTlXLoads = kTlStage / (kTlWaves * 1024);  // 1 KiB DMA instructions per wave per stage (4)
constexpr int kTlChunk = 4;                      // token tiles per pass over a weight column block

// Tiles of `bt` rows over all experts' row ranges (one full wave; every lane
// gets the same answer).
__device__ __forceinline__ int count_tiles(const int32_t* __restrict__ offsets, int E, int bt) {
  const int lane = threadIdx.x & 63;
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    if (e < E) local += (offsets[e + 1] - offsets[e] + bt - 1) / bt;
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) local += __shfl_xor(local, d, 64);
  return local;
}

// Work item (column block wx, token tile ty) of this block, from `total`
// real tiles: the gx * total items are split into 8 contiguous ranges, one
// per XCD (blocks are dealt to the XCDs round-robin in launch order); within
// a range, CHUNK consecutive tiles go with each column block in turn. False
// for a spare block.
template <int CHUNK>
__device__ __forceinline__ bool tile_work_item(int gx, int total, int& wx, int& ty) {
  const int nw = gx * total;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  const int q = nw / kXcds, r = nw % kXcds;
  if (idx >= q + (xcd < r ? 1 : 0)) return false;
  const int L = xcd * q + min(xcd, r) + idx;
  const int per = gx * CHUNK;
  const int chunk = L / per, rem = L - chunk * per;
  const int cy = min(CHUNK, total - chunk * CHUNK);
  wx = rem / cy;
  ty = chunk * CHUNK + (rem - wx * cy);
  return true;
}

// 16 bytes per lane from global memory straight into LDS at `lds_dst` +
// 16 * lane (lds_dst wave-uniform). Written as inline asm: the compiler then
// does not treat the DMA as an LDS write, so it issues no wait for it before
// the LDS reads of the other stages (it would otherwise wait for every
// outstanding load there); completion is tracked by the caller's vmcnt waits.
// The instruction has no register result.
__device__ __forceinline__ void lds_dma16(const void* src, const uint8_t* lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
}

struct TlStep {
  uint4 w[2][2];    // [jb][mt]
  uint32_t sc[2];   // [jb]: scale bytes of 16-row tiles m = 0..3 for this lane's (g, r)
};

struct TlWeights {
  const uint8_t* cg;
  const uint8_t* sg;
  int lane_c, lane_c_last, lane_s;   // byte offsets of this lane inside a step
  __device__ __forceinline__ void init(const FfnArgs& a, int e, int G, int lane) {
    const size_t grp = (size_t)e * (a.N >> 6) + G;
    cg = a.codes + grp * kGroupCodeBytes;
    sg = a.scales + grp * kGroupScaleBytes;
    const int h = lane >> 5, c = lane & 31;
    const int mhi = c >> 4, rr = c & 15;
    lane_c = mhi * 1024 + (16 * h + rr) * 16;
    lane_c_last = mhi * 512 + (16 * h + rr) * 16;
    lane_s = (16 * h + rr) * 4;
  }
  // half jb of step s: codes of both 32-row tiles and the scale dword (the
  // half last step has only jb = 0); 3 loads
  __device__ __forceinline__ void load_half(int s, int jb, TlStep& st) const {
    // the step's offsets are made opaque so that each step computes its own
    // addresses (hoisted, 23 steps' worth of 64-bit addresses would not fit
    // beside the accumulators)
    int co = s * kStepCodeBytes, so = s * 256;
    asm volatile("" : "+s"(co), "+s"(so));
    if (s < kFullSteps) {
      const uint8_t* c = cg + co + lane_c;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        st.w[jb][mt] = *reinterpret_cast<const uint4*>(c + mt * 2048 + jb * 512);
      st.sc[jb] = *reinterpret_cast<const uint32_t*>(sg + so + lane_s + jb * 128);
    } else if (jb == 0) {
      const uint8_t* c = cg + co + lane_c_last;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) st.w[0][mt] = *reinterpret_cast<const uint4*>(c + mt * 1024);
      st.sc[0] = *reinterpret_cast<const uint32_t*>(sg + so + lane_s);
    }
  }
};

// The vmcnt each K step s waits for before its barrier (between substeps 3
// and 4): the next step's stage X(s+1) and this step's second weight half
// W(s) half 1 must have landed; everything issued after W(s) half 1 may stay
// in flight. Issue order: prologue W(0), W(1), X(0), X(1), X(2); step s,
// after its barrier: W(s+2) half 0, X(s+3) (substeps 4..7), W(s+2) half 1
// (after substep 7). X(s+1) goes before W(s) half 1 (both in step s - 2),
// except that X(1), X(2) are prologue loads.
__host__ __device__ constexpr int tl_issued_after_barrier(int s) {
  return (s + 2 < kSteps ? 3 : 0) + (s + 3 < kSteps ? kTlXLoads : 0) + (s + 2 < kSteps - 1 ? 3 : 0);
}
__host__ __device__ constexpr int tl_wait_mid(int s) {
  return s == 0 ? kTlXLoads                        // X(2)
       : s == 1 ? tl_issued_after_barrier(0)       // after X(2): step 0's loads
       : tl_issued_after_barrier(s - 1);
}

// tile_run: NTL = 32-token tiles of the block's tile that are loaded (4, or
// 2 for a tile of at most 64 tokens); this wave computes NTA of them from
// tile nt0 on, for weight group G (local group gloc of the column block).
template <int EPI, int NTL, int NTA, bool W_OK>
__device__ __forceinline__ void tile_run(const FfnArgs& a, uint8_t* xs, int* slot_of,
                                         int* xrow_of, uint16_t* bias_s, int e, int G,
                                         int gloc, int nt0, int rb, int re) {
  constexpr bool w_ok = W_OK;
  // the down projection reads rows rb + t of h (sorted order): its copies need
  // no lookup, and its slot and bias rows are loaded behind them
  constexpr bool kDirect = EPI != EPI_SWIGLU;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  const int rr = c & 15, mhi = c >> 4;

  // Activation DMA: wave w, instruction j fills token rows 4(4w + j) .. + 3
  // of a stage; lane i takes row t = 4(4w + j) + (i >> 4) and LDS piece
  // q = i & 15, which holds K piece q ^ (t & 15). Padded rows read the tile's
  // first row; the K tail (last step, pieces past the row) re-reads the row's
  // last piece. The instructions whose rows lie in token tiles a half tile
  // skips are not issued.
  const int q_lds = lane & 15;
  constexpr int kLoadRows = NTL * 32;
  const uint16_t* xsrc[kTlXLoads];   // this lane's row (and K piece) per instruction
#pragma unroll
  for (int j = 0; j < kTlXLoads; ++j) {
    const int t = 4 * (kTlXLoads * wave + j) + (lane >> 4);
    const int kp = (q_lds ^ ((4 * j + (lane >> 4)) & 15)) * 8;   // t & 15 = (4j + (lane >> 4)) & 15
    const int xrow = kDirect ? rb + (rb + t < re ? t : 0) : xrow_of[t];
    xsrc[j] = a.act + (size_t)xrow * kH + kp;
  }
  auto load_x_one = [&](uint8_t* dst, int s, int j) __attribute__((always_inline)) {
    if (4 * (kTlXLoads * wave + j) >= kLoadRows) return;   // wave-uniform
    int ko = s * 128;
    asm volatile("" : "+s"(ko));
    const uint16_t* src = xsrc[j] + ko;
    if (s == kSteps - 1) {
      // pieces past the row's end: its last piece instead
      const uint16_t* row_end = xsrc[j] - ((q_lds ^ ((4 * j + (lane >> 4)) & 15)) * 8) + kH - 8;
      src = src > row_end ? row_end : src;
    }
    lds_dma16(src, dst + (kTlXLoads * wave + j) * 1024);
  };
  auto stage = [&](int s) __attribute__((always_inline)) {
    int so = (s & (kTlStages - 1)) * kTlStage;
    asm volatile("" : "+s"(so));
    return xs + so;
  };

  TlWeights wsrc;
  wsrc.init(a, e, w_ok ? G : 0, lane);
  TlStep wq[2];
  f32x16 acc[2][NTA];   // set from the biases once the first loads are issued

  // One K step: 8 substeps (jb, i) of 2 x NTA MFMAs each. The activation DMA
  // of step s + 3 and the weights of step s + 2 (into this step's register
  // slot, half by half once each half has been consumed) are spread over the
  // substeps, so the wave keeps the matrix cores fed while its memory
  // instructions wait to issue.
  // this wave's activation rows: token tiles nt0 .. nt0 + NTA - 1
  const int xrow0 = (32 * nt0 + c) * kXRow;
  auto read_x = [&](const uint8_t* xsb, int q, bf16x8 (&xf)[NTA]) __attribute__((always_inline)) {
    const int jb = q >> 2, i = q & 3;
#pragma unroll
    for (int nt = 0; nt < NTA; ++nt)
      xf[nt] = *reinterpret_cast<const bf16x8*>(xsb + xrow0 + 32 * nt * kXRow +
                                                (((8 * jb + 4 * h + i) ^ rr) * 16));
  };
  auto wait_for = [&](int n) __attribute__((always_inline)) {
    switch (n) {
      case 0: wait_vmcnt<0>(); break;
      case 3: wait_vmcnt<3>(); break;
      case 4: wait_vmcnt<4>(); break;
      case 8: wait_vmcnt<8>(); break;
      case 10: wait_vmcnt<10>(); break;
      default: wait_vmcnt<0>(); break;
    }
  };

  // One K step: 8 substeps q = (jb, i) of 2 x NTA MFMAs each (the half last
  // step: 4). The block synchronises once per step, between substeps 3 and 4:
  // by then every wave has waited for its own DMA of the next step's stage
  // (so that stage is complete) and has finished reading the stage of the
  // previous step (so the DMA of step s + 3 may refill it: it is issued in
  // substeps 4..7). The next step's first activation fragments are read at
  // the end of the step, so no step starts with an LDS wait. The weights of
  // step s + 2 refill this step's register slot half by half, as each half
  // is consumed.
  bf16x8 xf[NTA];
  auto kstep = [&](int s, TlStep& st) __attribute__((always_inline)) {
    const uint8_t* xsb = stage(s);
    const int nq = s == kSteps - 1 ? 4 : 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q >= nq) break;
      const int jb = q >> 2, i = q & 3;
      bf16x8 wf[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float sf = e8m0_to_f32((st.sc[jb] >> (8 * (2 * mt + mhi))) & 0xFFu);
        wf[mt] = fp4x8_to_bf16x8(dword_of(st.w[jb][mt], i), sf);
      }
      // fragment nt of the next substep (or of the next step's first, once
      // the block has passed this step's barrier) is read into xf[nt] as
      // soon as this substep's two MFMAs on it are issued
      const bool next_here = q + 1 < nq;
      const bool next_step = q == nq - 1 && s + 1 < kSteps;
#pragma unroll
      for (int nt = 0; nt < NTA; ++nt) {
        if (w_ok) {
          acc[0][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[0], xf[nt], acc[0][nt], 0, 0, 0);
          acc[1][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[1], xf[nt], acc[1][nt], 0, 0, 0);
        }
        if (next_here || next_step) {
          const uint8_t* src = next_here ? xsb : stage(s + 1);
          const int qn = next_here ? q + 1 : 0;
          xf[nt] = *reinterpret_cast<const bf16x8*>(src + xrow0 + 32 * nt * kXRow +
                                                    (((8 * (qn >> 2) + 4 * h + (qn & 3)) ^ rr) * 16));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (q == 3) {
        if (s + 1 < kSteps) {
          wait_for(tl_wait_mid(s));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 2 < kSteps) wsrc.load_half(s + 2, 0, st);
      }
      if (q >= 4 && s + 3 < kSteps) load_x_one(stage(s + 3), s + 3, q - 4);
      if (q == 7 && s + 2 < kSteps) wsrc.load_half(s + 2, 1, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  wsrc.load_half(0, 0, wq[0]);
  wsrc.load_half(0, 1, wq[0]);
  wsrc.load_half(1, 0, wq[1]);
  wsrc.load_half(1, 1, wq[1]);
#pragma unroll
  for (int s = 0; s < kTlStages - 1; ++s)
#pragma unroll
    for (int j = 0; j < kTlXLoads; ++j) load_x_one(stage(s), s, j);
  // D[weight row][token]: lane holds token column c of tile nt and weight
  // rows 32mt + 8q + 4h + j (j = 0..3) of the wave's group. The accumulators
  // start from the rows' biases, so the epilogue has no bias to add.
  auto init_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = w_ok ? bf16_bits_to_f32(bias_s[gloc * 64 + 32 * mt + 8 * q + 4 * h + j]) : 0.f;
#pragma unroll
          for (int nt = 0; nt < NTA; ++nt) acc[mt][nt][4 * q + j] = b;
        }
  };
  if constexpr (kDirect) {
    // the tile's slots (for the y rows) and biases, behind its first copies;
    // every thread's LDS stores are done before the barrier below
    const int tid0 = threadIdx.x;
    if (tid0 < kTlBT) slot_of[tid0] = rb + tid0 < re ? a.sorted_rows[rb + tid0] : -1;
    const int row = (G / kTlWaves) * kTlRows + tid0;   // the column block's row tid0
    bias_s[tid0] = row < a.N ? a.bias[(size_t)e * a.N + row] : 0;
    // the barrier below does not wait for LDS stores: this thread's are done
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  } else {
    init_acc();   // while the first loads are in flight
  }
  wait_for(2 * kTlXLoads);   // X(0) and both weight steps
  __builtin_amdgcn_s_barrier();
  if constexpr (kDirect) init_acc();
  read_x(stage(0), 0, xf);
  // every step is its own straight-line code (compile-time step index): the
  // waits, ring slots and stage offsets are constants, and the compiler's own
  // load accounting stays exact
  static_for<kSteps>([&](auto S) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    kstep(s, wq[s & 1]);
  });
  static_assert(tl_wait_mid(0) == 4 && tl_wait_mid(1) == 10 && tl_wait_mid(10) == 10 &&
                tl_wait_mid(20) == 10 && tl_wait_mid(21) == 3, "load accounting");

  if (!w_ok) return;

  if constexpr (EPI == EPI_STORE_Y) {
    // y goes out through 8 KiB of LDS of the wave's own, one 32-token tile
    // at a time, so that each token's 64 outputs (256 bytes) leave as one
    // segment instead of 32-byte pieces of 32 rows per store instruction
    // (measured 2-3% faster). The slices lie in the ring stages of steps 19
    // and 20, which no wave reads or fills once all have passed the barrier
    // of step 21; no barrier is needed: only this wave touches its slice,
    // and a wave's LDS accesses complete in order. D[weight row][token]:
    // lane holds token column c of tile nt and weight rows 32mt + 8q + 4h +
    // j of the wave's group; unit u (16 bytes) of row r sits at u ^ (r & 15).
    static_assert(((kSteps - 3) & (kTlStages - 1)) == 0 && ((kSteps - 4) & (kTlStages - 1)) == 3,
                  "the stages of steps 19 and 20");
    uint8_t* own = xs + __builtin_amdgcn_readfirstlane((wave < 4 ? 0 : 3 * kTlStage) + (wave & 3) * 8192);
    const int uu = lane & 15;
#pragma unroll
    for (int nt = 0; nt < NTA; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& A = acc[mt][nt];
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = A[4 * q + j];
          const int u = 8 * mt + 2 * q + h;
          *reinterpret_cast<float4*>(own + c * 256 + 16 * (u ^ (c & 15))) = make_float4(v[0], v[1], v[2], v[3]);
        }
      asm volatile("" ::: "memory");
      // 4 rows of 256 bytes per instruction, 16 bytes per lane
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = 4 * it + (lane >> 4);
        const int t = 32 * (nt0 + nt) + r;
        const float4 v = *reinterpret_cast<const float4*>(own + r * 256 + 16 * (uu ^ (r & 15)));
        if (rb + t < re)
          *reinterpret_cast<float4*>(a.y_out + (size_t)slot_of[t] * kH + G * 64 + 4 * uu) = v;
      }
      asm volatile("" ::: "memory");
    }
    return;
  }

#pragma unroll
  for (int nt = 0; nt < NTA; ++nt) {
    const int t = 32 * (nt0 + nt) + c;
    if (rb + t >= re) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = 32 * mt + 8 * q + 4 * h;   // row within the group
        const f32x16& A = acc[mt][nt];
        const float v0 = A[4 * q + 0], v1 = A[4 * q + 1], v2 = A[4 * q + 2], v3 = A[4 * q + 3];
        const int R0 = G * 64 + lr;
        if constexpr (EPI == EPI_SWIGLU) {
          *reinterpret_cast<uint32_t*>(a.h_out + (size_t)(rb + t) * kI + R0 / 2) =
              f32x2_to_bf16x2_bits(swiglu_pair(v0, v1), swiglu_pair(v2, v3));
        } else if constexpr (EPI == EPI_COMBINE) {
          const int slot = slot_of[t];
          const float wt = a.topk_w[slot];
          float* o = a.out + (size_t)(slot / a.k) * kH + R0;
          unsafeAtomicAdd(o + 0, wt * v0);
          unsafeAtomicAdd(o + 1, wt * v1);
          unsafeAtomicAdd(o + 2, wt * v2);
          unsafeAtomicAdd(o + 3, wt * v3);
        } else {
          *reinterpret_cast<float4*>(a.y_out + (size_t)slot_of[t] * kH + R0) = make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
}

// What wave `wave` computes in a column block of gl valid 64-row groups
// (1 .. 8) over a tile of ntl loaded 32-token tiles: 0 = group gloc, all ntl
// token tiles; 1 = group gloc, token tile nt0 only; 2 = nothing (the wave
// still loads its share of the activation tile). Waves w and w + 4 share a
// SIMD.
__device__ __forceinline__ int tl_wave_role(int gl, int ntl, int wave, int& gloc, int& nt0) {
  gloc = wave;
  nt0 = 0;
  if (gl >= kTlWaves) return 0;
  if (gl <= 2) {
    // each group's token tiles on waves of their own: at most one token
    // tile per wave
    if (wave >= gl * ntl) return 2;
    gloc = wave % gl;
    nt0 = wave / gl;
    return 1;
  }
  if (gl == 5) {
    // four whole groups on waves 0..3, one per SIMD; the fifth group's
    // token tiles on waves 4.., one each
    if (wave < 4) return 0;
    if (wave - 4 >= ntl) return 2;
    gloc = 4;
    nt0 = wave - 4;
    return 1;
  }
  return wave < gl ? 0 : 2;
}

// The instance of tile_run for a wave's role (tl_wave_role) in a tile of NTL
// loaded 32-token tiles; with one token tile roles 0 and 1 coincide.
template <int EPI, int NTL>
__device__ __forceinline__ void tile_roles(int role, const FfnArgs& a, uint8_t* xs, int* slot_of,
                                           int* xrow_of, uint16_t* bias_s, int e, int G,
                                           int gloc, int nt0, int rb, int re) {
  if (role == 2) {
    // G only locates the column block here (the wave loads group 0's weights)
    tile_run<EPI, NTL, 1, false>(a, xs, slot_of, xrow_of, bias_s, e, G, 0, 0, rb, re);
  } else if (NTL == 1 || role == 1) {
    tile_run<EPI, NTL, 1, true>(a, xs, slot_of, xrow_of, bias_s, e, G, gloc, nt0, rb, re);
  } else {
    tile_run<EPI, NTL, NTL, true>(a, xs, slot_of, xrow_of, bias_s, e, G, gloc, 0, rb, re);
  }
}

template <int EPI>
__global__ __launch_bounds__(kTlThreads) __attribute__((amdgpu_waves_per_eu(2))) void ffn_tile_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs[kTlStages * kTlStage];
  __shared__ int slot_of[kTlBT];
  __shared__ int xrow_of[kTlBT];
  __shared__ uint16_t bias_s[kTlRows];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int gx = ((a.N >> 6) + kTlWaves - 1) / kTlWaves;
  int wx, ty, e, rb, re;
  // The grid holds an upper bound of the tiles; the real work (gx column
  // blocks x the experts' tiles) is dealt to the 8 XCDs in equal contiguous
  // ranges, so the spare blocks of the bound spread over all XCDs instead of
  // leaving the last ones idle.
  const int total = count_tiles(a.offsets, a.E, kTlBT);
  if (!tile_work_item<kTlChunk>(gx, total, wx, ty)) return;
  find_tile(a.offsets, a.E, kTlBT, ty, e, rb, re);
  const int nvalid = re - rb;
  const int ntl = (nvalid + 31) >> 5;   // 32-token tiles that hold rows (1..4)
  const int gl = min(kTlWaves, (a.N >> 6) - wx * kTlWaves);
  int gloc, nt0;
  const int role = __builtin_amdgcn_readfirstlane(tl_wave_role(gl, ntl, wave, gloc, nt0));
  gloc = __builtin_amdgcn_readfirstlane(gloc);
  nt0 = __builtin_amdgcn_readfirstlane(nt0);
  const int G = wx * kTlWaves + gloc;
  if constexpr (EPI == EPI_SWIGLU) {
    // gate/up: the activation rows come through the slots
    if (tid < kTlBT) slot_of[tid] = tid < nvalid ? a.sorted_rows[rb + tid] : -1;
    {
      const int row = wx * kTlRows + tid;
      bias_s[tid] = row < a.N ? a.bias[(size_t)e * a.N + row] : 0;
    }
    __syncthreads();
    // activation row of each token row of the tile (padded rows: the first)
    if (tid < kTlBT) {
      const int tv = tid < nvalid ? tid : 0;
      xrow_of[tid] = a.gather ? slot_of[tv] / a.k : rb + tv;
    }
    __syncthreads();
  }
  switch (ntl) {
    case 4: tile_roles<EPI, 4>(role, a, xs, slot_of, xrow_of, bias_s, e, G, gloc, nt0, rb, re); break;
    case 3: tile_roles<EPI, 3>(role, a, xs, slot_of, xrow_of, bias_s, e, G, gloc, nt0, rb, re); break;
    case 2: tile_roles<EPI, 2>(role, a, xs, slot_of, xrow_of, bias_s, e, G, gloc, nt0, rb, re); break;
    default: tile_roles<EPI, 1>(role, a, xs, slot_of, xrow_of, bias_s, e, G, gloc, nt0, rb, re); break;
  }
}

// ------------------------------------------------------------------ dispatch
// Largest mean routed rows per expert (T*k / E) for the weight-streaming
// schedule (two 16-token tiles per pass above 10 rows). Measured layer
// crossovers against the tiled schedule: about 28 rows at E = 8 and E = 32,
// 20 at E = 128, 10 at E = 256 (with more experts more of them exceed one
// pass and stream their weights again).
int skinny_max_mean_rows(int E) { return E <= 32 ? 28 : (E <= 128 ? 20 : 10); }

bool ffn_uses_tiles(int n_rows, int E) {
  return (long long)n_rows > (long long)skinny_max_mean_rows(E) * E;
}

hipError_t launch_ffn(const FfnArgs& a, Epilogue epi, int n_rows, hipStream_t s) {
  const int groups = a.N >> 6;
  const bool skinny = !a.act6 && !ffn_uses_tiles(n_rows, a.E);   // records: tiled only
  if (skinny) {
    switch (epi) {
      case EPI_SWIGLU: return launch_skinny<EPI_SWIGLU>(a, n_rows, s);
      case EPI_COMBINE: return launch_skinny<EPI_COMBINE>(a, n_rows, s);
      default: return launch_skinny<EPI_STORE_Y>(a, n_rows, s);
    }
  } else {
    const int tiles = (n_rows + kWdBT - 1) / kWdBT + min(a.E, n_rows);
    const dim3 grid(((groups + kWdGroups - 1) / kWdGroups) * tiles);
    if (a.act6) {
      switch (epi) {
        case EPI_SWIGLU: hipLaunchKernelGGL((ffn_wide6_kernel<EPI_SWIGLU, false>), grid, dim3(256), 0, s, a); break;
        case EPI_COMBINE: hipLaunchKernelGGL((ffn_wide6_kernel<EPI_COMBINE, true>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((ffn_wide6_kernel<EPI_STORE_Y, true>), grid, dim3(256), 0, s, a); break;
      }
      return hipGetLastError();
    }
    // the tiled down instances take h rows in sorted order (rb + t)
    if (epi != EPI_SWIGLU && a.gather) return hipErrorInvalidValue;
    const int tl_tiles = (n_rows + kTlBT - 1) / kTlBT + min(a.E, n_rows);
    const dim3 tl_grid(((groups + kTlWaves - 1) / kTlWaves) * tl_tiles);
    switch (epi) {
      case EPI_SWIGLU: hipLaunchKernelGGL((ffn_tile_kernel<EPI_SWIGLU>), tl_grid, dim3(kTlThreads), 0, s, a); break;
      case EPI_COMBINE: hipLaunchKernelGGL((ffn_tile_kernel<EPI_COMBINE>), tl_grid, dim3(kTlThreads), 0, s, a); break;
      default: hipLaunchKernelGGL((ffn_tile_kernel<EPI_STORE_Y>), tl_grid, dim3(kTlThreads), 0, s, a); break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
