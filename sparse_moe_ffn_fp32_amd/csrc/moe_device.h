// Device-side building blocks shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace moe {

constexpr int kH = 2880;            // hidden_size (GPT-OSS raw config.json fields)
constexpr int kI = 2880;            // intermediate_size
constexpr int kN13 = 2 * kI;        // gate/up rows, interleaved gate 2i / up 2i+1
constexpr int kKB = kH / 32;        // MX blocks along K; H == I so both GEMMs have 90
constexpr int kRowCodeBytes = kH / 2;   // 1440 code bytes per weight row
constexpr int kRowScaleBytes = kKB;     // 90 scale bytes per weight row
constexpr float kSwigluAlpha = 1.702f;  // reading: the techniques map names alpha, no value
constexpr float kSwigluLimit = 7.0f;    // swiglu_limit, raw config.json fields
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

// Packed MXFP4 order (moe_pack_weights): per 64-row group, K steps of four MX
// blocks; step s holds four 16-row tiles of 64 lanes x 16 code bytes (the
// last step, blocks 88 and 89, only lanes 0..31), then scales as 4 bytes per
// lane (one per tile).
constexpr int kSteps = 23;               // ceil(90 / 4)
constexpr int kFullSteps = 22;           // steps with all four blocks
constexpr int kStepCodeBytes = 4096;     // four tiles x 1 KiB
constexpr int kGroupCodeBytes = 64 * kRowCodeBytes;    // 92,160
constexpr int kGroupScaleBytes = 64 * kRowScaleBytes;  // 5,760

// Two-piece MX FP6 activation records (the block-scaled matrix-core path):
// an activation row v is held as P1 + P2, P1 the MX E2M3 encoding of v and
// P2 that of the exact residual v - P1 (OCP MX v1.0 conversion: shared
// exponent floor(log2(amax)) - 2, round to nearest even, saturate at 7.5).
// Per row, one 256-byte record per K step s of four MX blocks (blocks 90, 91
// of the last step are zero codes with scale 2^0). A record is sixteen
// 16-byte pieces: 0..3 = piece 1 code bytes 0..15 of block g; 4..7 = piece 2
// the same; 8, 9 = piece 1 code bytes 16..23 of blocks (0, 1) and (2, 3);
// 10, 11 = piece 2 the same; 12 = scale bytes, byte 2g + p for piece p of
// block g, then 8 zero bytes; 13..15 = zero. Element j of a block sits at
// bits 6j..6j+5 of its 24 code bytes (little endian), the operand order of
// the f8f6f4 matrix-core instructions.
constexpr int kRecBytes = 256;
constexpr int kRowRecBytes = kSteps * kRecBytes;   // 5,888 per activation row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

// operand format codes of the f8f6f4 matrix-core instructions
constexpr int kFmtE2M3 = 2;
constexpr int kFmtFp4 = 4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats -> packed bf16 bits, lo in the low half (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2));
}

// E8M0 byte -> the fp32 scale 2^(s-127) (s in [1, 254]).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s << 23);
}

// Eight FP4 E2M1 codes (one dword, low nibble first) -> eight bf16 values
// scaled by `scale`, in K order. v_cvt_scalef32_pk_bf16_fp4 converts the two
// codes of one byte; the byte is chosen by the last operand.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8 u4_as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// bf16(x * inv * scale) of 8 consecutive bf16 values (two per dword) and their
// 8 scale values: the decoder block's RMSNorm applied to one 16-byte piece
__device__ __forceinline__ uint4 norm_apply8(const uint4 d, float inv, const float4 s0,
                                             const float4 s1) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = f32x2_to_bf16x2_bits(bf16_bits_to_f32(dw[q] & 0xFFFFu) * inv * s[2 * q],
                                bf16_bits_to_f32(dw[q] >> 16) * inv * s[2 * q + 1]);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// gpt-oss gated unit for one (gate, up) pair, after the bias.
__device__ __forceinline__ float swiglu_pair(float gate, float up) {
  constexpr float kNegAlphaLog2e = -kSwigluAlpha * 1.44269504088896341f;
  gate = fminf(gate, kSwigluLimit);
  up = fminf(fmaxf(up, -kSwigluLimit), kSwigluLimit);
  // sigma(alpha * gate) = 1 / (1 + 2^(-alpha * log2(e) * gate)) on v_exp_f32
  // and v_rcp_f32 (about 1 ulp each; the result is rounded to bf16)
  const float glu = gate * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gate * kNegAlphaLog2e));
  return fmaf(up, glu, glu);   // (up + 1) * glu
}

// Locate token tile `tile` of a grouped GEMM whose experts own the row ranges
// [offsets[e], offsets[e+1]) split into tiles of `bt` rows. Run by one full
// wave (all 64 lanes get the same answer). Returns false past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int bt,
                                          int tile, int& expert, int& row_begin, int& row_end) {
  const int lane = threadIdx.x & 63;
  int cnt[4], tiles[4];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane * 4 + q;
    int c = 0;
    if (e < E) c = offsets[e + 1] - offsets[e];
    cnt[q] = c;
    tiles[q] = (c + bt - 1) / bt;
    local += tiles[q];
  }
  // inclusive scan of per-lane totals across the wave
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  const int excl = incl - local;
  const int total = __shfl(incl, 63, 64);
  if (tile >= total) return false;
  // the lane whose range holds `tile`
  const bool mine = (tile >= excl) && (tile < incl);
  const unsigned long long ball = __ballot(mine);
  const int owner = __ffsll((long long)ball) - 1;
  int e_found = 0, t_in = 0;
  if (mine) {
    int t = tile - excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (t >= 0 && t < tiles[q]) { e_found = lane * 4 + q; t_in = t; }
      t -= tiles[q];
    }
  }
  e_found = __shfl(e_found, owner, 64);
  t_in = __shfl(t_in, owner, 64);
  expert = e_found;
  const int base = offsets[e_found];
  const int n = offsets[e_found + 1] - base;
  row_begin = base + t_in * bt;
  row_end = base + min(n, (t_in + 1) * bt);
  (void)cnt;
  return true;
}

// ------------------------------------------------- MX FP6 (E2M3) encoding
// Shared exponent of a block with largest magnitude amax: floor(log2(amax))
// - 2 (emax of E2M3), clamped to the E8M0 range; 0 for an all-zero block.
__device__ __forceinline__ int mx6_shared_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const int X = __builtin_amdgcn_frexp_expf(amax) - 3;   // amax = f * 2^e, f in [0.5, 1)
  return min(max(X, -127), 127);
}

// E2M3 magnitude code nearest to a >= 0 (ties to the even code, saturating
// at 7.5) and its value q. Within the binade [2^e, 2^(e+1)) (e = 0 also
// covers the subnormals) the grid step is 2^(e-3), so the code is 8e plus
// the rounded multiple of the step; a carry into the next binade lands on
// the right code because codes count up through the binades.
__device__ __forceinline__ uint32_t e2m3_mag_code(float a, float& q) {
  a = fminf(a, 7.5f);
  const int e = a >= 4.f ? 2 : (a >= 2.f ? 1 : 0);
  const float n = rintf(ldexpf(a, 3 - e));
  q = ldexpf(n, e - 3);
  return 8u * (uint32_t)e + (uint32_t)n;
}

// One MX E2M3 piece of 32 values: codes packed 6 bits each (element j at
// bits 6j) into w[0..5], the scale byte, and the exact residual v - piece.
__device__ __forceinline__ void mx6_encode_piece(const float (&v)[32], uint32_t (&w)[6],
                                                 uint32_t& scale, float (&res)[32]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int X = mx6_shared_exp(amax);
#pragma unroll
  for (int i = 0; i < 6; ++i) w[i] = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float q;
    uint32_t c = e2m3_mag_code(ldexpf(fabsf(v[j]), -X), q);
    if (v[j] < 0.f) {
      c |= 32u;
      q = -q;
    }
    res[j] = v[j] - ldexpf(q, X);
    const int bit = 6 * j, word = bit >> 5, off = bit & 31;
    w[word] |= c << off;
    if (off > 26) w[word + 1] |= c >> (32 - off);
  }
  scale = (uint32_t)(X + 127);
}

// The same piece on CDNA4's scaled conversion instructions: the 32 values
// divided by 2^X and rounded to E2M3 (nearest even, saturating) in one
// instruction, whose two 16-value operands are interleaved in its output
// (output j = operand a[j/2] for even j, b[j/2] for odd j), and the piece's
// values back by the inverse conversion. Returns false, leaving the outputs
// unset, when 2^X or the piece's smallest values would not be normal floats
// (X < -120): the caller then takes the arithmetic path above. Bit for bit
// the same codes as mx6_encode_piece for every input but -0.0, which the
// instruction encodes with its sign bit set (callers pass +0.0).
__device__ __forceinline__ bool mx6_encode_piece_cvt(const float (&v)[32], uint32_t (&w)[6],
                                                     uint32_t& scale, float (&res)[32]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int X = mx6_shared_exp(amax);
  if (X < -120) return false;
  const float sc = ldexpf(1.0f, X);
  f32x16 a, b;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = v[2 * i];
    b[i] = v[2 * i + 1];
  }
  const u32x6 c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, sc);
  const f32x32 q = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, sc);
#pragma unroll
  for (int i = 0; i < 6; ++i) w[i] = c[i];
#pragma unroll
  for (int j = 0; j < 32; ++j) res[j] = v[j] - q[j];
  scale = (uint32_t)(X + 127);
  return true;
}

// Both pieces of a 32-value block.
__device__ __forceinline__ void mx6x2_encode(const float (&v)[32], uint32_t (&w1)[6], uint32_t& s1,
                                             uint32_t (&w2)[6], uint32_t& s2) {
  float v0[32], r1[32], r2[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v0[j] = v[j] + 0.0f;   // -0.0 -> +0.0
  if (!mx6_encode_piece_cvt(v0, w1, s1, r1)) mx6_encode_piece(v0, w1, s1, r1);
  if (!mx6_encode_piece_cvt(r1, w2, s2, r2)) mx6_encode_piece(r1, w2, s2, r2);
}

// Compile-time loop: f(integral_constant<int, i>) for i = 0 .. N-1, each call
// its own code (a fully unrolled loop whose steps cannot be merged or rolled).
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

}  // namespace moe
