// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum Epilogue : int {
  EPI_SWIGLU = 0,   // gate/up GEMM: + b13, clamp, SwiGLU, write h (bf16, sorted order)
  EPI_COMBINE = 1,  // down GEMM: + b2, times routing weight, atomic add into out[t]
  EPI_STORE_Y = 2,  // down GEMM: + b2, write y[t*k + j] (fp32)
};

struct FfnArgs {
  const uint16_t* act;          // activations, bf16 [rows, 2880]
  const int32_t* offsets;       // [E + 1]
  const int32_t* sorted_rows;   // [T*k]
  const uint8_t* codes;         // [E, N, 1440]
  const uint8_t* scales;        // [E, N, 90]
  const uint16_t* bias;         // [E, N] bf16
  const float* topk_w;          // [T*k]       (EPI_COMBINE)
  uint16_t* h_out;              // [T*k, 2880] (EPI_SWIGLU)
  float* y_out;                 // [T*k, 2880] (EPI_STORE_Y)
  float* out;                   // [T, 2880]   (EPI_COMBINE)
  int N;                        // weight rows: 5760 (gate/up) or 2880 (down)
  int E;
  int k;
  int gather;                   // 1: activation row = sorted_rows[p] / k, 0: row p
  // Weight-streaming kernels only: when not null, each wave finds its
  // expert's slots in the routing ids [n_slots] itself (same stable order and
  // positions as the permutation) and offsets / sorted_rows are not read.
  const int32_t* ids;
  int n_slots;
  // Tiled kernels only: when not null, the activations are read from these
  // two-piece MX FP6 records ([rows, 23 steps, 256 B], moe_device.h) through
  // the block-scaled FP4 x FP6 matrix-core instruction instead of `act`.
  const uint8_t* act6;
  // Tiled gate/up on records (EPI_SWIGLU with act6) only: when not null, h is written as two-piece
  // MX FP6 records [T*k, 23 steps, 256 B] for a block-scaled down projection
  // instead of bf16 into h_out (the bytes no kernel reads are left unwritten).
  uint8_t* h6_out;
};

// The decoder block's RMSNorm folded into the router: the router's input is
// t = x * inv * scale per token (inv = 1 / sqrt(mean(x^2) + eps)), computed as
// inv * (x . (Wr[e] * scale)). `inv_ready`: inv [T] was written by the norm
// kernel (required with many tokens). Otherwise (few tokens) the router forms
// inv from x itself, and with `t_out` also writes the expert GEMMs' input
// t_out = bf16(x * inv * scale) [T, 2880] (not with a permutation).
struct RouteNorm {
  const float* scale;   // [2880]
  float eps;
  const float* inv;     // [T]
  bool inv_ready;
  uint16_t* t_out;
};

// Router + top-k + softmax; with `counts` non-null the expert permutation is
// built as well. `scratch` holds route_scratch_bytes(T, E) bytes. `norm`
// (may be null): the decoder block's norm, above.
hipError_t launch_route(const uint16_t* x, const float* Wr, const float* br, int T, int E, int k,
                        int32_t* ids, float* w, float* logits, float* scratch,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                        const RouteNorm* norm, hipStream_t s);
bool route_few_tokens(int T, int E);
size_t route_scratch_bytes(int T, int E);

// canonical MXFP4 codes/scales [E, N, ...] -> the packed order of the GEMMs
hipError_t launch_pack(const uint8_t* codes, const uint8_t* scales, int E, int N, uint8_t* pcodes,
                       uint8_t* pscales, hipStream_t s);
// smallest and largest E8M0 scale byte (255 excluded) of each expert: lohi [2E]
hipError_t launch_scale_range(const uint8_t* scales, int E, int N, int32_t* lohi, hipStream_t s);

// Stable permutation of n = T*k slots. Up to 1024 slots (or without hist):
// one workgroup; above: a histogram pass into hist (ceil(T/32)*E ints), a
// scan and a parallel scatter.
hipError_t launch_permute(const int32_t* ids, int n, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_rows, int32_t* hist, hipStream_t s);
// Same permutation from per-block expert histograms hist[nb][E] of
// consecutive slot ranges of spb slots each (spb <= 256); hist is
// overwritten (it becomes the blocks' base positions).
hipError_t launch_permute_blocks(const int32_t* ids, int n, int E, int32_t* hist, int nb, int spb,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                                 hipStream_t s);

// Picks the weight-streaming (few rows per expert) or the tiled (many rows)
// grouped GEMM from the mean rows per expert, n_rows / E.
hipError_t launch_ffn(const FfnArgs& a, Epilogue epi, int n_rows, hipStream_t s);
bool ffn_uses_tiles(int n_rows, int E);

// bf16 rows [rows, 2880] -> two-piece MX FP6 records [rows, 23, 256 B]
hipError_t launch_mx6_encode(const uint16_t* x, int rows, uint8_t* rec, hipStream_t s);

// out[t] = resid[t] (bf16, optional) + sum_j w[t, j] y[t*k + j]
hipError_t launch_combine(const float* y, const float* w, int T, int k, const uint16_t* resid,
                          float* out, hipStream_t s);

// t = bf16(x / sqrt(mean(x^2) + eps) * scale) per row of x [T, 2880] bf16;
// with `inv` non-null also each row's 1 / sqrt(mean(x^2) + eps) [T]
hipError_t launch_rmsnorm(const uint16_t* x, const float* scale, float eps, int T, uint16_t* t,
                          float* inv, hipStream_t s);

}  // namespace moe
