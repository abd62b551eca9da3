/*
 * moe.h -- C ABI of the gpt-oss mixture-of-experts FFN layer on AMD MI355X (gfx950).
 *
 * The layer (one MoE block of gpt-oss-20b / gpt-oss-120b):
 *   logits = x Wr^T + br                         router, fp32
 *   ids    = top-k(logits), k = 4                descending, ties -> lower expert id
 *   w      = softmax(logits[ids])                over the k selected logits
 *   for each selected expert e of a token:
 *     gu   = x W13[e]^T + b13[e]                 W13 in MXFP4, rows interleaved gate/up
 *     gate = min(gu[2i], 7), up = clamp(gu[2i+1], -7, 7)
 *     h    = (up + 1) * gate * sigmoid(1.702 * gate)
 *     y    = h W2[e]^T + b2[e]                   W2 in MXFP4
 *   out    = sum_j w_j y_j
 * Sources: gpt-oss-120b techniques map (models.inteligile.com), "Checked in
 * its code" table -- rows "Mixture of experts" (top-k over router logits),
 * "Auxiliary-loss-free load balancing" (router = linear layer with bias,
 * softmax top-k) and "SwiGLU feed-forward" (gate * sigmoid(gate * alpha),
 * (up + 1) * glu); its "inference & serving" list (MXFP4 weight quantization,
 * MXFP4 tensor packing, BF16 inference); the GPT-OSS 20B / 120B raw
 * config.json tables (hidden_size = intermediate_size = 2880,
 * experts_per_token = 4, num_local_experts = 32 / 128, swiglu_limit = 7).
 * The value alpha = 1.702, the clamp sides, the gate/up interleave and the
 * MXFP4 bit layout are readings where the pages are silent (see below).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - H = I = 2880 are fixed. T >= 0 tokens, 1 <= k <= 8, k <= E <= 256,
 *   T * k <= MOE_MAX_ROUTED. T == 0 returns MOE_SUCCESS at once: no pointer
 *   is examined and nothing is launched.
 * - Every pointer is DEVICE memory owned by the caller. The library allocates
 *   nothing, keeps no state between calls and never modifies inputs.
 *   Outputs are fully overwritten.
 * - bf16 tensors are passed as uint16_t bit patterns. All tensors are
 *   row-major and contiguous; weights are [out_features, in_features].
 * - MXFP4 (OCP Microscaling v1.0), checkpoint ("canonical") layout of a
 *   weight [E, N, K = 2880]: codes [E, N, 1440] u8, byte b of a row holds two
 *   FP4 E2M1 codes, the low nibble for K = 2b and the high nibble for
 *   K = 2b + 1; scales [E, N, 90] u8, byte j is an E8M0 exponent s meaning
 *   2^(s - 127) for K in [32j, 32j + 31]. Scale bytes in [2, 252] give exact
 *   bf16 weights; 255 (NaN) and the extremes are not supported (undefined
 *   results, never checked on the device).
 * - The expert GEMMs read the weights in PACKED order, produced once per
 *   weight tensor by moe_pack_weights (the "MXFP4 tensor packing" step named
 *   in the techniques map's inference list; the order itself is this
 *   library's). Packing permutes bytes inside each group of 64 rows only, so
 *   the packed arrays have the canonical sizes. The GEMM entry points take a
 *   packed tensor only through a moe_packed_weight_t descriptor that
 *   moe_pack_weights has filled: raw code or scale pointers, in either
 *   layout, cannot be passed to them, and a descriptor whose tag, expert
 *   count or row count does not match the call is refused
 *   (MOE_ERROR_LAYOUT).
 * - w13 rows are interleaved: row 2i is gate unit i, row 2i + 1 is up unit i.
 * - Alignment: x, Wr, out, y, h and every code array must be 16-byte aligned,
 *   the bias arrays b13 / b2 8-byte aligned and every scale array 4-byte
 *   aligned; otherwise MOE_ERROR_MISALIGNED. Other arrays need their natural
 *   alignment.
 * - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *   and the call returns without synchronising. Calls on different streams
 *   are independent when they use different workspaces and outputs.
 * - Arguments are validated on the host before anything is launched; a
 *   failed launch returns MOE_ERROR_HIP. Device faults surface at the
 *   caller's next synchronisation. NaN/Inf inputs give undefined results.
 * - `ws` is caller-owned device scratch, 256-byte aligned, of at least
 *   moe_workspace_size_op(op, T, E, k) bytes for the entry point's op
 *   (moe_workspace_size(T, E, k) is enough for every op). Its contents on
 *   entry do not matter. After a layer call (moe_forward, moe_forward_mx6,
 *   moe_forward_block, on the stream) it starts with the routing: the
 *   selected experts int32 [T*k] at offset 0, then their weights fp32 [T*k]
 *   at offset T*k*4 rounded up to a multiple of 256.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_HIDDEN 2880
#define MOE_INTERMEDIATE 2880
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_MAX_ROUTED 4194304 /* T * k: keeps every launch grid in range */

typedef enum moe_status {
  MOE_SUCCESS = 0,
  MOE_ERROR_INVALID_VALUE = 1, /* null pointer or size out of range           */
  MOE_ERROR_MISALIGNED = 2,    /* a pointer lacks the alignment stated above  */
  MOE_ERROR_WORKSPACE = 3,     /* ws is NULL or smaller than required         */
  MOE_ERROR_UNSUPPORTED = 4,   /* current device is not gfx950                */
  MOE_ERROR_HIP = 5,           /* a HIP runtime call or launch failed         */
  MOE_ERROR_LAYOUT = 6,        /* a weight descriptor not filled by           */
                               /* moe_pack_weights, or of other E / N         */
  MOE_ERROR_RANGE = 7          /* weights whose scale spread exceeds what the */
                               /* FP6-piece path is accurate for              */
} moe_status_t;

/* One packed MXFP4 weight tensor [E, N, K = 2880] (E experts of N rows).
 * moe_pack_weights fills it; the library reads it on the host at call time
 * only (the descriptor itself may live anywhere; codes and scales are device
 * memory owned by the caller and must stay valid while kernels run). */
#define MOE_PACKED_TAG 0x3450584Du /* "MXP4" */
typedef struct moe_packed_weight {
  const uint8_t* codes;   /* packed codes, E * N * 1440 bytes, 16-byte aligned */
  const uint8_t* scales;  /* packed scales, E * N * 90 bytes, 4-byte aligned   */
  int32_t E;              /* experts                                           */
  int32_t N;              /* rows per expert: 5760 (gate/up) or 2880 (down)    */
  uint32_t tag;           /* MOE_PACKED_TAG once packed                        */
  uint32_t scale_spread;  /* largest (max - min) of the E8M0 scale exponents   */
                          /* within one expert (NaN bytes excluded), in binades */
} moe_packed_weight_t;

/* Largest scale_spread for which the FP6-piece path (moe_forward_mx6 on its
 * tiled schedule, moe_gate_up_mx6) meets the accuracy bar of moe_forward. */
#define MOE_MX6_MAX_SCALE_SPREAD 16u

/* The entry points that take a workspace, for moe_workspace_size_op. */
typedef enum moe_op {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_EXPERT_FFN = 2,
  MOE_OP_FORWARD = 3,
  MOE_OP_FORWARD_MX6 = 4,
  MOE_OP_FORWARD_BLOCK = 5
} moe_op_t;

/* Bytes of scratch `ws` that the entry point `op` needs for (T, E, k): the
 * routing arrays, the router's scratch and, for the layer calls, the
 * intermediate h [T*k, 2880] bf16 and per-slot outputs [T*k, 2880] fp32
 * (plus the FP6 records of moe_forward_mx6 and the normed input of
 * moe_forward_block). At least 256. Returns 0 when the sizes or op are out
 * of range. */
size_t moe_workspace_size_op(moe_op_t op, int T, int E, int k);

/* The largest moe_workspace_size_op over every op: one workspace of this size
 * serves any call with these sizes. Returns 0 when the sizes are out of
 * range. */
size_t moe_workspace_size(int T, int E, int k);

/* Packs one MXFP4 weight tensor from the canonical layout into the order the
 * expert GEMMs read (see the conventions above) and fills `desc` (host
 * memory) with the packed arrays, E, N, MOE_PACKED_TAG and the tensor's
 * scale_spread. N % 64 == 0, 64 <= N <= 65536, 1 <= E <= 256; K = 2880.
 * A one-time setup call: it allocates a small device buffer for the scale
 * ranges and synchronises `stream` before returning.
 *   codes [E, N, 1440] u8, scales [E, N, 90] u8 (canonical, in)
 *   packed_codes, packed_scales: same sizes (out; must not overlap the input)
 *   desc: written only when the call succeeds
 * Packed order, per group G of rows [64G, 64G + 64) of one expert:
 *   codes: 23 K steps s of four MX blocks (4s .. 4s + 3); step s holds four
 *     16-row tiles m; tile m holds 64 lanes l = 16g + r of 16 bytes, lane l
 *     carrying the codes of row 64G + 16m + r, block 4s + g. The last step
 *     (blocks 88, 89) holds lanes 0..31 only: 512 bytes per tile.
 *     offset = G*92160 + s*4096 + m*(s < 22 ? 1024 : 512) + l*16.
 *   scales: offset = G*5760 + s*256 + l*4 + m for the same (s, m, l). */
moe_status_t moe_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N,
                              uint8_t* packed_codes, uint8_t* packed_scales,
                              moe_packed_weight_t* desc, void* stream);

/* Router: logits = x Wr^T + br in fp32, then per token the k largest logits
 * (descending; equal logits -> lower expert id) and their softmax.
 *   x        [T, 2880] bf16      Wr [E, 2880] fp32     br [E] fp32
 *   topk_ids [T, k] int32 (out)  topk_w [T, k] fp32 (out)
 *   logits   [T, E] fp32 (out, optional: NULL to skip)
 * Uses the same kernels, in the same order, as moe_forward's routing, so both
 * select the same experts. Source: techniques map rows "Mixture of experts"
 * and "Auxiliary-loss-free load balancing". */
moe_status_t moe_route(const uint16_t* x, const float* Wr, const float* br,
                       int T, int E, int k,
                       int32_t* topk_ids, float* topk_w, float* logits,
                       void* ws, size_t ws_bytes, void* stream);

/* Group the T*k routed slots by expert (counting sort, stable):
 *   counts[e]      number of slots routed to expert e            [E]
 *   offsets[e]     exclusive prefix sum of counts, offsets[E]=T*k [E + 1]
 *   sorted_rows[p] flat slot index t*k + j; slots of expert e are
 *                  sorted_rows[offsets[e] .. offsets[e+1]), ascending [T*k]
 * topk_ids [T, k] int32, every entry in [0, E). Not on the pages: this is the
 * grouping step of a grouped-GEMM MoE. */
moe_status_t moe_permute(const int32_t* topk_ids, int T, int E, int k,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_rows,
                         void* ws, size_t ws_bytes, void* stream);

/* Every routed slot through its expert, unweighted:
 *   y[t*k + j, :] = W2[e] h + b2[e],  h = SwiGLU(W13[e] x[t] + b13[e]), e = ids[t, j]
 *   offsets, sorted_rows   as produced by moe_permute
 *   w13 packed gate/up weights (E experts x 5760 rows)    b13 [E, 5760] bf16
 *   w2  packed down weights    (E experts x 2880 rows)    b2  [E, 2880] bf16
 *   y [T*k, 2880] fp32 (out)
 * The gate/up intermediate h is rounded to bf16 (the matrix-core input type).
 * Source: techniques map row "SwiGLU feed-forward"; swiglu_limit from the raw
 * config.json tables; MXFP4 from the "inference & serving" list. */
moe_status_t moe_expert_ffn(const uint16_t* x, const int32_t* offsets,
                            const int32_t* sorted_rows,
                            const moe_packed_weight_t* w13, const uint16_t* b13,
                            const moe_packed_weight_t* w2, const uint16_t* b2,
                            int T, int E, int k, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_expert_ffn / moe_forward as separate calls.
 *
 * moe_gate_up: gate/up projection and SwiGLU of every routed slot, in
 * expert-sorted order:
 *   h[p, :] = bf16( SwiGLU( W13[e] x[t] + b13[e] ) ),  t = sorted_rows[p] / k,
 *   e = the expert whose range [offsets[e], offsets[e+1]) contains p.
 *   h [T*k, 2880] bf16 (out). Source: techniques map row "SwiGLU feed-forward".
 *
 * moe_down_accumulate: down projection of h, weighted by the routing weight
 * and ADDED into out:
 *   out[t, :] += topk_w[s] * ( W2[e] h[p, :] + b2[e] ),  s = sorted_rows[p], t = s / k
 *   h [T*k, 2880] bf16 as moe_gate_up wrote it; topk_w [T, k] fp32, indexed
 *   by slot s = t*k + j (moe_route's weights).
 *   out [T, 2880] fp32 is accumulated, not overwritten: pass zeros for the
 *   layer output, or the residual stream to fold the residual add in. The
 *   order in which a token's k contributions are added is not fixed (atomic
 *   adds), so results may differ in the last bits from run to run.
 *   Source: techniques map, "Mixture of experts" (weighted sum of experts). */
moe_status_t moe_gate_up(const uint16_t* x, const int32_t* offsets,
                         const int32_t* sorted_rows,
                         const moe_packed_weight_t* w13, const uint16_t* b13,
                         int T, int E, int k,
                         uint16_t* h, void* stream);

moe_status_t moe_down_accumulate(const uint16_t* h, const int32_t* offsets,
                                 const int32_t* sorted_rows, const float* topk_w,
                                 const moe_packed_weight_t* w2, const uint16_t* b2,
                                 int T, int E, int k,
                                 float* out, void* stream);

/* out[t, :] = sum_j topk_w[t, j] * y[t*k + j, :]
 *   y [T*k, 2880] fp32, topk_w [T, k] fp32, out [T, 2880] fp32 (out).
 * Source: the weighted sum of the selected experts' outputs (techniques map,
 * "Mixture of experts"). */
moe_status_t moe_combine(const float* y, const float* topk_w, int T, int k,
                         float* out, void* stream);

/* The whole layer: route -> permute -> gate/up + SwiGLU -> down projection
 * -> routing-weighted combine (a token's k expert outputs summed in slot
 * order: results are reproducible bit for bit). Few routed rows per expert
 * (T*k <= 28*E for E <= 32, 20*E for E <= 128, else 10*E) take the
 * weight-streaming schedule, which finds each expert's slots in the routing
 * ids instead of building the permutation.
 * Arguments as above; out [T, 2880] fp32 is overwritten. */
moe_status_t moe_forward(const uint16_t* x, const float* Wr, const float* br,
                         const moe_packed_weight_t* w13, const uint16_t* b13,
                         const moe_packed_weight_t* w2, const uint16_t* b2,
                         int T, int E, int k, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/* The same layer with the tiled (many rows per expert) expert GEMMs on the
 * block-scaled FP4 matrix cores of CDNA4 (v_mfma_scale_f32_16x16x128_f8f6f4):
 * the MXFP4 weights enter the instruction as they are (their E8M0 scales are
 * the instruction's block scales) and each activation row x[t] is held as
 * two MX FP6 (E2M3) pieces, P1 + P2 (moe_encode_mx6), each multiplied by the
 * weights at the FP4 x FP6 rate; the down projection takes the gate/up output
 * h the same way (rounded to bf16, then encoded by the gate/up kernel as it
 * writes h). The pieces stand for a row to within max|block| / 256 per
 * 32-value block; the layer output stays within the accuracy bar of
 * moe_forward while the weight scales of an expert span up to 16 binades
 * (checkpoint-like weights span a few): where the tiled schedule runs and
 * w13 or w2 has a scale_spread above MOE_MX6_MAX_SCALE_SPREAD the call is
 * refused with MOE_ERROR_RANGE (use moe_forward). The few-rows-per-expert
 * (decode) schedule is that of moe_forward and has no such limit.
 * Arguments and errors as moe_forward; the workspace (moe_workspace_size)
 * also holds the records of x and h. Source: the pages fix MXFP4 weights
 * and their packing for inference (techniques map, "inference & serving");
 * the piece encoding follows the OCP Microscaling v1.0 conversion and is
 * this library's. */
moe_status_t moe_forward_mx6(const uint16_t* x, const float* Wr, const float* br,
                             const moe_packed_weight_t* w13, const uint16_t* b13,
                             const moe_packed_weight_t* w2, const uint16_t* b2,
                             int T, int E, int k, float* out,
                             void* ws, size_t ws_bytes, void* stream);

/* Two-piece MX FP6 encoding of bf16 activation rows, as moe_forward_mx6 uses it:
 *   x       [rows, 2880] bf16 (in), 16-byte aligned
 *   records [rows, 23, 256] u8 (out), 16-byte aligned
 * 0 <= rows <= MOE_MAX_ROUTED. For each 32-value block V of a row (OCP MX
 * v1.0 conversion to FP6 E2M3): X = floor(log2(max|V|)) - 2, clamped to
 * [-127, 127] (0 for an all-zero block); codes = V / 2^X rounded to the
 * nearest E2M3 value, ties to even, saturating at 7.5; sign bit set for
 * negative values; scale byte X + 127. Piece 1 encodes V, piece 2 the exact
 * residual V - piece 1. Record s of a row covers MX blocks 4s .. 4s+3 (blocks
 * 90, 91 are zero codes with scale byte 127) as sixteen 16-byte chunks:
 *   0..3   piece 1, block g = 0..3: code bytes 0..15
 *   4..7   piece 2, the same
 *   8, 9   piece 1: code bytes 16..23 of blocks 0, 1 (chunk 8) and 2, 3 (chunk 9)
 *   10, 11 piece 2, the same
 *   12     scale bytes: byte 2g = piece 1, byte 2g + 1 = piece 2 of block g;
 *          bytes 8..15 zero
 *   13..15 zero
 * Element j of a block sits at bits 6j .. 6j+5 of its 24 code bytes (little
 * endian). */
moe_status_t moe_encode_mx6(const uint16_t* x, int rows, uint8_t* records, void* stream);

/* moe_gate_up with the activations given as moe_encode_mx6 records
 * x_records [T, 23, 256] u8 (16-byte aligned) instead of bf16 rows: the
 * block-scaled FP4 x FP6 gate/up GEMM of moe_forward_mx6, always in its tiled
 * schedule: refused with MOE_ERROR_RANGE when w13's scale_spread exceeds
 * MOE_MX6_MAX_SCALE_SPREAD. Other arguments, output and errors as
 * moe_gate_up. */
moe_status_t moe_gate_up_mx6(const uint8_t* x_records, const int32_t* offsets,
                             const int32_t* sorted_rows,
                             const moe_packed_weight_t* w13, const uint16_t* b13,
                             int T, int E, int k,
                             uint16_t* h, void* stream);

/* The MoE sublayer of a gpt-oss decoder layer with its neighbours: the
 * pre-MoE RMSNorm and the residual add.
 *   t   = x / sqrt(mean_h(x^2) + norm_eps) * norm_scale   per token (fp32)
 *   out = x + layer(t): the router on t, the expert GEMMs on bf16(t)
 *   x          [T, 2880] bf16, the residual stream entering the sublayer
 *   norm_scale [2880] fp32 (16-byte aligned); norm_eps >= 0 (gpt-oss: 1e-5)
 *   out        [T, 2880] fp32 (overwritten)
 * Other arguments, workspace and errors as moe_forward. Sources: the
 * "gpt-oss-20b" page, "Structure" table (every layer runs RMSNorm_i_2 ->
 * MoE_i -> Add_i_ffn); techniques map, "normalization & residual" (RMSNorm,
 * Pre-LN); rms_norm_eps from the raw config.json tables. Readings: the norm
 * is computed in fp32; the fp32 router takes it unrounded, as
 * inv_rms * (x . (Wr[e] * norm_scale)); the expert GEMMs take it rounded to
 * bf16 (their matrix-core input type); the residual is added in fp32. With
 * few tokens (T <= 128, T*E <= 4096) on the weight-streaming schedule no
 * norm kernel runs: the router forms each token's inverse RMS from its own
 * sums of squares and its finish launch writes the normed rows. */
moe_status_t moe_forward_block(const uint16_t* x, const float* norm_scale, float norm_eps,
                               const float* Wr, const float* br,
                               const moe_packed_weight_t* w13, const uint16_t* b13,
                               const moe_packed_weight_t* w2, const uint16_t* b2,
                               int T, int E, int k, float* out,
                               void* ws, size_t ws_bytes, void* stream);

/* The RMSNorm of moe_forward_block alone:
 *   t[r, :] = bf16( x[r, :] / sqrt(mean(x[r, :]^2) + eps) * scale )
 *   x [T, 2880] bf16, t [T, 2880] bf16 (out), both 16-byte aligned;
 *   scale [2880] fp32, 16-byte aligned; eps >= 0; 0 <= T <= MOE_MAX_ROUTED.
 * Source as moe_forward_block. */
moe_status_t moe_rmsnorm(const uint16_t* x, const float* scale, float eps, int T,
                         uint16_t* t, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same layer and kernels, with the workspace taken from a scratch array the
 * library holds in device memory (MOE_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends) instead of a `ws` argument. The call allocates
 * nothing: on its first call on a device it looks up that device's copy of
 * the array (hipGetSymbolAddress, with the device current) and keeps the
 * address. Sizes whose moe_workspace_size_op(MOE_OP_FORWARD, T, E, k) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES are refused with MOE_ERROR_WORKSPACE (up to
 * about 3,100 routed slots fit: T = 784 at k = 4 for any E). Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or graphs replayed concurrently) race and give
 * undefined results; calls ordered on one stream are safe. No part of the
 * array needs clearing between calls. Other arguments, output and errors as
 * moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (56u << 20)
moe_status_t moe_forward_noalloc(const uint16_t* x, const float* Wr, const float* br,
                                 const moe_packed_weight_t* w13, const uint16_t* b13,
                                 const moe_packed_weight_t* w2, const uint16_t* b2,
                                 int T, int E, int k, float* out, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
