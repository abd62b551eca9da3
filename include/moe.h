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
 * - MXFP4 (OCP Microscaling v1.0): codes[n, b] holds two FP4 E2M1 codes, the
 *   low nibble for K = 2b and the high nibble for K = 2b + 1; scales[n, j] is
 *   an E8M0 byte s meaning 2^(s - 127) for K in [32j, 32j + 31]. Scale bytes
 *   in [2, 252] give exact bf16 weights; 255 (NaN) and the extremes are not
 *   supported (undefined results, never checked on the device).
 * - w13 rows are interleaved: row 2i is gate unit i, row 2i + 1 is up unit i.
 * - Alignment: x, Wr, out, y and every code array must be 16-byte aligned;
 *   otherwise MOE_ERROR_MISALIGNED. Other arrays need their natural alignment.
 * - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *   and the call returns without synchronising. Calls on different streams
 *   are independent when they use different workspaces and outputs.
 * - Arguments are validated on the host before anything is launched; a
 *   failed launch returns MOE_ERROR_HIP. Device faults surface at the
 *   caller's next synchronisation. NaN/Inf inputs give undefined results.
 * - `ws` is caller-owned device scratch of at least moe_workspace_size(T,E,k)
 *   bytes, 256-byte aligned. Its contents on entry do not matter.
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
  MOE_ERROR_HIP = 5            /* a HIP runtime call or launch failed         */
} moe_status_t;

/* Bytes of scratch `ws` that every entry point below may use for (T, E, k).
 * Returns 0 when the sizes are out of range. */
size_t moe_workspace_size(int T, int E, int k);

/* Router: logits = x Wr^T + br in fp32, then per token the k largest logits
 * (descending; equal logits -> lower expert id) and their softmax.
 *   x        [T, 2880] bf16      Wr [E, 2880] fp32     br [E] fp32
 *   topk_ids [T, k] int32 (out)  topk_w [T, k] fp32 (out)
 *   logits   [T, E] fp32 (out, optional: NULL to skip)
 * Source: techniques map rows "Mixture of experts" and "Auxiliary-loss-free
 * load balancing". */
moe_status_t moe_route(const uint16_t* x, const float* Wr, const float* br,
                       int T, int E, int k,
                       int32_t* topk_ids, float* topk_w, float* logits,
                       void* stream);

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
 *   w13_codes [E, 5760, 1440] u8   w13_scales [E, 5760, 90] u8   b13 [E, 5760] bf16
 *   w2_codes  [E, 2880, 1440] u8   w2_scales  [E, 2880, 90] u8   b2  [E, 2880] bf16
 *   y [T*k, 2880] fp32 (out)
 * The gate/up intermediate h is rounded to bf16 (the matrix-core input type).
 * Source: techniques map row "SwiGLU feed-forward"; swiglu_limit from the raw
 * config.json tables; MXFP4 from the "inference & serving" list. */
moe_status_t moe_expert_ffn(const uint16_t* x, const int32_t* offsets,
                            const int32_t* sorted_rows,
                            const uint8_t* w13_codes, const uint8_t* w13_scales,
                            const uint16_t* b13,
                            const uint8_t* w2_codes, const uint8_t* w2_scales,
                            const uint16_t* b2,
                            int T, int E, int k, float* y,
                            void* ws, size_t ws_bytes, void* stream);

/* out[t, :] = sum_j topk_w[t, j] * y[t*k + j, :]
 *   y [T*k, 2880] fp32, topk_w [T, k] fp32, out [T, 2880] fp32 (out).
 * Source: the weighted sum of the selected experts' outputs (techniques map,
 * "Mixture of experts"). */
moe_status_t moe_combine(const float* y, const float* topk_w, int T, int k,
                         float* out, void* stream);

/* The whole layer: route -> permute -> gate/up + SwiGLU -> down projection
 * with the routing-weighted combine fused into its epilogue.
 * Arguments as above; out [T, 2880] fp32 is overwritten. */
moe_status_t moe_forward(const uint16_t* x, const float* Wr, const float* br,
                         const uint8_t* w13_codes, const uint8_t* w13_scales,
                         const uint16_t* b13,
                         const uint8_t* w2_codes, const uint8_t* w2_scales,
                         const uint16_t* b2,
                         int T, int E, int k, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
