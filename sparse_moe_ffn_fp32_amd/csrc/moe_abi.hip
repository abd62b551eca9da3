// C ABI of the MoE layer: argument validation on the host, workspace carve-up,
// kernel launches on the caller's stream. No allocation, no host sync (unless
// MOE_DEBUG_SYNC=1 is set in the environment, which synchronises and checks
// after every launch).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>
#include <algorithm>

#include "moe.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace {

using moe::FfnArgs;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
  size_t ids, w, counts, offsets, sorted, scratch, h, y, xrec, xnorm, hrec, inv, total;
};

bool sizes_ok(int T, int E, int k) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < k || E > MOE_MAX_EXPERTS) return false;
  return (long long)T * k <= MOE_MAX_ROUTED;
}

bool op_ok(int op) { return op >= MOE_OP_ROUTE && op <= MOE_OP_FORWARD_BLOCK; }

// moe_forward_block without a norm kernel: the few-token router forms each
// token's inverse RMS from its chunk sums of squares, and its finish launch
// (without a permutation: the weight-streaming schedule) also writes the
// normed rows for the expert GEMMs. Otherwise the norm kernel writes the rows
// and the inverse RMS, which the router takes.
bool block_norm_folded(int T, int E, int k) {
  return moe::route_few_tokens(T, E) && !moe::ffn_uses_tiles(T * k, E);
}

// Carve-up of the workspace of entry point `op`: only what that call uses.
// Regions an op does not use have size 0 (their offsets are then unused).
WsLayout layout(moe_op_t op, int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const bool layer = op == MOE_OP_FORWARD || op == MOE_OP_FORWARD_MX6 || op == MOE_OP_FORWARD_BLOCK;
  const bool tiles = n > 0 && moe::ffn_uses_tiles((int)n, E);
  WsLayout l;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off = align_up(off + bytes);
  };
  // routing results and the permutation (the layer calls)
  take(l.ids, layer ? n * 4 : 0);
  take(l.w, layer ? n * 4 : 0);
  take(l.counts, layer ? (size_t)E * 4 : 0);
  take(l.offsets, layer ? (size_t)(E + 1) * 4 : 0);
  take(l.sorted, layer ? n * 4 : 0);
  // router partial logits or per-block expert histograms; the standalone
  // permutation's histograms (only above one workgroup's slots)
  size_t scratch = 0;
  if (op == MOE_OP_ROUTE || layer) scratch = moe::route_scratch_bytes(T, E);
  if (op == MOE_OP_PERMUTE) scratch = n > 1024 ? (size_t)((T + 31) / 32) * E * 4 : 0;
  take(l.scratch, scratch);
  // the gate/up output h [T*k, 2880] bf16 in expert-sorted order
  take(l.h, (layer || op == MOE_OP_EXPERT_FFN) ? n * (size_t)moe::kI * 2 : 0);
  // per-slot fp32 expert outputs: the layer stores them and sums a token's k
  // rows in a second pass instead of atomically adding into out
  take(l.y, layer ? n * (size_t)moe::kH * 4 : 0);
  // moe_forward_mx6, tiled schedule: x and h as two-piece MX FP6 records
  const bool mx6 = op == MOE_OP_FORWARD_MX6 && tiles;
  take(l.xrec, mx6 ? (size_t)T * moe::kRowRecBytes : 0);
  take(l.hrec, mx6 ? n * (size_t)moe::kRowRecBytes : 0);
  // moe_forward_block: the normed bf16 input of the expert GEMMs, and the
  // tokens' inverse RMS from the norm kernel (not when the router forms it,
  // block_norm_folded)
  const bool block = op == MOE_OP_FORWARD_BLOCK;
  take(l.xnorm, block ? (size_t)T * moe::kH * 2 : 0);
  take(l.inv, block && !block_norm_folded(T, E, k) ? (size_t)T * 4 : 0);
  l.total = off < kAlign ? kAlign : off;
  return l;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Current device must be gfx950; the answer is cached per device.
std::atomic<int> g_arch_state[64];  // 0 unknown, 1 gfx950, 2 other

moe_status_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERROR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERROR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERROR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MOE_SUCCESS : MOE_ERROR_UNSUPPORTED;
}

bool debug_sync() {
  static const int on = [] {
    const char* v = std::getenv("MOE_DEBUG_SYNC");
    return (v && v[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

moe_status_t after_launch(hipError_t err, hipStream_t s) {
  if (err != hipSuccess) return MOE_ERROR_HIP;
  if (debug_sync()) {
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERROR_HIP;
    if (hipGetLastError() != hipSuccess) return MOE_ERROR_HIP;
  }
  return MOE_SUCCESS;
}

#define MOE_TRY(expr)                       \
  do {                                      \
    moe_status_t st_ = (expr);              \
    if (st_ != MOE_SUCCESS) return st_;     \
  } while (0)

// A packed weight tensor: filled by moe_pack_weights, with the call's expert
// count and rows per expert.
moe_status_t check_packed(const moe_packed_weight_t* w, int E, int N) {
  if (!w) return MOE_ERROR_INVALID_VALUE;
  if (w->tag != MOE_PACKED_TAG || w->E != E || w->N != N) return MOE_ERROR_LAYOUT;
  if (!w->codes || !w->scales) return MOE_ERROR_LAYOUT;
  if (!aligned(w->codes, 16) || !aligned(w->scales, 4)) return MOE_ERROR_MISALIGNED;
  return MOE_SUCCESS;
}

moe_status_t check_weights(const moe_packed_weight_t* w13, const uint16_t* b13,
                           const moe_packed_weight_t* w2, const uint16_t* b2, int E) {
  if (!b13 || !b2) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_packed(w13, E, moe::kN13));
  MOE_TRY(check_packed(w2, E, moe::kH));
  if (!aligned(b13, 8) || !aligned(b2, 8)) return MOE_ERROR_MISALIGNED;
  return MOE_SUCCESS;
}

moe_status_t check_ws(void* ws, size_t ws_bytes, moe_op_t op, int T, int E, int k) {
  if (!ws || !aligned(ws, kAlign)) return MOE_ERROR_WORKSPACE;
  if (ws_bytes < layout(op, T, E, k).total) return MOE_ERROR_WORKSPACE;
  return MOE_SUCCESS;
}

FfnArgs ffn_args(const uint16_t* act, const int32_t* offsets, const int32_t* sorted_rows,
                 const moe_packed_weight_t* w, const uint16_t* bias, int N, int E, int k,
                 int gather) {
  FfnArgs a;
  std::memset(&a, 0, sizeof a);
  a.act = act;
  a.offsets = offsets;
  a.sorted_rows = sorted_rows;
  a.codes = w->codes;
  a.scales = w->scales;
  a.bias = bias;
  a.N = N;
  a.E = E;
  a.k = k;
  a.gather = gather;
  return a;
}

}  // namespace

extern "C" {

size_t moe_workspace_size_op(moe_op_t op, int T, int E, int k) {
  if (!sizes_ok(T, E, k) || !op_ok(op)) return 0;
  return layout(op, T, E, k).total;
}

size_t moe_workspace_size(int T, int E, int k) {
  if (!sizes_ok(T, E, k)) return 0;
  size_t m = 0;
  for (int op = MOE_OP_ROUTE; op <= MOE_OP_FORWARD_BLOCK; ++op) {
    const size_t b = layout(static_cast<moe_op_t>(op), T, E, k).total;
    m = b > m ? b : m;
  }
  return m;
}

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_SUCCESS: return "MOE_SUCCESS";
    case MOE_ERROR_INVALID_VALUE: return "MOE_ERROR_INVALID_VALUE: null pointer or size out of range";
    case MOE_ERROR_MISALIGNED: return "MOE_ERROR_MISALIGNED: pointer lacks the required alignment";
    case MOE_ERROR_WORKSPACE: return "MOE_ERROR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERROR_UNSUPPORTED: return "MOE_ERROR_UNSUPPORTED: current device is not gfx950";
    case MOE_ERROR_HIP: return "MOE_ERROR_HIP: a HIP runtime call or kernel launch failed";
    case MOE_ERROR_LAYOUT:
      return "MOE_ERROR_LAYOUT: weight descriptor not filled by moe_pack_weights or of other E / N";
    case MOE_ERROR_RANGE:
      return "MOE_ERROR_RANGE: weight scale spread beyond what the FP6-piece path is accurate for; use moe_forward";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_route(const uint16_t* x, const float* Wr, const float* br, int T, int E, int k,
                       int32_t* topk_ids, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !Wr || !br || !topk_ids || !topk_w) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(br, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(logits, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_ws(ws, ws_bytes, MOE_OP_ROUTE, T, E, k));
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scratch =
      reinterpret_cast<float*>(static_cast<char*>(ws) + layout(MOE_OP_ROUTE, T, E, k).scratch);
  return after_launch(moe::launch_route(x, Wr, br, T, E, k, topk_ids, topk_w, logits, scratch, nullptr,
                                        nullptr, nullptr, nullptr, s), s);
}

moe_status_t moe_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N,
                              uint8_t* packed_codes, uint8_t* packed_scales,
                              moe_packed_weight_t* desc, void* stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || N < 64 || N > 65536 || N % 64 != 0)
    return MOE_ERROR_INVALID_VALUE;
  if (!codes || !scales || !packed_codes || !packed_scales || !desc) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(codes, 16) || !aligned(packed_codes, 16) || !aligned(packed_scales, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(after_launch(moe::launch_pack(codes, scales, E, N, packed_codes, packed_scales, s), s));
  // the tensor's scale spread, for the FP6-piece path's accuracy limit
  int32_t* lohi_dev = nullptr;
  if (hipMalloc(&lohi_dev, sizeof(int32_t) * 2 * E) != hipSuccess) return MOE_ERROR_HIP;
  std::vector<int32_t> lohi(2 * (size_t)E);
  hipError_t err = moe::launch_scale_range(scales, E, N, lohi_dev, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(lohi.data(), lohi_dev, sizeof(int32_t) * 2 * E, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  hipFree(lohi_dev);
  if (err != hipSuccess) return MOE_ERROR_HIP;
  uint32_t spread = 0;
  for (int e = 0; e < E; ++e)
    if (lohi[2 * e + 1] >= lohi[2 * e]) spread = std::max(spread, (uint32_t)(lohi[2 * e + 1] - lohi[2 * e]));
  desc->codes = packed_codes;
  desc->scales = packed_scales;
  desc->E = E;
  desc->N = N;
  desc->tag = MOE_PACKED_TAG;
  desc->scale_spread = spread;
  return MOE_SUCCESS;
}

moe_status_t moe_permute(const int32_t* topk_ids, int T, int E, int k, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_rows, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!topk_ids || !counts || !offsets || !sorted_rows) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_rows, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_ws(ws, ws_bytes, MOE_OP_PERMUTE, T, E, k));
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* hist =
      reinterpret_cast<int32_t*>(static_cast<char*>(ws) + layout(MOE_OP_PERMUTE, T, E, k).scratch);
  return after_launch(moe::launch_permute(topk_ids, T * k, E, k, counts, offsets, sorted_rows, hist, s),
                      s);
}

moe_status_t moe_expert_ffn(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_rows,
                            const moe_packed_weight_t* w13, const uint16_t* b13,
                            const moe_packed_weight_t* w2, const uint16_t* b2, int T, int E, int k,
                            float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !offsets || !sorted_rows || !y) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_weights(w13, b13, w2, b2, E));
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(offsets, 4) || !aligned(sorted_rows, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_ws(ws, ws_bytes, MOE_OP_EXPERT_FFN, T, E, k));
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const WsLayout l = layout(MOE_OP_EXPERT_FFN, T, E, k);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + l.h);
  const int n = T * k;
  FfnArgs a13 = ffn_args(x, offsets, sorted_rows, w13, b13, moe::kN13, E, k, 1);
  a13.h_out = h;
  MOE_TRY(after_launch(moe::launch_ffn(a13, moe::EPI_SWIGLU, n, s), s));
  FfnArgs a2 = ffn_args(h, offsets, sorted_rows, w2, b2, moe::kH, E, k, 0);
  a2.y_out = y;
  return after_launch(moe::launch_ffn(a2, moe::EPI_STORE_Y, n, s), s);
}

moe_status_t moe_gate_up(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_rows,
                         const moe_packed_weight_t* w13, const uint16_t* b13, int T, int E, int k,
                         uint16_t* h, void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !offsets || !sorted_rows || !b13 || !h) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_packed(w13, E, moe::kN13));
  if (!aligned(x, 16) || !aligned(h, 16) || !aligned(b13, 8) || !aligned(offsets, 4) ||
      !aligned(sorted_rows, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  FfnArgs a = ffn_args(x, offsets, sorted_rows, w13, b13, moe::kN13, E, k, 1);
  a.h_out = h;
  return after_launch(moe::launch_ffn(a, moe::EPI_SWIGLU, T * k, s), s);
}

moe_status_t moe_gate_up_mx6(const uint8_t* x_records, const int32_t* offsets,
                             const int32_t* sorted_rows, const moe_packed_weight_t* w13,
                             const uint16_t* b13, int T, int E, int k, uint16_t* h, void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x_records || !offsets || !sorted_rows || !b13 || !h) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_packed(w13, E, moe::kN13));
  if (w13->scale_spread > MOE_MX6_MAX_SCALE_SPREAD) return MOE_ERROR_RANGE;
  if (!aligned(x_records, 16) || !aligned(h, 16) || !aligned(b13, 8) || !aligned(offsets, 4) ||
      !aligned(sorted_rows, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  FfnArgs a = ffn_args(nullptr, offsets, sorted_rows, w13, b13, moe::kN13, E, k, 1);
  a.act6 = x_records;
  a.h_out = h;
  return after_launch(moe::launch_ffn(a, moe::EPI_SWIGLU, T * k, s), s);
}

moe_status_t moe_down_accumulate(const uint16_t* h, const int32_t* offsets,
                                 const int32_t* sorted_rows, const float* topk_w,
                                 const moe_packed_weight_t* w2, const uint16_t* b2, int T, int E,
                                 int k, float* out, void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!h || !offsets || !sorted_rows || !topk_w || !b2 || !out) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_packed(w2, E, moe::kH));
  if (!aligned(h, 16) || !aligned(out, 16) || !aligned(b2, 8) || !aligned(offsets, 4) ||
      !aligned(sorted_rows, 4) || !aligned(topk_w, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  FfnArgs a = ffn_args(h, offsets, sorted_rows, w2, b2, moe::kH, E, k, 0);
  a.topk_w = topk_w;
  a.out = out;
  return after_launch(moe::launch_ffn(a, moe::EPI_COMBINE, T * k, s), s);
}

moe_status_t moe_combine(const float* y, const float* topk_w, int T, int k, float* out,
                         void* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || (long long)T * k > MOE_MAX_ROUTED)
    return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!y || !topk_w || !out) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_w, 4)) return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(moe::launch_combine(y, topk_w, T, k, nullptr, out, s), s);
}

}  // extern "C"

namespace {

struct LayerWeights {
  const moe_packed_weight_t* w13;
  const uint16_t* b13;
  const moe_packed_weight_t* w2;
  const uint16_t* b2;
};

// The decoder block around the layer: the router's norm (scale, eps, the
// inverse RMS or where the router writes the normed rows) and the expert
// GEMMs' input, the normed bf16 rows `t`.
struct BlockNorm {
  moe::RouteNorm rn;
  const uint16_t* t;
};

// The layer on x; with `resid` (bf16 [T, 2880]) the output is resid + layer;
// with `blk` the layer of the decoder block on RMSNorm(x).
// Arguments are validated by the caller; `l` is the caller's workspace layout.
moe_status_t forward_launch(const uint16_t* x, const float* Wr, const float* br,
                            const LayerWeights& lw, int T, int E, int k, float* out, char* base,
                            const WsLayout& l, hipStream_t s, bool mx6, const uint16_t* resid,
                            const BlockNorm* blk = nullptr) {
  int32_t* ids = reinterpret_cast<int32_t*>(base + l.ids);
  float* w = reinterpret_cast<float*>(base + l.w);
  int32_t* counts = reinterpret_cast<int32_t*>(base + l.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + l.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + l.sorted);
  float* scratch = reinterpret_cast<float*>(base + l.scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + l.h);
  const int n = T * k;
  // router + top-k + softmax + expert permutation
  const bool tiles = moe::ffn_uses_tiles(n, E);
  // The weight-streaming schedule needs no permutation arrays: its waves find
  // their slots in the routing ids.
  MOE_TRY(after_launch(moe::launch_route(x, Wr, br, T, E, k, ids, w, nullptr, scratch,
                                         tiles ? counts : nullptr, offsets, sorted,
                                         blk ? &blk->rn : nullptr, s), s));
  FfnArgs a13 = ffn_args(blk ? blk->t : x, offsets, sorted, lw.w13, lw.b13, moe::kN13, E, k, 1);
  a13.h_out = h;
  if (!tiles) {
    a13.ids = ids;
    a13.n_slots = n;
  } else if (mx6) {
    // x and h as two-piece MX FP6 records: x by the encoder, h by the
    // gate/up epilogue, for the block-scaled matrix cores of both GEMMs
    uint8_t* xrec = reinterpret_cast<uint8_t*>(base + l.xrec);
    MOE_TRY(after_launch(moe::launch_mx6_encode(x, T, xrec, s), s));
    a13.act6 = xrec;
    a13.h6_out = reinterpret_cast<uint8_t*>(base + l.hrec);
  }
  MOE_TRY(after_launch(moe::launch_ffn(a13, moe::EPI_SWIGLU, n, s), s));
  FfnArgs a2 = ffn_args(h, offsets, sorted, lw.w2, lw.b2, moe::kH, E, k, 0);
  if (!tiles) {
    a2.ids = ids;
    a2.n_slots = n;
  }
  // Store y per slot, then out[t] = resid[t] + sum_j w[t, j] y[t*k + j] in a
  // fixed order. Adding w * y into out atomically from the down epilogue
  // instead costs more than the extra pass: the T*k*2880 fp32 atomics are
  // served far from the CUs at a fraction of the store rate.
  float* y = reinterpret_cast<float*>(base + l.y);
  a2.y_out = y;
  if (tiles && mx6) a2.act6 = reinterpret_cast<uint8_t*>(base + l.hrec);   // written by the gate/up epilogue
  MOE_TRY(after_launch(moe::launch_ffn(a2, moe::EPI_STORE_Y, n, s), s));
  return after_launch(moe::launch_combine(y, w, T, k, resid, out, s), s);
}

moe_status_t forward_impl(const uint16_t* x, const float* Wr, const float* br,
                          const LayerWeights& lw, int T, int E, int k, float* out, void* ws,
                          size_t ws_bytes, void* stream, bool mx6) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !Wr || !br || !out) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_weights(lw.w13, lw.b13, lw.w2, lw.b2, E));
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(out, 16) || !aligned(br, 4))
    return MOE_ERROR_MISALIGNED;
  const moe_op_t op = mx6 ? MOE_OP_FORWARD_MX6 : MOE_OP_FORWARD;
  // the FP6-piece path (tiled schedule only) holds the bar up to a bounded
  // scale spread
  if (mx6 && moe::ffn_uses_tiles(T * k, E) &&
      (lw.w13->scale_spread > MOE_MX6_MAX_SCALE_SPREAD || lw.w2->scale_spread > MOE_MX6_MAX_SCALE_SPREAD))
    return MOE_ERROR_RANGE;
  MOE_TRY(check_ws(ws, ws_bytes, op, T, E, k));
  MOE_TRY(check_device());
  return forward_launch(x, Wr, br, lw, T, E, k, out, static_cast<char*>(ws), layout(op, T, E, k),
                        static_cast<hipStream_t>(stream), mx6, nullptr);
}

}  // namespace

extern "C" {

moe_status_t moe_forward(const uint16_t* x, const float* Wr, const float* br,
                         const moe_packed_weight_t* w13, const uint16_t* b13,
                         const moe_packed_weight_t* w2, const uint16_t* b2, int T, int E, int k,
                         float* out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(x, Wr, br, LayerWeights{w13, b13, w2, b2}, T, E, k, out, ws, ws_bytes, stream,
                      false);
}

moe_status_t moe_forward_mx6(const uint16_t* x, const float* Wr, const float* br,
                             const moe_packed_weight_t* w13, const uint16_t* b13,
                             const moe_packed_weight_t* w2, const uint16_t* b2, int T, int E, int k,
                             float* out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(x, Wr, br, LayerWeights{w13, b13, w2, b2}, T, E, k, out, ws, ws_bytes, stream,
                      true);
}

moe_status_t moe_rmsnorm(const uint16_t* x, const float* scale, float eps, int T, uint16_t* t,
                         void* stream) {
  if (T < 0 || T > MOE_MAX_ROUTED || !(eps >= 0.f) || !(eps < 1e30f)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !scale || !t) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(x, 16) || !aligned(t, 16) || !aligned(scale, 16)) return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(moe::launch_rmsnorm(x, scale, eps, T, t, nullptr, s), s);
}

moe_status_t moe_forward_block(const uint16_t* x, const float* norm_scale, float norm_eps,
                               const float* Wr, const float* br, const moe_packed_weight_t* w13,
                               const uint16_t* b13, const moe_packed_weight_t* w2,
                               const uint16_t* b2, int T, int E, int k, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!sizes_ok(T, E, k) || !(norm_eps >= 0.f) || !(norm_eps < 1e30f)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !norm_scale || !Wr || !br || !out) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_weights(w13, b13, w2, b2, E));
  if (!aligned(x, 16) || !aligned(norm_scale, 16) || !aligned(Wr, 16) || !aligned(out, 16) ||
      !aligned(br, 4))
    return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_ws(ws, ws_bytes, MOE_OP_FORWARD_BLOCK, T, E, k));
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const WsLayout l = layout(MOE_OP_FORWARD_BLOCK, T, E, k);
  char* base = static_cast<char*>(ws);
  uint16_t* t = reinterpret_cast<uint16_t*>(base + l.xnorm);
  BlockNorm blk;
  blk.rn = moe::RouteNorm{norm_scale, norm_eps, nullptr, false, t};
  blk.t = t;
  if (!block_norm_folded(T, E, k)) {
    // the norm kernel writes the rows and the inverse RMS the router takes
    float* inv = reinterpret_cast<float*>(base + l.inv);
    MOE_TRY(after_launch(moe::launch_rmsnorm(x, norm_scale, norm_eps, T, t, inv, s), s));
    blk.rn = moe::RouteNorm{norm_scale, norm_eps, inv, true, nullptr};
  }
  return forward_launch(x, Wr, br, LayerWeights{w13, b13, w2, b2}, T, E, k, out, base, l, s, false,
                        x, &blk);
}

}  // extern "C"

namespace {

// The workspace of moe_forward_noalloc: one copy per GPU, in device memory for
// the life of the process. In host code `noalloc_scratch` only names the
// symbol; its device address on the current GPU comes from
// hipGetSymbolAddress and is kept per device.
static __device__ __align__(256) unsigned char noalloc_scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array (looked up once per
// device, with that device current).
moe_status_t noalloc_scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERROR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERROR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return MOE_ERROR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_SUCCESS;
}

}  // namespace

extern "C" {

moe_status_t moe_forward_noalloc(const uint16_t* x, const float* Wr, const float* br,
                                 const moe_packed_weight_t* w13, const uint16_t* b13,
                                 const moe_packed_weight_t* w2, const uint16_t* b2, int T, int E,
                                 int k, float* out, void* stream) {
  if (!sizes_ok(T, E, k)) return MOE_ERROR_INVALID_VALUE;
  if (T == 0) return MOE_SUCCESS;
  if (!x || !Wr || !br || !out) return MOE_ERROR_INVALID_VALUE;
  MOE_TRY(check_weights(w13, b13, w2, b2, E));
  if (!aligned(x, 16) || !aligned(Wr, 16) || !aligned(out, 16) || !aligned(br, 4))
    return MOE_ERROR_MISALIGNED;
  const WsLayout l = layout(MOE_OP_FORWARD, T, E, k);
  if (l.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERROR_WORKSPACE;
  MOE_TRY(check_device());
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch_ptr(&ws));
  return forward_launch(x, Wr, br, LayerWeights{w13, b13, w2, b2}, T, E, k, out,
                        static_cast<char*>(ws), l, static_cast<hipStream_t>(stream), false, nullptr);
}

moe_status_t moe_encode_mx6(const uint16_t* x, int rows, uint8_t* records, void* stream) {
  if (rows < 0 || rows > MOE_MAX_ROUTED) return MOE_ERROR_INVALID_VALUE;
  if (rows == 0) return MOE_SUCCESS;
  if (!x || !records) return MOE_ERROR_INVALID_VALUE;
  if (!aligned(x, 16) || !aligned(records, 16)) return MOE_ERROR_MISALIGNED;
  MOE_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(moe::launch_mx6_encode(x, rows, records, s), s);
}

}  // extern "C"
