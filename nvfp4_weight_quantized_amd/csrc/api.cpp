// C ABI of libmoe_nvfp4: host-side validation, workspace carving and launch sequencing.
// Every entry point validates on the host before enqueuing anything (loud failure instead of
// silently wrong output -- the failure mode the DGX Spark pages keep warning about), never
// synchronises and never allocates.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <functional>

#include "common.h"

namespace {

using moe::GemmBank;
using moe::GemmProblem;

constexpr size_t kAlign = 256;

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// gfx950 check, cached per device (the value never changes for a device).
int g_arch_ok[64];  // 0 unknown, 1 ok, 2 not gfx950

moe_status_t check_arch(const char* arch) {
  if (arch) return std::strncmp(arch, "gfx950", 6) == 0 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev >= 0 && dev < 64 && g_arch_ok[dev]) return g_arch_ok[dev] == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev] = ok ? 1 : 2;
  return ok ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

// The kernels move weights, activations and outputs with 16-byte vector accesses.
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool valid_bank(const moe_nvfp4_experts_t& b, int32_t H, int32_t expected_experts) {
  if (b.num_experts != expected_experts || b.hidden != H) return false;
  if (b.inter <= 0 || b.inter % 128 != 0) return false;
  if (b.format != MOE_WEIGHT_NVFP4 && b.format != MOE_WEIGHT_MXFP4 && b.format != MOE_WEIGHT_MXFP4_A4) return false;
  if (!(b.w13 && b.w13_scale && b.w2 && b.w2_scale)) return false;
  if (b.format == MOE_WEIGHT_NVFP4 && !(b.w13_gscale && b.w2_gscale)) return false;
  return al16(b.w13) && al16(b.w13_scale) && al16(b.w2) && al16(b.w2_scale);
}

// Banks the W4A16 kernels read (the W4A4 tile layout is for the W4A4 entry points only).
bool w4a16_format(int32_t f) { return f == MOE_WEIGHT_NVFP4 || f == MOE_WEIGHT_MXFP4; }

// The LDS-staging kernels address activation rows with 32-bit byte offsets.
constexpr int64_t kMaxActivationBytes = (int64_t)1 << 32;

bool valid_route_dims(int32_t T, int32_t H, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return false;
  if (H <= 0 || H % 128 != 0) return false;
  if ((int64_t)T * H * 2 >= kMaxActivationBytes) return false;
  return (int64_t)T * k < (int64_t)0x7FFFFFFF;
}

GemmBank bank_w13(const moe_nvfp4_experts_t& b) { return GemmBank{b.w13, b.w13_scale, b.w13_gscale, 2, b.format}; }
GemmBank bank_w2(const moe_nvfp4_experts_t& b) { return GemmBank{b.w2, b.w2_scale, b.w2_gscale, 1, b.format}; }

struct ForwardLayout {
  size_t logits, ids, w, counts, offsets, sorted_slot, slot_to_row, block_hist, x16, row_shift, h, h_shared, y,
      ctr, xa, tiles, hshift, rpart;
  size_t total;
};

// a4: the NVFP4 W4A4 forward, which also holds x's 4-bit values as bf16 rows (xa) and keeps h
// row-major.
ForwardLayout forward_layout(int32_t T, int32_t H, int32_t I, int32_t I_shared, int32_t E, int32_t k,
                             bool a4 = false) {
  ForwardLayout L{};
  const size_t S = (size_t)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.logits = take((size_t)T * E * 4);
  L.ids = take(S * 4);
  L.w = take(S * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.sorted_slot = take(S * 4);
  L.slot_to_row = take(S * 4);
  L.block_hist = take(S > (size_t)moe::kPermuteChunk ? (size_t)moe::permute_blocks((int64_t)S) * E * 4 : 0);
  // x as fp16 rows with per-row power-of-two shifts (the NVFP4 128-row gate/up path)
  L.x16 = take((size_t)T * H * 2);
  L.row_shift = take((size_t)T * 4);
  // h rows (row-major, shared-expert rows right after the routed ones), or the same bytes reused
  // for h in the fragment-tiled layout of the 128-row GEMM path (one 128-row block per m-tile),
  // which the forward takes exactly when its gate/up problem runs on 128-row tiles
  const size_t h_rows_bytes = align_up(S * I * 2) + align_up((size_t)T * I_shared * 2);
  GemmProblem gu{};
  gu.G = E;
  gu.M = (int32_t)std::min<size_t>(S, 0x7FFFFFFF);
  gu.has_extra = I_shared == I ? 1 : 0;
  gu.M_extra = I_shared == I ? T : 0;
  const bool tiled = (I_shared == 0 || I_shared == I) && moe::grouped_gemm_uses_tall_tiles(gu);
  const size_t mt_bound = std::min<size_t>((size_t)E, S) + S / 128 + ((size_t)T + 127) / 128;
  const size_t h_tiled_bytes = tiled ? mt_bound * 128 * (size_t)I * 2 : 0;
  L.h = take(std::max(h_rows_bytes, h_tiled_bytes));
  L.h_shared = L.h + align_up(S * I * 2);
  L.y = take((S + (I_shared > 0 ? (size_t)T : 0)) * H * 2);
  // hand-off counters of the fused decode launch (few tokens only)
  L.ctr = take(T <= moe::kFusedDecodeMaxTokens && S <= (size_t)moe::kFusedDecodeMaxSlots
                   ? (size_t)moe::fused_decode_counter_words(T, k, E, I_shared > 0) * 4
                   : 0);
  L.xa = take(a4 ? (size_t)T * H * 2 : 0);
  // tile counters of the gate/up and down launches (cleared by the router launch of the forward)
  L.tiles = take(2 * moe::kTileCounterWords * 4);
  // the power of two of each h row when h is held as fp16 (tiled h only)
  L.hshift = take(tiled && !a4 ? (S + (size_t)T) * 4 : 0);
  // partial router sums of a split router GEMM beyond the first (which goes to the logits)
  L.rpart = take((size_t)(moe::router_k_splits(T, H, E, k) - 1) * T * E * 4);
  L.total = off;
  return L;
}

// W4A4 forward: routing buffers as above, then the 4-bit activations (x, then h), h in bf16
// (row-major; the shared expert's rows after the routed ones) and the expert outputs y.
struct ForwardLayoutA4 {
  size_t logits, ids, w, counts, offsets, sorted_slot, slot_to_row, block_hist;
  size_t xq, xs, h, hq, hs, y;
  size_t total;
};

ForwardLayoutA4 forward_layout_a4(int32_t T, int32_t H, int32_t I, int32_t I_shared, int32_t E, int32_t k) {
  ForwardLayoutA4 L{};
  const size_t S = (size_t)T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.logits = take((size_t)T * E * 4);
  L.ids = take(S * 4);
  L.w = take(S * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.sorted_slot = take(S * 4);
  L.slot_to_row = take(S * 4);
  L.block_hist = take(S > (size_t)moe::kPermuteChunk ? (size_t)moe::permute_blocks((int64_t)S) * E * 4 : 0);
  L.xq = take((size_t)T * H / 2);
  L.xs = take((size_t)T * H / 32);
  const size_t h_elems = S * I + (size_t)T * I_shared;   // both parts are multiples of 128 elements
  L.h = take(h_elems * 2);
  L.hq = take(h_elems / 2);
  L.hs = take(h_elems / 32);
  L.y = take((S + (I_shared > 0 ? (size_t)T : 0)) * H * 2);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE (gfx950 required)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_route(const uint16_t* x, const uint16_t* w_router, const float* router_bias, int32_t T,
                       int32_t H, int32_t E, int32_t k, uint32_t flags, float* logits, int32_t* topk_ids,
                       float* topk_w, void* stream) {
  const bool given = (flags & MOE_ROUTE_LOGITS_GIVEN) != 0;
  if ((flags & ~MOE_ROUTE_LOGITS_GIVEN) != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return MOE_ERR_INVALID_ARGUMENT;
  if (!given && !valid_route_dims(T, H, E, k)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!given && (!x || !w_router || !al16(x) || !al16(w_router))) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_route(x, w_router, router_bias, T, H, E, k, given, logits, topk_ids, topk_w,
                           static_cast<hipStream_t>(stream));
}

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const int64_t S = (int64_t)T * k;
  if (S <= moe::kPermuteChunk) return 0;
  return align_up((size_t)moe::permute_blocks(S) * E * 4);
}

moe_status_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* sorted_slot, int32_t* slot_to_row, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || (int64_t)T * k >= (int64_t)0x7FFFFFFF)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!topk_ids || !sorted_slot || !slot_to_row)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe_permute_workspace_size(T, k, E);
  if (workspace_bytes < need || (need > 0 && !workspace)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (moe_status_t st = check_arch(nullptr)) return st;
  // T == 0 still defines counts = 0 and offsets = 0 (S = 0 runs the single-workgroup path)
  return moe::launch_permute(topk_ids, T, k, E, expert_counts, expert_offsets, sorted_slot, slot_to_row,
                             static_cast<int32_t*>(workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// A usable activation dequant global scale: finite and positive (a zero would silently zero every
// expert).
bool valid_act_gscale(float d) { return std::isfinite(d) && d > 0.f; }

// moe_nvfp4_grouped_gemm, with the activation global scale of NVFP4 W4A4 rows (0: W4A16).
moe_status_t grouped_gemm_entry(int32_t stage, const moe_nvfp4_experts_t* w, const uint16_t* a, float a_gscale,
                                const int32_t* row_index, int32_t row_divisor, const int32_t* expert_offsets,
                                int32_t M_total, uint16_t* out, void* stream) {
  if (!w || (stage != MOE_GEMM_GATE_UP && stage != MOE_GEMM_DOWN)) return MOE_ERR_INVALID_ARGUMENT;
  if (w->num_experts < 1 || w->num_experts > 1024) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_bank(*w, w->hidden, w->num_experts) || !w4a16_format(w->format) || w->hidden <= 0 ||
      w->hidden % 128 != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M_total < 0 || row_divisor < 1) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t K_ = stage == MOE_GEMM_GATE_UP ? w->hidden : w->inter;
  if ((int64_t)M_total * K_ * 2 >= kMaxActivationBytes) return MOE_ERR_INVALID_ARGUMENT;
  if (stage == MOE_GEMM_DOWN && row_index) return MOE_ERR_INVALID_ARGUMENT;
  if (M_total == 0) return MOE_OK;
  if (!a || !expert_offsets || !out || !al16(a) || !al16(out)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  GemmProblem p{};
  p.stage = stage;
  const bool gu = stage == MOE_GEMM_GATE_UP;
  p.N = gu ? w->inter : w->hidden;
  p.K = gu ? w->hidden : w->inter;
  p.bank = gu ? bank_w13(*w) : bank_w2(*w);
  p.offsets = expert_offsets;
  p.G = w->num_experts;
  p.M = M_total;
  p.a = a;
  p.row_index = row_index;
  p.row_divisor = row_divisor;
  p.out = out;
  p.has_extra = 0;
  p.a_gscale = a_gscale;
  return moe::launch_grouped_gemm(p, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

moe_status_t moe_nvfp4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w, const uint16_t* a,
                                    const int32_t* row_index, int32_t row_divisor, const int32_t* expert_offsets,
                                    int32_t M_total, uint16_t* out, void* stream) {
  return grouped_gemm_entry(stage, w, a, 0.f, row_index, row_divisor, expert_offsets, M_total, out, stream);
}

moe_status_t moe_nvfp4_w4a4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w, const uint16_t* a,
                                         float act_gscale, const int32_t* row_index, int32_t row_divisor,
                                         const int32_t* expert_offsets, int32_t M_total, uint16_t* out,
                                         void* stream) {
  if (!valid_act_gscale(act_gscale) || !w || w->format != MOE_WEIGHT_NVFP4) return MOE_ERR_INVALID_ARGUMENT;
  return grouped_gemm_entry(stage, w, a, act_gscale, row_index, row_divisor, expert_offsets, M_total, out, stream);
}

moe_status_t moe_combine(const uint16_t* y_rows, const int32_t* slot_to_row, const float* topk_w,
                         const uint16_t* y_shared, int32_t T, int32_t k, int32_t H, uint16_t* out, void* stream) {
  if (T < 0 || k < 1 || k > 1024 || H <= 0 || H % 8 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!y_rows || !slot_to_row || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(y_rows) || !al16(out) || (y_shared && !al16(y_shared))) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_combine(y_rows, slot_to_row, topk_w, y_shared, T, k, H, out, static_cast<hipStream_t>(stream));
}

size_t moe_nvfp4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared, int32_t E, int32_t k) {
  if (T < 0 || H <= 0 || I <= 0 || I_shared < 0 || E < 1 || k < 1) return 0;
  return forward_layout(T, H, I, I_shared, E, k).total;
}

}  // extern "C"

namespace {

// Shapes, pointers and formats of a layer for T tokens (every check of a forward pass but the
// workspace size and the device).
moe_status_t validate_layer(const moe_nvfp4_layer_t* layer, int32_t T) {
  if (!layer) return MOE_ERR_INVALID_ARGUMENT;
  const int32_t H = layer->hidden, E = layer->num_experts, k = layer->top_k;
  if (!valid_route_dims(T, H, E, k)) return MOE_ERR_INVALID_ARGUMENT;
  if (!layer->w_router || !al16(layer->w_router)) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_bank(layer->routed, H, E)) return MOE_ERR_INVALID_ARGUMENT;
  const bool has_shared = layer->shared.num_experts != 0;
  if (has_shared && !valid_bank(layer->shared, H, 1)) return MOE_ERR_INVALID_ARGUMENT;
  if (has_shared && layer->shared.format != layer->routed.format) return MOE_ERR_INVALID_ARGUMENT;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  if (((int64_t)T * k + T) * std::max(I, Is) * 2 >= kMaxActivationBytes) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                  const char* gfx_arch) {
  if (moe_status_t st = validate_layer(layer, T)) return st;
  if (!w4a16_format(layer->routed.format)) return MOE_ERR_INVALID_ARGUMENT;
  const bool has_shared = layer->shared.num_experts != 0;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  if (T > 0 && workspace_bytes < moe_nvfp4_forward_workspace_size(T, layer->hidden, I, Is, layer->num_experts,
                                                                   layer->top_k))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return check_arch(gfx_arch);
}

moe_status_t moe_mxfp4_w4a4_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                             const char* gfx_arch) {
  if (moe_status_t st = validate_layer(layer, T)) return st;
  if (layer->routed.format != MOE_WEIGHT_MXFP4_A4) return MOE_ERR_INVALID_ARGUMENT;
  const bool has_shared = layer->shared.num_experts != 0;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  if (T > 0 && workspace_bytes < moe_mxfp4_w4a4_forward_workspace_size(T, layer->hidden, I, Is, layer->num_experts,
                                                                        layer->top_k))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return check_arch(gfx_arch);
}

namespace {

// S1-S3 of a forward pass: router logits, top-k, permutation (stage event 1 after S1; the caller
// records event 2).
// rpart: room for the partial sums of a split router GEMM (moe::router_k_splits - 1 arrays of
// [T][E] floats), or NULL for one pass.
moe_status_t run_routing(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T, float* logits, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* sorted_slot, int32_t* slot_to_row,
                         int32_t* block_hist, const std::function<moe_status_t(int)>& mark, hipStream_t stream,
                         int32_t* zero = nullptr, int32_t n_zero = 0, float* rpart = nullptr) {
  const int32_t H = layer->hidden, E = layer->num_experts, k = layer->top_k;
  const int32_t splits = rpart ? moe::router_k_splits(T, H, E, k) : 1;
  moe_status_t st = moe::launch_router_logits(x, layer->w_router, layer->router_bias, T, H, E, logits, stream, zero,
                                              n_zero, rpart, splits);
  if (st || (st = mark(1))) return st;
  if ((int64_t)T * k <= moe::kPermuteChunk) {
    // few tokens: top-k and permutation together in one workgroup
    st = moe::launch_topk_permute_small(logits, T, E, k, ids, w, counts, offsets, sorted_slot, slot_to_row, stream);
  } else {
    if (splits > 1)
      st = moe::launch_topk_sum(logits, rpart, splits, layer->router_bias, T, E, k, ids, w, stream);
    else
      st = moe::launch_route(nullptr, nullptr, nullptr, T, H, E, k, true, logits, ids, w, stream);
    if (st) return st;
    st = moe::launch_permute(ids, T, k, E, counts, offsets, sorted_slot, slot_to_row, block_hist, stream);
  }
  return st;
}

}  // namespace

namespace {

// The W4A16 forward (a4 == nullptr) or the NVFP4 W4A4 forward (a4 = {d_x, d_h}: the activation
// dequant global scales of the gate/up and down inputs).  Arguments validated by the caller.
moe_status_t forward_impl(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T, uint16_t* out,
                          void* workspace, const moe_forward_aux_t* aux, void* stream_, const float* a4) {
  if (T == 0) return MOE_OK;
  if (!x || !out || !workspace || !al16(x) || !al16(out) || !al16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int32_t H = layer->hidden, E = layer->num_experts, k = layer->top_k;
  const bool has_shared = layer->shared.num_experts != 0;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  const int32_t S = T * k;
  const ForwardLayout L = forward_layout(T, H, I, Is, E, k, a4 != nullptr);

  float* logits = (aux && aux->logits) ? aux->logits : at<float>(workspace, L.logits);
  int32_t* ids = (aux && aux->topk_ids) ? aux->topk_ids : at<int32_t>(workspace, L.ids);
  float* w = (aux && aux->topk_w) ? aux->topk_w : at<float>(workspace, L.w);
  int32_t* counts = (aux && aux->expert_counts) ? aux->expert_counts : at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted_slot = at<int32_t>(workspace, L.sorted_slot);
  int32_t* slot_to_row = at<int32_t>(workspace, L.slot_to_row);
  int32_t* block_hist = at<int32_t>(workspace, L.block_hist);
  uint16_t* h = at<uint16_t>(workspace, L.h);
  uint16_t* h_shared = at<uint16_t>(workspace, L.h_shared);
  uint16_t* y = (aux && aux->y_rows) ? aux->y_rows : at<uint16_t>(workspace, L.y);
  if (!al16(y)) return MOE_ERR_INVALID_ARGUMENT;

  void* const* events = aux ? aux->stage_events : nullptr;
  const std::function<moe_status_t(int)> mark = [&](int i) -> moe_status_t {
    if (!events || !events[i]) return MOE_OK;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  };

  moe_status_t st = mark(0);
  if (st) return st;

  // S4: routed rows gathered through sorted_slot; the shared expert rides in the same launch when
  // its width matches, otherwise it gets a launch of its own.
  const bool fuse_shared = has_shared && Is == I;
  GemmProblem gu{};
  gu.stage = MOE_GEMM_GATE_UP;
  gu.N = I;
  gu.K = H;
  gu.bank = bank_w13(layer->routed);
  gu.offsets = offsets;
  gu.G = E;
  gu.M = S;
  gu.a = x;
  gu.row_index = sorted_slot;
  gu.row_divisor = k;
  gu.out = h;
  if (fuse_shared) {
    // h_shared directly follows h: rows S..S+T-1 of one [S+T][I] matrix
    gu.has_extra = 1;
    gu.extra = bank_w13(layer->shared);
    gu.M_extra = T;
    gu.a_extra = x;
  }
  // S5 on the same rows (the shared expert's h rows follow the routed ones)
  GemmProblem dn{};
  dn.stage = MOE_GEMM_DOWN;
  dn.N = H;
  dn.K = I;
  dn.bank = bank_w2(layer->routed);
  dn.offsets = offsets;
  dn.G = E;
  dn.M = S;
  dn.a = h;
  dn.row_index = nullptr;
  dn.row_divisor = 1;
  dn.out = y;
  if (fuse_shared) {
    dn.has_extra = 1;
    dn.extra = bank_w2(layer->shared);
    dn.M_extra = T;
    dn.a_extra = h + (size_t)S * I;
  }

  // Few tokens, on request: two launches -- the router (which also clears the hand-off counters),
  // then S2-S6 fused (micro.hip).  Same tiles and arithmetic as the staged launches below.
  const bool fused = !a4 && aux && (aux->flags & MOE_FORWARD_FUSED_DECODE);
  if (fused && (fuse_shared || !has_shared) && moe::fused_decode_applies(gu, T, k)) {
    int32_t* ctr = at<int32_t>(workspace, L.ctr);
    const int n_ctr = moe::fused_decode_counter_words(T, k, E, fuse_shared);
    st = moe::launch_router_logits(x, layer->w_router, layer->router_bias, T, H, E, logits, stream, ctr, n_ctr);
    if (st || (st = mark(1))) return st;
    moe::FusedDecodeProblem fp{};
    fp.gu = gu;
    fp.dn = dn;
    fp.logits = logits;
    fp.T = T;
    fp.E = E;
    fp.k = k;
    fp.H = H;
    fp.ids = ids;
    fp.w = w;
    fp.counts = counts;
    fp.offsets = offsets;
    fp.sorted_slot = sorted_slot;
    fp.slot_to_row = slot_to_row;
    fp.out = out;
    fp.ctr = ctr;
    if ((st = moe::launch_fused_decode(fp, stream))) return st;
    for (int i = 2; i <= 5; ++i)
      if ((st = mark(i))) return st;
    return MOE_OK;
  }

  // the router launch clears the tile counters of the two GEMM launches
  int32_t* tile_ctr = at<int32_t>(workspace, L.tiles);
  st = run_routing(layer, x, T, logits, ids, w, counts, offsets, sorted_slot, slot_to_row, block_hist, mark, stream,
                   tile_ctr, 2 * moe::kTileCounterWords, at<float>(workspace, L.rpart));
  if (st) return st;
  gu.tile_ctr = tile_ctr;
  dn.tile_ctr = tile_ctr + moe::kTileCounterWords;

  // W4A4: the gate/up GEMMs read x's 4-bit values (e2m1 * block scale, exact in bf16) instead of x,
  // with d_x applied in their epilogues
  const uint16_t* xg = x;
  if (a4) {
    if ((st = mark(2))) return st;
    uint16_t* xa = at<uint16_t>(workspace, L.xa);
    if ((st = moe::launch_quantize_act_nv(x, T, H, a4[0], nullptr, nullptr, xa, stream))) return st;
    xg = xa;
    gu.a = xa;
    gu.a_extra = fuse_shared ? xa : nullptr;
    gu.a_gscale = a4[0];
  }

  // 128-row tiles for both GEMMs (and one m-tile numbering): h goes through the fragment-tiled
  // layout, so the down GEMM's A tiles are contiguous 1 KB loads (W4A16 only: the W4A4 forward
  // quantizes the row-major h between the GEMMs)
  const bool tiled = !a4 && (fuse_shared || !has_shared) && moe::grouped_gemm_uses_tall_tiles(gu);
  if (tiled) gu.out_tiled = h;
  // h as fp16 too (the down GEMM then also runs on fp16 operands): NVFP4 on both 128-row eight-wave
  // GEMMs, and the layer's bounds on the gate and up weight row norms given
  const bool h16 = tiled && !a4 && layer->h16_norm[0] > 0.f && layer->h16_norm[1] > 0.f &&
                   std::isfinite(layer->h16_norm[0]) && std::isfinite(layer->h16_norm[1]) &&
                   moe::grouped_gemm_takes_f16_rows(gu) && moe::grouped_gemm_takes_f16_rows(dn);
  if (moe::grouped_gemm_takes_f16_rows(gu)) {
    // fp16 operands halve the dequantization work of the NVFP4 weights (exact, see launch_act_to_f16)
    uint16_t* x16 = at<uint16_t>(workspace, L.x16);
    int32_t* row_shift = at<int32_t>(workspace, L.row_shift);
    if ((st = moe::launch_act_to_f16(xg, T, H, x16, row_shift, h16 ? layer->h16_norm[0] : 0.f,
                                     h16 ? layer->h16_norm[1] : 0.f, stream)))
      return st;
    gu.a16 = x16;
    gu.row_shift = row_shift;
  }
  // W4A16: event 2 after S3 and the fp16 row pass that prepares S4's operand rows, so that the S4
  // interval is the GEMM launches alone (with W4A4 the activation quantizer, a step of that method,
  // and the row pass on its output are in S4)
  if (!a4 && (st = mark(2))) return st;
  if (h16) {
    int32_t* hshift = at<int32_t>(workspace, L.hshift);
    gu.h16 = 1;
    gu.hshift_out = hshift;
    dn.h16 = 1;
    dn.a16 = h;
    dn.row_shift = hshift;
  }
  if ((st = moe::launch_grouped_gemm(gu, stream))) return st;
  if (has_shared && !fuse_shared) {
    GemmProblem gs{};
    gs.stage = MOE_GEMM_GATE_UP;
    gs.N = Is;
    gs.K = H;
    gs.bank = bank_w13(layer->shared);
    gs.G = 0;
    gs.M = 0;
    gs.out = h_shared;
    gs.has_extra = 1;
    gs.extra = gs.bank;
    gs.M_extra = T;
    gs.a_extra = xg;
    gs.a_gscale = a4 ? a4[0] : 0.f;
    if ((st = moe::launch_grouped_gemm(gs, stream))) return st;
  }
  if ((st = mark(3))) return st;

  // S5 (W4A4: h to its 4-bit values in place first, d_h in the epilogues)
  if (a4) {
    if (fuse_shared || !has_shared) {
      if ((st = moe::launch_quantize_act_nv(h, (int64_t)S + (has_shared ? T : 0), I, a4[1], nullptr, nullptr, h,
                                            stream)))
        return st;
    } else {
      if ((st = moe::launch_quantize_act_nv(h, S, I, a4[1], nullptr, nullptr, h, stream))) return st;
      if ((st = moe::launch_quantize_act_nv(h_shared, T, Is, a4[1], nullptr, nullptr, h_shared, stream))) return st;
    }
    dn.a_gscale = a4[1];
  }
  dn.a_tiled = tiled ? 1 : 0;
  if ((st = moe::launch_grouped_gemm(dn, stream))) return st;
  if (has_shared && !fuse_shared) {
    GemmProblem ds{};
    ds.stage = MOE_GEMM_DOWN;
    ds.N = H;
    ds.K = Is;
    ds.bank = bank_w2(layer->shared);
    ds.G = 0;
    ds.M = S;  // output rows start after the routed rows
    ds.out = y;
    ds.has_extra = 1;
    ds.extra = ds.bank;
    ds.M_extra = T;
    ds.a_extra = h_shared;
    ds.a_gscale = a4 ? a4[1] : 0.f;
    if ((st = moe::launch_grouped_gemm(ds, stream))) return st;
  }
  if ((st = mark(4))) return st;

  // S6
  st = moe::launch_combine(y, slot_to_row, w, has_shared ? y + (size_t)S * H : nullptr, T, k, H, out, stream);
  if (st) return st;
  return mark(5);
}

}  // namespace

moe_status_t moe_nvfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T, uint16_t* out,
                               void* workspace, size_t workspace_bytes, const moe_forward_aux_t* aux,
                               void* stream) {
  if (moe_status_t st = moe_validate_forward(layer, T, workspace_bytes, nullptr)) return st;
  return forward_impl(layer, x, T, out, workspace, aux, stream, nullptr);
}

size_t moe_nvfp4_w4a4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared, int32_t E, int32_t k) {
  if (T < 0 || H <= 0 || I <= 0 || I_shared < 0 || E < 1 || k < 1) return 0;
  return forward_layout(T, H, I, I_shared, E, k, true).total;
}

moe_status_t moe_nvfp4_w4a4_validate_forward(const moe_nvfp4_layer_t* layer, int32_t T, size_t workspace_bytes,
                                             float act_gscale_x, float act_gscale_h, const char* gfx_arch) {
  if (!valid_act_gscale(act_gscale_x) || !valid_act_gscale(act_gscale_h)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = validate_layer(layer, T)) return st;
  if (layer->routed.format != MOE_WEIGHT_NVFP4) return MOE_ERR_INVALID_ARGUMENT;
  const bool has_shared = layer->shared.num_experts != 0;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  if (T > 0 && workspace_bytes < moe_nvfp4_w4a4_forward_workspace_size(T, layer->hidden, I, Is, layer->num_experts,
                                                                        layer->top_k))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return check_arch(gfx_arch);
}

moe_status_t moe_nvfp4_w4a4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                                    float act_gscale_x, float act_gscale_h, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, const moe_forward_aux_t* aux, void* stream) {
  if (moe_status_t st = moe_nvfp4_w4a4_validate_forward(layer, T, workspace_bytes, act_gscale_x, act_gscale_h,
                                                        nullptr))
    return st;
  const float a4[2] = {act_gscale_x, act_gscale_h};
  return forward_impl(layer, x, T, out, workspace, aux, stream, a4);
}

moe_status_t moe_nvfp4_quantize_act(const uint16_t* a, int32_t rows, int32_t cols, float gscale, uint8_t* packed,
                                    uint8_t* scales, uint16_t* values, void* stream) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || !valid_act_gscale(gscale)) return MOE_ERR_INVALID_ARGUMENT;
  if (!packed && !scales && !values) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)rows * cols == 0) return MOE_OK;
  if (!a || !al16(a) || (packed && !al16(packed)) || (values && !al16(values))) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_quantize_act_nv(a, rows, cols, gscale, packed, scales, values, static_cast<hipStream_t>(stream));
}

moe_status_t moe_gscale_from_quant_scale(const float* q_host, float* d_host, int32_t n) {
  if (n < 0 || (n > 0 && (!q_host || !d_host))) return MOE_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n; ++i)
    if (!(std::isfinite(q_host[i])) || q_host[i] == 0.0f) return MOE_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < n; ++i) d_host[i] = 1.0f / q_host[i];
  return MOE_OK;
}

moe_status_t moe_nvfp4_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream) {
  if (num_tensors < 0 || rows < 0 || cols < 0 || rows % 16 != 0 || cols % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_tensors * rows * cols == 0) return MOE_OK;
  if (!packed || !scales || !tiled || !tiled_scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(packed) || !al16(scales) || !al16(tiled) || !al16(tiled_scales)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_pack_tiles(packed, scales, num_tensors, rows, cols, tiled, tiled_scales,
                                static_cast<hipStream_t>(stream));
}

moe_status_t moe_nvfp4_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols, const float* gscale,
                                uint8_t* packed, uint8_t* scales, void* stream) {
  if (num_tensors < 0 || rows < 0 || cols < 0 || cols % 16 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_tensors * rows * cols == 0) return MOE_OK;
  if (!w || !gscale || !packed || !scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(w) || !al16(packed)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_quantize(w, num_tensors, rows, cols, gscale, packed, scales, static_cast<hipStream_t>(stream));
}

moe_status_t moe_nvfp4_h16_bound(const moe_nvfp4_experts_t* bank, float* bound, void* stream) {
  if (!bank || !bound) return MOE_ERR_INVALID_ARGUMENT;
  if (bank->format != MOE_WEIGHT_NVFP4 || bank->num_experts < 0 || bank->inter <= 0 || bank->inter % 16 != 0 ||
      bank->hidden <= 0 || bank->hidden % 128 != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (bank->num_experts == 0) return MOE_OK;
  if (!bank->w13 || !bank->w13_scale || !bank->w13_gscale || !al16(bank->w13) || (reinterpret_cast<uintptr_t>(bound) & 3))
    return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_h16_bound(bank->w13, bank->w13_scale, bank->w13_gscale, bank->num_experts, bank->inter,
                               bank->hidden, bound, static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp4_pack_tiles(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                  int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream) {
  if (num_tensors < 0 || rows < 0 || cols < 0 || rows % 16 != 0 || cols % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_tensors * rows * cols == 0) return MOE_OK;
  if (!packed || !scales || !tiled || !tiled_scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(packed) || !al16(scales) || !al16(tiled) || !al16(tiled_scales)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_pack_tiles_mx(packed, scales, num_tensors, rows, cols, tiled, tiled_scales,
                                   static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp4_quantize(const float* w, int32_t num_tensors, int32_t rows, int32_t cols, uint8_t* packed,
                                uint8_t* scales, void* stream) {
  if (num_tensors < 0 || rows < 0 || cols < 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_tensors * rows * cols == 0) return MOE_OK;
  if (!w || !packed || !scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(w) || !al16(packed)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_quantize_mx(w, num_tensors, rows, cols, packed, scales, static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp4_quantize_act(const uint16_t* a, int32_t rows, int32_t cols, uint8_t* packed, uint8_t* scales,
                                    void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)rows * cols == 0) return MOE_OK;
  if (!a || !packed || !scales || !al16(a) || !al16(packed)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_quantize_act_mx(a, rows, cols, packed, scales, static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp4_pack_tiles_a4(const uint8_t* packed, const uint8_t* scales, int32_t num_tensors, int32_t rows,
                                     int32_t cols, uint8_t* tiled, uint8_t* tiled_scales, void* stream) {
  if (num_tensors < 0 || rows < 0 || cols < 0 || rows % 16 != 0 || cols % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)num_tensors * rows * cols == 0) return MOE_OK;
  if (!packed || !scales || !tiled || !tiled_scales) return MOE_ERR_INVALID_ARGUMENT;
  if (!al16(packed) || !al16(scales) || !al16(tiled) || !al16(tiled_scales)) return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  return moe::launch_pack_tiles_a4(packed, scales, num_tensors, rows, cols, tiled, tiled_scales,
                                   static_cast<hipStream_t>(stream));
}

moe_status_t moe_mxfp4_w4a4_grouped_gemm(int32_t stage, const moe_nvfp4_experts_t* w, const uint8_t* a,
                                         const uint8_t* a_scale, const int32_t* row_index, int32_t row_divisor,
                                         const int32_t* expert_offsets, int32_t M_total, uint16_t* out, void* stream) {
  if (!w || (stage != MOE_GEMM_GATE_UP && stage != MOE_GEMM_DOWN)) return MOE_ERR_INVALID_ARGUMENT;
  if (w->num_experts < 1 || w->num_experts > 1024) return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_bank(*w, w->hidden, w->num_experts) || w->format != MOE_WEIGHT_MXFP4_A4) return MOE_ERR_INVALID_ARGUMENT;
  if (w->hidden <= 0 || w->hidden % 128 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (M_total < 0 || row_divisor < 1) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t K_ = stage == MOE_GEMM_GATE_UP ? w->hidden : w->inter;
  if ((int64_t)M_total * K_ / 2 >= kMaxActivationBytes) return MOE_ERR_INVALID_ARGUMENT;
  if (stage == MOE_GEMM_DOWN && row_index) return MOE_ERR_INVALID_ARGUMENT;
  if (M_total == 0) return MOE_OK;
  if (!a || !a_scale || !expert_offsets || !out || !al16(a) || !al16(a_scale) || !al16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  if (moe_status_t st = check_arch(nullptr)) return st;
  moe::GemmProblemA4 p{};
  p.stage = stage;
  const bool gu = stage == MOE_GEMM_GATE_UP;
  p.N = gu ? w->inter : w->hidden;
  p.K = gu ? w->hidden : w->inter;
  p.bank = gu ? bank_w13(*w) : bank_w2(*w);
  p.offsets = expert_offsets;
  p.G = w->num_experts;
  p.M = M_total;
  p.a = a;
  p.a_scale = a_scale;
  p.row_index = row_index;
  p.row_divisor = row_divisor;
  p.out = out;
  return moe::launch_grouped_gemm_a4(p, static_cast<hipStream_t>(stream));
}

size_t moe_mxfp4_w4a4_forward_workspace_size(int32_t T, int32_t H, int32_t I, int32_t I_shared, int32_t E, int32_t k) {
  if (T < 0 || H <= 0 || I <= 0 || I_shared < 0 || E < 1 || k < 1) return 0;
  return forward_layout_a4(T, H, I, I_shared, E, k).total;
}

moe_status_t moe_mxfp4_w4a4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T, uint16_t* out,
                                    void* workspace, size_t workspace_bytes, const moe_forward_aux_t* aux,
                                    void* stream_) {
  if (moe_status_t st = moe_mxfp4_w4a4_validate_forward(layer, T, workspace_bytes, nullptr)) return st;
  if (T == 0) return MOE_OK;
  const int32_t H = layer->hidden, E = layer->num_experts, k = layer->top_k;
  const bool has_shared = layer->shared.num_experts != 0;
  const int32_t I = layer->routed.inter, Is = has_shared ? layer->shared.inter : 0;
  if (!x || !out || !workspace || !al16(x) || !al16(out) || !al16(workspace)) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int32_t S = T * k;
  const ForwardLayoutA4 L = forward_layout_a4(T, H, I, Is, E, k);

  float* logits = (aux && aux->logits) ? aux->logits : at<float>(workspace, L.logits);
  int32_t* ids = (aux && aux->topk_ids) ? aux->topk_ids : at<int32_t>(workspace, L.ids);
  float* w = (aux && aux->topk_w) ? aux->topk_w : at<float>(workspace, L.w);
  int32_t* counts = (aux && aux->expert_counts) ? aux->expert_counts : at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted_slot = at<int32_t>(workspace, L.sorted_slot);
  int32_t* slot_to_row = at<int32_t>(workspace, L.slot_to_row);
  int32_t* block_hist = at<int32_t>(workspace, L.block_hist);
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  uint8_t* xs = at<uint8_t>(workspace, L.xs);
  uint16_t* h = at<uint16_t>(workspace, L.h);
  uint8_t* hq = at<uint8_t>(workspace, L.hq);
  uint8_t* hs = at<uint8_t>(workspace, L.hs);
  uint16_t* y = (aux && aux->y_rows) ? aux->y_rows : at<uint16_t>(workspace, L.y);
  if (!al16(y)) return MOE_ERR_INVALID_ARGUMENT;
  // the shared expert's rows follow the routed ones in h and in its 4-bit copy
  uint16_t* h_sh = h + (size_t)S * I;
  uint8_t* hq_sh = hq + (size_t)S * I / 2;
  uint8_t* hs_sh = hs + (size_t)S * I / 32;

  void* const* events = aux ? aux->stage_events : nullptr;
  const std::function<moe_status_t(int)> mark = [&](int i) -> moe_status_t {
    if (!events || !events[i]) return MOE_OK;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  };

  moe_status_t st = mark(0);
  if (st) return st;
  st = run_routing(layer, x, T, logits, ids, w, counts, offsets, sorted_slot, slot_to_row, block_hist, mark, stream);
  if (st || (st = mark(2))) return st;

  // S4: x to MXFP4 once per token; routed rows gathered through sorted_slot, the shared expert in
  // the same launch when its width matches
  if ((st = moe::launch_quantize_act_mx(x, T, H, xq, xs, stream))) return st;
  const bool fuse_shared = has_shared && Is == I;
  moe::GemmProblemA4 gu{};
  gu.stage = MOE_GEMM_GATE_UP;
  gu.N = I;
  gu.K = H;
  gu.bank = bank_w13(layer->routed);
  gu.offsets = offsets;
  gu.G = E;
  gu.M = S;
  gu.a = xq;
  gu.a_scale = xs;
  gu.row_index = sorted_slot;
  gu.row_divisor = k;
  gu.out = h;
  if (fuse_shared) {
    gu.has_extra = 1;
    gu.extra = bank_w13(layer->shared);
    gu.M_extra = T;
    gu.a_extra = xq;
    gu.a_extra_scale = xs;
  }
  if ((st = moe::launch_grouped_gemm_a4(gu, stream))) return st;
  if (has_shared && !fuse_shared) {
    moe::GemmProblemA4 gs{};
    gs.stage = MOE_GEMM_GATE_UP;
    gs.N = Is;
    gs.K = H;
    gs.bank = bank_w13(layer->shared);
    gs.out = h_sh;
    gs.has_extra = 1;
    gs.extra = gs.bank;
    gs.M_extra = T;
    gs.a_extra = xq;
    gs.a_extra_scale = xs;
    if ((st = moe::launch_grouped_gemm_a4(gs, stream))) return st;
  }
  if ((st = mark(3))) return st;

  // S5: h (bf16) to MXFP4, then the down GEMM
  if (fuse_shared || !has_shared) {
    if ((st = moe::launch_quantize_act_mx(h, (int64_t)S + (has_shared ? T : 0), I, hq, hs, stream))) return st;
  } else {
    if ((st = moe::launch_quantize_act_mx(h, S, I, hq, hs, stream))) return st;
    if ((st = moe::launch_quantize_act_mx(h_sh, T, Is, hq_sh, hs_sh, stream))) return st;
  }
  moe::GemmProblemA4 dn{};
  dn.stage = MOE_GEMM_DOWN;
  dn.N = H;
  dn.K = I;
  dn.bank = bank_w2(layer->routed);
  dn.offsets = offsets;
  dn.G = E;
  dn.M = S;
  dn.a = hq;
  dn.a_scale = hs;
  dn.row_divisor = 1;
  dn.out = y;
  if (fuse_shared) {
    dn.has_extra = 1;
    dn.extra = bank_w2(layer->shared);
    dn.M_extra = T;
    dn.a_extra = hq_sh;
    dn.a_extra_scale = hs_sh;
  }
  if ((st = moe::launch_grouped_gemm_a4(dn, stream))) return st;
  if (has_shared && !fuse_shared) {
    moe::GemmProblemA4 ds{};
    ds.stage = MOE_GEMM_DOWN;
    ds.N = H;
    ds.K = Is;
    ds.bank = bank_w2(layer->shared);
    ds.M = S;  // output rows start after the routed rows
    ds.out = y;
    ds.has_extra = 1;
    ds.extra = ds.bank;
    ds.M_extra = T;
    ds.a_extra = hq_sh;
    ds.a_extra_scale = hs_sh;
    if ((st = moe::launch_grouped_gemm_a4(ds, stream))) return st;
  }
  if ((st = mark(4))) return st;

  // S6
  st = moe::launch_combine(y, slot_to_row, w, has_shared ? y + (size_t)S * H : nullptr, T, k, H, out, stream);
  if (st) return st;
  return mark(5);
}

}  // extern "C"
