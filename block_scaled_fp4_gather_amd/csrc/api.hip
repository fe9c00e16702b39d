// C-ABI of libmoe_fp4.so (declared in include/moe_fp4.h): argument checks,
// sizing, and the launches.  Every check runs before any HIP call, so a
// rejected call touches neither the device nor the stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/moe_fp4.h"
#include "decode_path.h"
#include "layout.h"
#include "mxfp8.h"
#include "prefill.h"

using moe::Layout;

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Chunks of decode_max_tokens(k) tokens a call with bf16 activations takes
// on the decode path by default: up to kDecodeAnyChunks whatever the
// routing, up to kDecodeMaxChunks when the chunks' route slots (chunks x
// tokens per chunk x k) are fewer than E (few routes per expert: the decode
// path reads an expert once per chunk, the grouped path batches an expert's
// routes); other calls take the grouped path.  Measured on MI355X: two chunks were faster than the grouped path on
// every layer from E8/H256 to E512/H2560; at 3-6 chunks E256-E512 layers
// gained up to 1.0-1.5 E routes, while E128/H2048 at 1.5 E and E64/H1024 at
// 3 E ran faster grouped.
constexpr int kDecodeAnyChunks = 2;
constexpr int kDecodeMaxChunks = 6;

moe_fp4_status desc_layout(const moe_fp4_desc* d, Layout* L) {
  if (!d) return MOE_FP4_EINVAL;
  if (d->format != MOE_FP4_MXFP4 && d->format != MOE_FP4_NVFP4) return MOE_FP4_EINVAL;
  if (d->num_experts <= 0 || d->hidden <= 0 || d->inter <= 0 || d->top_k <= 0 || d->max_tokens < 0)
    return MOE_FP4_EINVAL;
  const int G = d->format == MOE_FP4_MXFP4 ? 32 : 16;
  if (d->hidden % G || d->inter % G) return MOE_FP4_EINVAL;  // not whole scale blocks
  if (d->hidden % 32 || d->inter % 32) return MOE_FP4_EUNSUPPORTED;
  if ((int64_t)d->hidden * d->inter > (int64_t)1 << 30) return MOE_FP4_EUNSUPPORTED;
  if (d->act_format != MOE_FP4_ACT_BF16 && d->act_format != MOE_FP4_ACT_MXFP8) return MOE_FP4_EINVAL;
  if (d->act_format == MOE_FP4_ACT_MXFP8 && d->format != MOE_FP4_MXFP4) return MOE_FP4_EUNSUPPORTED;
  if (d->act_fn != MOE_FP4_FN_SILU && d->act_fn != MOE_FP4_FN_GELU_TANH && d->act_fn != MOE_FP4_FN_SWIGLUOAI &&
      d->act_fn != MOE_FP4_FN_RELU2)
    return MOE_FP4_EINVAL;
  const bool gated = d->act_fn != MOE_FP4_FN_RELU2;
  if (!gated && d->inter % 64) return MOE_FP4_EUNSUPPORTED;  // two 32-row halves per FC1 tile
  if (d->act_fn == MOE_FP4_FN_SWIGLUOAI &&
      (!std::isfinite(d->act_alpha) || !std::isfinite(d->act_beta) || !(d->act_limit > 0.0f)))
    return MOE_FP4_EINVAL;
  if (d->scale_format != MOE_FP4_SCALES_PLAIN && d->scale_format != MOE_FP4_SCALES_CSF) return MOE_FP4_EINVAL;
  if (!moe::make_layout(d->format, d->num_experts, d->hidden, d->inter, L, gated,
                        d->scale_format == MOE_FP4_SCALES_CSF))
    return MOE_FP4_EINVAL;
  L->act = moe::ActParams{d->act_fn, d->act_alpha, d->act_beta, d->act_limit};
  return MOE_FP4_OK;
}

// Route slots the decode workspace is sized for (every route of max_tokens
// tokens: the decode path keeps the activation rows of all its chunks); it
// depends only on the descriptor.
int decode_slots(const moe_fp4_desc* d) {
  return (d->max_tokens < 1 ? 1 : d->max_tokens) * d->top_k;
}

// Routes the grouped path's workspace is sized for (desc capacity).
int64_t prefill_routes(const moe_fp4_desc* d) {
  return (int64_t)(d->max_tokens < 1 ? 1 : d->max_tokens) * d->top_k;
}

bool act_mxfp8(const moe_fp4_desc* d) { return d->act_format == MOE_FP4_ACT_MXFP8; }

// Tokens the grouped path's workspace is sized for.
int64_t prefill_tokens(const moe_fp4_desc* d) { return d->max_tokens < 1 ? 1 : d->max_tokens; }

moe::PrefillWs prefill_layout(const Layout& L, const moe_fp4_desc* d) {
  return moe::prefill_ws(L, prefill_routes(d), prefill_tokens(d), act_mxfp8(d));
}

// Workspace layout: both paths start at offset 0 and never run in one call.
int64_t workspace_total(const Layout& L, const moe_fp4_desc* d) {
  const int64_t a = moe::decode_ws(L, decode_slots(d)).total;
  const int64_t b = prefill_layout(L, d).total;
  return a > b ? a : b;
}

moe_fp4_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_FP4_OK : MOE_FP4_EHIP; }

// The path and launch shape of a call: MOE_FP4_PATH_GROUPED or
// MOE_FP4_PATH_DECODE, and the decode shape with every field resolved.
struct Plan {
  int path;
  moe::DecodeShape shape;
};

moe_fp4_status make_plan(const moe_fp4_desc* desc, const Layout& L, int32_t M,
                         const moe_fp4_tuning* tuning, Plan* plan) {
  moe::DecodeShape shape{0, 0, 0};
  int path = MOE_FP4_PATH_AUTO;
  if (tuning) {
    shape = moe::DecodeShape{tuning->fc1_chunks_per_wave, tuning->fc1_rows, tuning->fc2_rows};
    path = tuning->path;
    if (path < MOE_FP4_PATH_AUTO || path > MOE_FP4_PATH_GROUPED || !moe::valid_shape(L, shape))
      return MOE_FP4_EINVAL;
  }
  if (prefill_routes(desc) > moe::kPrefillMaxRoutes ||
      moe::prefill_max_workgroups(L, prefill_routes(desc)) >= ((int64_t)1 << 31))
    return MOE_FP4_EUNSUPPORTED;
  const int k = desc->top_k;
  // The decode path takes any M in chunks of at most decode_max_tokens(k)
  // tokens.  By default with bf16 activations: up to kDecodeAnyChunks
  // chunks, up to kDecodeMaxChunks when chunks mc k < E (MXFP8 activations: one
  // chunk, their grouped path quantises them); the grouped path beyond; the
  // decode path for any M when E is past what the grouped path's route
  // grouping holds.
  const bool decode_ok = k <= moe::kDecodeMaxSlots;
  const int mc = decode_ok ? moe::decode_max_tokens(k) : 1;
  const int64_t chunks = ((int64_t)(M < 1 ? 1 : M) + mc - 1) / mc;
  const bool few_routes = chunks * mc * k < (int64_t)L.E;
  const int64_t auto_chunks = act_mxfp8(desc) ? 1 : (few_routes ? kDecodeMaxChunks : kDecodeAnyChunks);
  if (path == MOE_FP4_PATH_AUTO)
    path = decode_ok && (chunks <= auto_chunks || L.E > moe::kRouteMaxExperts) ? MOE_FP4_PATH_DECODE
                                                                               : MOE_FP4_PATH_GROUPED;
  if (path == MOE_FP4_PATH_DECODE && !decode_ok) return MOE_FP4_EUNSUPPORTED;
  // the decode launches put token chunks and groups (at most M of them) on
  // the grid's second dimension, which holds at most 65535 workgroups
  if (path == MOE_FP4_PATH_DECODE && M > 65535) return MOE_FP4_EUNSUPPORTED;
  if (path == MOE_FP4_PATH_GROUPED && L.E > moe::kRouteMaxExperts) return MOE_FP4_EUNSUPPORTED;
  if (path == MOE_FP4_PATH_DECODE) {
    const int mc_call = M < mc ? (M < 1 ? 1 : M) : mc;
    shape = moe::resolve_shape(L, mc_call * k, shape);
    // FC1 stages a token's H activations in LDS: past what a workgroup may
    // allocate, the decode path cannot run this layer
    if (moe::fc1_lds_bytes(L, mc_call, shape.r1) > moe::kMaxLdsBytes) {
      const bool auto_path = !tuning || tuning->path == MOE_FP4_PATH_AUTO;
      if (!auto_path || L.E > moe::kRouteMaxExperts) return MOE_FP4_EUNSUPPORTED;
      path = MOE_FP4_PATH_GROUPED;
      shape = moe::DecodeShape{0, 0, 0};
    }
  }
  plan->path = path;
  plan->shape = shape;
  return MOE_FP4_OK;
}

// With check_only, every check runs and nothing is launched.
template <typename IdT>
moe_fp4_status forward_impl(const moe_fp4_desc* desc, const void* prepared, const uint16_t* x,
                            int32_t M, const IdT* ids, const float* w, uint16_t* out,
                            void* workspace, size_t ws_bytes, const moe_fp4_tuning* tuning,
                            int32_t phases, void* stream, bool check_only = false) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (M < 0 || M > desc->max_tokens) return MOE_FP4_EINVAL;
  if (M == 0) return MOE_FP4_OK;
  if (!prepared || !x || !ids || !w || !out || !workspace) return MOE_FP4_EINVAL;
  if (!aligned(prepared, 256) || !aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(ids, sizeof(IdT)) || !aligned(w, 4))
    return MOE_FP4_EINVAL;
  if (phases != 1 && phases != 2 && phases != 3 && phases != 4 && phases != 8) return MOE_FP4_EINVAL;
  Plan plan;
  st = make_plan(desc, L, M, tuning, &plan);
  if (st != MOE_FP4_OK) return st;
  const int k = desc->top_k;
  if (plan.path != MOE_FP4_PATH_GROUPED && phases > 3) return MOE_FP4_EINVAL;
  if ((int64_t)ws_bytes < workspace_total(L, desc)) return MOE_FP4_EWORKSPACE;
  if (check_only) return MOE_FP4_OK;
  if (plan.path == MOE_FP4_PATH_GROUPED)
    return from_hip(moe::launch_prefill<IdT>(L, (const uint8_t*)prepared, x, M, k, ids, w, out,
                                             (uint8_t*)workspace, prefill_layout(L, desc), phases,
                                             act_mxfp8(desc), (hipStream_t)stream));
  // decode: one FC1 launch over all chunks of decode_max_tokens(k) tokens
  // (the grid's second dimension), one FC2 launch over all tokens
  const moe::DecodeWs W = moe::decode_ws(L, decode_slots(desc));
  return from_hip(moe::launch_decode<IdT>(L, (const uint8_t*)prepared, x, M, k, ids, w, out,
                                          (uint8_t*)workspace, W, plan.shape, phases, (hipStream_t)stream));
}

// The workspace of moe_fp4_forward_noalloc: device memory the library holds
// for callers that cannot allocate, one copy per GPU the library runs on
// (it lives until the process ends).  Host code never passes the array's
// name to a kernel: it stands for a host-side stand-in, not the device
// address, which scratch_address() looks up once per device.
constexpr int64_t kNoAllocScratchBytes = (int64_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).
moe_fp4_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_FP4_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_FP4_EHIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MOE_FP4_OK;
}

}  // namespace

extern "C" {

const char* moe_fp4_status_string(moe_fp4_status s) {
  switch (s) {
    case MOE_FP4_OK: return "ok";
    case MOE_FP4_EINVAL: return "invalid argument";
    case MOE_FP4_EUNSUPPORTED: return "unsupported shape or size";
    case MOE_FP4_EWORKSPACE: return "buffer too small";
    case MOE_FP4_EHIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

moe_fp4_status moe_fp4_prepared_bytes(const moe_fp4_desc* desc, size_t* bytes) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!bytes) return MOE_FP4_EINVAL;
  *bytes = (size_t)moe::layout_total(L);
  return MOE_FP4_OK;
}

moe_fp4_status moe_fp4_prepare(const moe_fp4_desc* desc, const uint8_t* w13_codes,
                               const uint8_t* w13_scales, const uint8_t* w2_codes,
                               const uint8_t* w2_scales, const float* g13, const float* g2,
                               void* prepared, size_t prepared_bytes, void* stream) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!w13_codes || !w13_scales || !w2_codes || !w2_scales || !prepared) return MOE_FP4_EINVAL;
  const bool nv = desc->format == MOE_FP4_NVFP4;
  if (nv != (g13 != nullptr) || nv != (g2 != nullptr)) return MOE_FP4_EINVAL;
  if (!aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(prepared, 256)) return MOE_FP4_EINVAL;
  if ((nv && (!aligned(g13, 4) || !aligned(g2, 4)))) return MOE_FP4_EINVAL;
  if ((int64_t)prepared_bytes < moe::layout_total(L)) return MOE_FP4_EWORKSPACE;
  return from_hip(moe::launch_repack(L, 0, (uint8_t*)w13_codes, (uint8_t*)w13_scales,
                                     (uint8_t*)w2_codes, (uint8_t*)w2_scales, (float*)g13,
                                     (float*)g2, (uint8_t*)prepared, (hipStream_t)stream));
}

moe_fp4_status moe_fp4_unprepare(const moe_fp4_desc* desc, const void* prepared,
                                 uint8_t* w13_codes, uint8_t* w13_scales, uint8_t* w2_codes,
                                 uint8_t* w2_scales, float* g13, float* g2, void* stream) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!w13_codes || !w13_scales || !w2_codes || !w2_scales || !prepared) return MOE_FP4_EINVAL;
  const bool nv = desc->format == MOE_FP4_NVFP4;
  if (nv != (g13 != nullptr) || nv != (g2 != nullptr)) return MOE_FP4_EINVAL;
  if (!aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(prepared, 256)) return MOE_FP4_EINVAL;
  return from_hip(moe::launch_repack(L, 1, w13_codes, w13_scales, w2_codes, w2_scales, g13, g2,
                                     (uint8_t*)prepared, (hipStream_t)stream));
}

moe_fp4_status moe_fp4_workspace_bytes(const moe_fp4_desc* desc, int32_t M, size_t* bytes) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!bytes || M < 0 || M > desc->max_tokens) return MOE_FP4_EINVAL;
  if (prefill_routes(desc) > moe::kPrefillMaxRoutes) return MOE_FP4_EUNSUPPORTED;
  *bytes = (size_t)workspace_total(L, desc);
  return MOE_FP4_OK;
}

moe_fp4_status moe_fp4_forward(const moe_fp4_desc* desc, const void* prepared, const uint16_t* x,
                               int32_t M, const int32_t* topk_ids, const float* topk_w,
                               uint16_t* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return forward_impl<int32_t>(desc, prepared, x, M, topk_ids, topk_w, out, workspace,
                               workspace_bytes, nullptr, 3, stream);
}

moe_fp4_status moe_fp4_forward_i64(const moe_fp4_desc* desc, const void* prepared,
                                   const uint16_t* x, int32_t M, const int64_t* topk_ids,
                                   const float* topk_w, uint16_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return forward_impl<int64_t>(desc, prepared, x, M, topk_ids, topk_w, out, workspace,
                               workspace_bytes, nullptr, 3, stream);
}

moe_fp4_status moe_fp4_forward_noalloc(const moe_fp4_desc* desc, const void* prepared,
                                       const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                       const float* topk_w, uint16_t* out, void* stream) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (prefill_routes(desc) > moe::kPrefillMaxRoutes) return MOE_FP4_EUNSUPPORTED;
  const int64_t need = workspace_total(L, desc);
  if (need > kNoAllocScratchBytes) return MOE_FP4_EWORKSPACE;
  // every check of moe_fp4_forward, before any HIP call (an aligned stand-in
  // for the workspace pointer; nothing is launched)
  st = forward_impl<int32_t>(desc, prepared, x, M, topk_ids, topk_w, out, (void*)(uintptr_t)256,
                             (size_t)need, nullptr, 3, stream, true);
  if (st != MOE_FP4_OK || M == 0) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_FP4_OK) return st;
  return forward_impl<int32_t>(desc, prepared, x, M, topk_ids, topk_w, out, ws, (size_t)need, nullptr, 3,
                               stream);
}

moe_fp4_status moe_fp4_forward_ex(const moe_fp4_desc* desc, const void* prepared,
                                  const uint16_t* x, int32_t M, const int32_t* topk_ids,
                                  const float* topk_w, uint16_t* out, void* workspace,
                                  size_t workspace_bytes, const moe_fp4_tuning* tuning,
                                  int32_t phases, void* stream) {
  return forward_impl<int32_t>(desc, prepared, x, M, topk_ids, topk_w, out, workspace,
                               workspace_bytes, tuning, phases, stream);
}

moe_fp4_status moe_fp4_plan(const moe_fp4_desc* desc, int32_t M, const moe_fp4_tuning* tuning,
                            moe_fp4_tuning* plan) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!plan || M < 0 || M > desc->max_tokens) return MOE_FP4_EINVAL;
  Plan p;
  st = make_plan(desc, L, M, tuning, &p);
  if (st != MOE_FP4_OK) return st;
  const bool grouped = p.path == MOE_FP4_PATH_GROUPED;
  plan->fc1_chunks_per_wave = grouped ? 0 : p.shape.kl1;
  plan->fc1_rows = grouped ? 0 : p.shape.r1;
  plan->fc2_rows = grouped ? 0 : p.shape.r2;
  plan->path = p.path;
  return MOE_FP4_OK;
}

moe_fp4_status moe_fp4_dequant_export(const moe_fp4_desc* desc, const void* prepared,
                                      int32_t expert, int32_t which, float* out, void* stream) {
  Layout L;
  moe_fp4_status st = desc_layout(desc, &L);
  if (st != MOE_FP4_OK) return st;
  if (!prepared || !out || expert < 0 || expert >= L.E || (which != 0 && which != 1))
    return MOE_FP4_EINVAL;
  if (!aligned(prepared, 256) || !aligned(out, 4)) return MOE_FP4_EINVAL;
  return from_hip(moe::launch_export(L, expert, which, (const uint8_t*)prepared, out,
                                     (hipStream_t)stream));
}

moe_fp4_status moe_fp4_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* codes,
                                      uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return MOE_FP4_EINVAL;
  if (rows == 0) return MOE_FP4_OK;
  if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 8)) return MOE_FP4_EINVAL;
  if (rows > ((int64_t)1 << 40) / cols) return MOE_FP4_EUNSUPPORTED;
  return from_hip(launch_mxfp8_quantize(x, rows, cols, codes, scales, cols / 32, (hipStream_t)stream));
}

}  // extern "C"
