// C ABI of the MoE layer: argument validation, workspace carving and the
// kernel launches.  Every check runs on the host before anything is
// enqueued, so a refused call leaves the stream and every buffer untouched.
#include <stdint.h>

#include "moe_internal.h"

namespace {

constexpr int kMaxTopK = 8;
constexpr int kMaxRouteExperts = 256;
constexpr int kMaxExperts = 1023;
constexpr int32_t kMaxTokens = MOE_MAX_TOKENS;  // keeps every grid dimension and 32-bit row count in range

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_experts(const moe_experts* d) {
  if (!d || !d->base) return MOE_EINVAL;
  if (d->abi_version != MOE_ABI_VERSION) return MOE_ELAYOUT;
  if (d->layout != MOE_LAYOUT_GFX950_TILED_V1) return MOE_ELAYOUT;
  if ((d->flags & ~(MOE_FFN_SPLIT_FP8 | MOE_SHARED_MXFP8 | MOE_ROUTED_AFFINE2)) != 0) return MOE_EINVAL;
  if ((d->flags & MOE_FFN_SPLIT_FP8) && (d->flags & (MOE_SHARED_MXFP8 | MOE_ROUTED_AFFINE2))) return MOE_EINVAL;
  if (d->n_experts < 1 || d->n_experts > kMaxExperts) return MOE_ESHAPE;
  const bool a2 = (d->flags & MOE_ROUTED_AFFINE2) != 0;
  const uint64_t eb = a2 ? moe_expert_bytes_affine2(d->hidden, d->inter) : moe_expert_bytes(d->hidden, d->inter);
  if (eb == 0 || d->expert_bytes != eb) return MOE_ESHAPE;
  // the affine codec's decode-family kernels exist for these K sizes only
  if (a2 && !(moe::decode_k_ok(d->hidden) && moe::decode_k_ok(d->inter))) return MOE_ESHAPE;
  if (!aligned(d->base, 256)) return MOE_EALIGN;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EALIGN: return "MOE_EALIGN: misaligned pointer";
    case MOE_ELAYOUT: return "MOE_ELAYOUT: wrong layout tag or ABI version";
    case MOE_ESHAPE: return "MOE_ESHAPE: unsupported shape";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
    default: return "unknown moe status";
  }
}

uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

int moe_experts_init(moe_experts* d, const void* base, int32_t n_experts, int32_t hidden, int32_t inter) {
  if (!d || !base) return MOE_EINVAL;
  const uint64_t eb = moe_expert_bytes(hidden, inter);
  if (eb == 0 || n_experts < 1 || n_experts > kMaxExperts) return MOE_ESHAPE;
  d->abi_version = MOE_ABI_VERSION;
  d->layout = MOE_LAYOUT_GFX950_TILED_V1;
  d->n_experts = n_experts;
  d->hidden = hidden;
  d->inter = inter;
  d->flags = 0;
  d->expert_bytes = eb;
  d->base = base;
  return MOE_OK;
}

size_t moe_route_workspace_size(int32_t T, int32_t H, int32_t E) {
  if (T <= 0 || T > kMaxTokens || H <= 0 || H % 512 != 0 || H > MOE_MAX_DIM || E <= 0) return 0;
  return moe::route_ws_bytes(T, H, E);
}

int moe_route(const uint16_t* x, int32_t T, int32_t H, const float* w_router, const float* sel_bias,
              const int32_t* token_ids, const int32_t* hash_table, int32_t V, int32_t E, int32_t top_k,
              float route_scale, int32_t* ids, float* weights, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  if (top_k < 1 || top_k > kMaxTopK || E < top_k || E > kMaxRouteExperts) return MOE_ESHAPE;
  if (!(route_scale == route_scale)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!ids || !weights) return MOE_EINVAL;
  if (hash_table) {
    if (!token_ids || V <= 0) return MOE_EINVAL;
    return hip_status(moe::launch_route_hash(token_ids, T, hash_table, V, top_k, route_scale, ids, weights,
                                             as_stream(stream)));
  }
  if (!x || !w_router) return MOE_EINVAL;
  if (H <= 0 || H % 512 != 0 || H > MOE_MAX_DIM) return MOE_ESHAPE;
  if (!aligned(x, 16) || !aligned(w_router, 4)) return MOE_EALIGN;
  if (!ws) return MOE_EINVAL;
  if (!aligned(ws, 256)) return MOE_EALIGN;
  if (ws_bytes < moe_route_workspace_size(T, H, E)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_route_learned(x, T, H, w_router, sel_bias, E, top_k, route_scale, ids, weights, ws,
                                              as_stream(stream)));
}

size_t moe_dispatch_workspace_size(int32_t T, int32_t E, int32_t top_k) {
  if (T <= 0 || T > kMaxTokens || E <= 0 || E > kMaxExperts || top_k < 1 || top_k > kMaxTopK) return 0;
  return moe::dispatch_ws_bytes(T, E, top_k);
}

int moe_dispatch(const int32_t* ids, int32_t T, int32_t E, int32_t top_k, int32_t* offsets, int32_t* row_token,
                 int32_t* slot_row, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  if (top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxExperts) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ids || !offsets || !row_token || !slot_row || !ws) return MOE_EINVAL;
  if (!aligned(ws, 256)) return MOE_EALIGN;
  if (ws_bytes < moe_dispatch_workspace_size(T, E, top_k)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_dispatch(ids, T, E, top_k, offsets, row_token, slot_row, ws, as_stream(stream)));
}

int moe_dispatch_noalloc(const int32_t* ids, int32_t T, int32_t E, int32_t top_k, int32_t* offsets,
                         int32_t* row_token, int32_t* slot_row, void* stream) {
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  if (top_k < 1 || top_k > kMaxTopK || E < 1 || E > kMaxExperts) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ids || !offsets || !row_token || !slot_row) return MOE_EINVAL;
  if (moe::dispatch_ws_bytes(T, E, top_k) > MOE_DISPATCH_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  return hip_status(moe::launch_dispatch_noalloc(ids, T, E, top_k, offsets, row_token, slot_row, as_stream(stream)));
}

size_t moe_ffn_workspace_size(int32_t T, const moe_experts* experts, int32_t top_k) {
  if (T <= 0 || T > kMaxTokens || top_k < 1 || top_k > kMaxTopK || check_experts(experts) != MOE_OK) return 0;
  return moe::ffn_ws_bytes(T, experts->n_experts, experts->hidden, experts->inter, top_k,
                           (experts->flags & MOE_FFN_SPLIT_FP8) != 0, (experts->flags & MOE_ROUTED_AFFINE2) != 0);
}

namespace {

int ffn_call(const uint16_t* x, int32_t T, const moe_experts* experts, int32_t top_k, const int32_t* offsets,
             const int32_t* row_token, float clamp_limit, uint16_t* out_rows, void* ws, size_t ws_bytes, int32_t phase,
             void* stream) {
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  const int st = check_experts(experts);
  if (st != MOE_OK) return st;
  if (top_k < 1 || top_k > kMaxTopK) return MOE_ESHAPE;
  if (!(clamp_limit > 0.0f)) return MOE_EINVAL;
  if (phase < -1 || phase > 2) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !row_token || !out_rows || !ws) return MOE_EINVAL;
  if (!aligned(x, 16) || !aligned(out_rows, 16) || !aligned(ws, 256)) return MOE_EALIGN;
  if (ws_bytes < moe_ffn_workspace_size(T, experts, top_k)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_ffn(x, T, static_cast<const uint8_t*>(experts->base), experts->expert_bytes,
                                    experts->n_experts, experts->hidden, experts->inter, top_k, offsets, row_token,
                                    clamp_limit, out_rows, ws, phase, (experts->flags & MOE_FFN_SPLIT_FP8) != 0,
                                    (experts->flags & MOE_SHARED_MXFP8) != 0,
                                    (experts->flags & MOE_ROUTED_AFFINE2) != 0, as_stream(stream)));
}

}  // namespace

int moe_expert_ffn(const uint16_t* x, int32_t T, const moe_experts* experts, int32_t top_k, const int32_t* offsets,
                   const int32_t* row_token, float clamp_limit, uint16_t* out_rows, void* ws, size_t ws_bytes,
                   void* stream) {
  return ffn_call(x, T, experts, top_k, offsets, row_token, clamp_limit, out_rows, ws, ws_bytes, -1, stream);
}

int moe_expert_ffn_phase(const uint16_t* x, int32_t T, const moe_experts* experts, int32_t top_k,
                         const int32_t* offsets, const int32_t* row_token, float clamp_limit, uint16_t* out_rows,
                         void* ws, size_t ws_bytes, int32_t phase, void* stream) {
  return ffn_call(x, T, experts, top_k, offsets, row_token, clamp_limit, out_rows, ws, ws_bytes, phase, stream);
}

int moe_combine(const uint16_t* out_rows, const int32_t* slot_row, const float* weights, int32_t T, int32_t H,
                int32_t top_k, uint16_t* y, void* stream) {
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxTokens) return MOE_ESHAPE;
  if (top_k < 1 || top_k > kMaxTopK || H <= 0 || H % 8 != 0) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!out_rows || !slot_row || !weights || !y) return MOE_EINVAL;
  if (!aligned(out_rows, 16) || !aligned(y, 16)) return MOE_EALIGN;
  return hip_status(moe::launch_combine(out_rows, slot_row, weights, T, H, top_k, y, as_stream(stream)));
}

}  // extern "C"
