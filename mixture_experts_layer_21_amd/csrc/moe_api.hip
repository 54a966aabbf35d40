// C ABI of the MoE layer forward and backward: host-side validation,
// workspace layouts and the launch sequences.  Every entry point validates all of its arguments
// before enqueueing anything, so an error return leaves the device untouched.
#include "moe.h"

#include <initializer_list>

#include "forward.h"
#include "launch.h"

namespace {

using moe::align_up;
using moe::check_forward;
using moe::forward_body;
using moe::fwd_layout;
using moe::FwdLayout;

constexpr int64_t kMaxE = 1024;
constexpr int32_t kMaxTopK = 16;
constexpr int64_t kIndexLimit = ((int64_t)1 << 31) - 64;

size_t elem_bytes(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }

moe_status check_dtype(moe_dtype dt) {
  return (dt == MOE_F32 || dt == MOE_BF16) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// Router weight type: the token type, or fp32 for bf16 tokens.
moe_status check_router(moe_dtype dt, moe_dtype router_dtype, moe_gating gating) {
  if (gating != MOE_GATE_TOPK_SOFTMAX && gating != MOE_GATE_SOFTMAX_TOPK)
    return MOE_ERR_INVALID_ARG;
  if (router_dtype == dt) return MOE_OK;
  if (dt == MOE_BF16 && router_dtype == MOE_F32) return MOE_OK;
  return MOE_ERR_UNSUPPORTED;
}

// Shape checks shared by the entry points.  T may be 0 (nothing to do).
moe_status check_shape(int64_t T, int64_t H, int64_t E, int32_t top_k, int64_t F,
                       moe_dtype dt) {
  if (T < 0 || H <= 0 || E <= 0 || F <= 0) return MOE_ERR_INVALID_ARG;
  if (top_k < 1 || top_k > E) return MOE_ERR_INVALID_ARG;
  if (check_dtype(dt) != MOE_OK) return MOE_ERR_UNSUPPORTED;
  if (H % 8 != 0 || F % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (E > kMaxE || top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  const int64_t wide = H > F ? H : F;
  if (T * top_k >= kIndexLimit / wide) return MOE_ERR_UNSUPPORTED;
  if (H * F >= kIndexLimit) return MOE_ERR_UNSUPPORTED;   // one expert's W slab < 4 GiB
  return MOE_OK;
}

// expert FFN workspace: h[R,F], then (bf16) the GEMM's split-tile partials
size_t ffn_ws_bytes(int64_t R, int64_t F, moe_dtype dt) {
  size_t b = align_up((size_t)R * F * elem_bytes(dt));
  if (dt == MOE_BF16) b += moe::split_ws_bytes();
  return b;
}

// expert FFN over rows gathered from x: the FFN workspace, then (fp32, whose
// GEMM reads contiguous rows) the gathered rows xp[R,H]
size_t ffn_gather_ws_bytes(int64_t R, int64_t H, int64_t F, moe_dtype dt) {
  size_t b = ffn_ws_bytes(R, F, dt);
  if (dt == MOE_F32) b += align_up((size_t)R * H * 4);
  return b;
}

moe_status launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// Alignment the kernels rely on: tensors in the layer's dtype and the
// workspaces are read and written with 16-byte vector accesses, int32 and
// fp32 index/weight arrays with 4-byte accesses.  Null pointers pass (the
// null checks are separate).
bool aligned(std::initializer_list<const void*> a16, std::initializer_list<const void*> a4) {
  for (const void* p : a16)
    if ((uintptr_t)p & 15u) return false;
  for (const void* p : a4)
    if ((uintptr_t)p & 3u) return false;
  return true;
}

// Expert FFN.  The first GEMM reads its token rows from xp (a_rows = R rows,
// gather == nullptr) or straight from x through gather = sorted_token
// (a_rows = T rows); h[R,F] takes GELU(z) and, when z != nullptr, z[R,F] the
// pre-activation; split is the bf16 GEMM's split-tile workspace.
moe_status run_ffn(const void* xp, const int32_t* gather, int64_t a_rows, const int32_t* off,
                   const void* w1, const void* w2, int64_t R, int64_t H, int64_t E, int64_t F,
                   moe_dtype dt, void* yp, void* h, void* z, void* split, hipStream_t s) {
  if (R == 0) return MOE_OK;
  hipError_t err;
  if (dt == MOE_BF16) {
    err = moe::launch_gemm_bf16(xp, gather, (int)a_rows, w1, false, h, off, (int)E, (int)R,
                                (int)H, (int)F, moe::EP_GELU, nullptr, z, split, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_bf16(h, nullptr, (int)R, w2, false, yp, off, (int)E, (int)R,
                                  (int)F, (int)H, moe::EP_PLAIN, nullptr, nullptr, split, s);
  } else {
    err = moe::launch_gemm_f32((const float*)xp, (const float*)w1, (float*)h, off, (int)E,
                               (int)R, (int)H, (int)F, (int)F, true, (float*)z, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_f32((const float*)h, (const float*)w2, (float*)yp, off, (int)E,
                                 (int)R, (int)F, (int)H, (int)H, false, nullptr, s);
  }
  return launch_status(err);
}

// Expert FFN backward over dispatched rows: dz = (dyp W2^T) * GELU'(z),
// dW2 = h^T dyp, dxp = dz W1^T, dW1 = xp^T dz (dz[R,F] in `dz`; split is the
// bf16 GEMMs' split-tile workspace).  dxp may be dyp's buffer: dyp's last
// reader (dW2) runs before dxp is written.  With R == 0 only the (zero)
// weight gradients are written.
moe_status run_ffn_bwd(const void* dyp, const void* xp, const int32_t* off, const void* z,
                       const void* h, const void* w1, const void* w2, int64_t R, int64_t H,
                       int64_t E, int64_t F, moe_dtype dt, void* dxp, void* dw1, void* dw2,
                       void* dz, void* split, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (dt == MOE_BF16) {
    if (R > 0)
      err = moe::launch_gemm_bf16(dyp, nullptr, (int)R, w2, true, dz, off, (int)E, (int)R,
                                  (int)H, (int)F, moe::EP_DGELU, z, nullptr, split, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_bf16_wgrad(h, dyp, dw2, off, (int)E, (int)R, (int)F, (int)H, s);
    if (err == hipSuccess && R > 0)
      err = moe::launch_gemm_bf16(dz, nullptr, (int)R, w1, true, dxp, off, (int)E, (int)R,
                                  (int)F, (int)H, moe::EP_PLAIN, nullptr, nullptr, split, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_bf16_wgrad(xp, dz, dw1, off, (int)E, (int)R, (int)H, (int)F, s);
  } else {
    if (R > 0)
      err = moe::launch_gemm_f32_nt((const float*)dyp, (const float*)w2, (float*)dz, off, (int)E,
                                    (int)R, (int)H, (int)F, (const float*)z, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_f32_wgrad((const float*)h, (const float*)dyp, (float*)dw2, off,
                                       (int)E, (int)R, (int)F, (int)H, s);
    if (err == hipSuccess && R > 0)
      err = moe::launch_gemm_f32_nt((const float*)dz, (const float*)w1, (float*)dxp, off,
                                    (int)E, (int)R, (int)F, (int)H, nullptr, s);
    if (err == hipSuccess)
      err = moe::launch_gemm_f32_wgrad((const float*)xp, (const float*)dz, (float*)dw1, off,
                                       (int)E, (int)R, (int)H, (int)F, s);
  }
  return launch_status(err);
}

// h[R,F] then the split workspace, inside an expert-FFN workspace
void* ffn_split(void* ws, int64_t R, int64_t F, moe_dtype dt) {
  return (char*)ws + align_up((size_t)R * F * elem_bytes(dt));
}

// State a training forward keeps for the backward (caller-owned, opaque):
// dispatch indices, the fp32 logits, z and h of the first expert GEMM and
// the expert outputs yp.
struct SavedLayout {
  size_t offsets, sorted, inv, logits, z, h, yp, total;
};

SavedLayout saved_layout(int64_t T, int64_t H, int64_t E, int32_t k, int64_t F, moe_dtype dt) {
  const int64_t R = T * k;
  const size_t es = elem_bytes(dt);
  SavedLayout L;
  size_t o = 0;
  L.offsets = o; o += align_up((size_t)(E + 1) * 4);
  L.sorted = o;  o += align_up((size_t)R * 4);
  L.inv = o;     o += align_up((size_t)R * 4);
  L.logits = o;  o += align_up((size_t)T * E * 4);
  L.z = o;       o += align_up((size_t)R * F * es);
  L.h = o;       o += align_up((size_t)R * F * es);
  L.yp = o;      o += align_up((size_t)R * H * es);
  L.total = o;
  return L;
}

// moe_backward workspace: gate-weight and logit gradients, dyp (later dxp),
// dz, the re-gathered token rows xp, and one region shared in time by the
// router weight gradient's partials and the GEMMs' split-tile partials.
struct BwdLayout {
  size_t dw, dl, dlp, dlk, dyp, dz, xp, wrt, stage, total;
};

BwdLayout bwd_layout(int64_t T, int64_t H, int64_t E, int32_t k, int64_t F, moe_dtype dt) {
  const int64_t R = T * k;
  const size_t es = elem_bytes(dt);
  BwdLayout L;
  size_t o = 0;
  L.dw = o;    o += align_up((size_t)R * 4);
  L.dl = o;    o += align_up((size_t)T * E * 4);
  L.dlp = o;   o += align_up(moe::router_planes_bytes((int)T, (int)E));
  L.dlk = o;   o += align_up((size_t)R * 4);
  L.dyp = o;   o += align_up((size_t)R * H * es);
  L.dz = o;    o += align_up((size_t)R * F * es);
  L.xp = o;    o += align_up((size_t)R * H * es);
  L.wrt = o;   o += align_up((size_t)E * H * 4);      // W_r^T (fp32 at most)
  L.stage = o;
  size_t st = moe::router_wgrad_ws_bytes((int)T, (int)H, (int)E);
  if (dt == MOE_BF16) st = std::max(st, moe::split_ws_bytes());
  L.total = o + st;
  return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported dtype or size";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: HIP launch failed";
    default: return "MOE_ERR_UNKNOWN: unknown status";
  }
}

moe_status moe_workspace_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k, int64_t F,
                               moe_dtype dtype, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  *bytes = fwd_layout(T, H, E, top_k, F, dtype).total;
  return MOE_OK;
}

moe_status moe_stage_workspace_bytes(moe_stage stage, int64_t T, int64_t H, int64_t E,
                                     int32_t top_k, int64_t F, moe_dtype dtype,
                                     size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  switch (stage) {
    case MOE_STAGE_ROUTE:
      *bytes = moe::route_ws_bytes((int)T, (int)H, (int)E, dtype == MOE_BF16);
      return MOE_OK;
    case MOE_STAGE_PERMUTE:
      *bytes = moe::permute_ws_bytes((int)(T * top_k), (int)E);
      return MOE_OK;
    case MOE_STAGE_EXPERT_FFN:
      *bytes = ffn_ws_bytes(T * top_k, F, dtype);
      return MOE_OK;
    case MOE_STAGE_COMBINE:
      *bytes = 0;
      return MOE_OK;
    case MOE_STAGE_FORWARD:
      *bytes = fwd_layout(T, H, E, top_k, F, dtype).total;
      return MOE_OK;
    case MOE_STAGE_EXPERT_FFN_BACKWARD:
      *bytes = ffn_ws_bytes(T * top_k, F, dtype);
      return MOE_OK;
    case MOE_STAGE_EXPERT_FFN_GATHER:
      *bytes = ffn_gather_ws_bytes(T * top_k, H, F, dtype);
      return MOE_OK;
    default:
      return MOE_ERR_INVALID_ARG;
  }
}

moe_status moe_expert_capacity(int64_t T, int32_t top_k, int64_t E, int64_t factor_num,
                               int64_t factor_den, int32_t* capacity) {
  if (!capacity || T < 0 || top_k < 1 || E < 1 || factor_den <= 0) return MOE_ERR_INVALID_ARG;
  if (factor_num <= 0) {
    *capacity = 0;
    return MOE_OK;
  }
  // ceil(num * T * k / (den * E)) in integers; the operands stay far below
  // 2^63 for the sizes the other entry points accept
  if (factor_num > ((int64_t)1 << 20) || factor_den > ((int64_t)1 << 20) ||
      T > ((int64_t)1 << 31) || E > ((int64_t)1 << 20))
    return MOE_ERR_UNSUPPORTED;
  const int64_t num = factor_num * T * top_k, den = factor_den * E;
  const int64_t c = (num + den - 1) / den;
  if (c > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  *capacity = (int32_t)c;
  return MOE_OK;
}

moe_status moe_route_ex(const void* x, const void* w_r, const float* router_bias, int64_t T,
                        int64_t H, int64_t E, int32_t top_k, moe_dtype dtype,
                        moe_dtype router_dtype, moe_gating gating, int32_t* topk_ids,
                        float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(T, H, E, top_k, 8, dtype);
  if (st != MOE_OK) return st;
  st = check_router(dtype, router_dtype, gating);
  if (st != MOE_OK) return st;
  if (!x || !w_r || !topk_ids || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned({x, w_r, ws}, {router_bias, topk_ids, topk_w})) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe::route_ws_bytes((int)T, (int)H, (int)E, dtype == MOE_BF16))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  return launch_status(moe::launch_route(x, w_r, router_bias, (int)T, (int)H, (int)E, top_k,
                                         dtype == MOE_BF16, router_dtype != dtype,
                                         gating == MOE_GATE_SOFTMAX_TOPK, topk_ids, topk_w,
                                         nullptr, ws, (hipStream_t)stream));
}

moe_status moe_route(const void* x, const void* w_r, const float* router_bias, int64_t T,
                     int64_t H, int64_t E, int32_t top_k, moe_dtype dtype, int32_t* topk_ids,
                     float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  return moe_route_ex(x, w_r, router_bias, T, H, E, top_k, dtype, dtype, MOE_GATE_TOPK_SOFTMAX,
                      topk_ids, topk_w, ws, ws_bytes, stream);
}

moe_status moe_permute_ex(const void* x, const int32_t* topk_ids, int64_t T, int64_t H,
                          int64_t E, int32_t top_k, moe_dtype dtype, int32_t capacity,
                          int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_pos,
                          void* xp, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_shape(T, H, E, top_k, 8, dtype);
  if (st != MOE_OK) return st;
  // (xp may be NULL: indices only)
  if (!x || !topk_ids || !expert_offsets || !sorted_token || !inv_pos || !ws)
    return MOE_ERR_INVALID_ARG;
  if (!aligned({x, xp, ws}, {topk_ids, expert_offsets, sorted_token, inv_pos}))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe::permute_ws_bytes((int)(T * top_k), (int)E)) return MOE_ERR_INVALID_ARG;
  return launch_status(moe::launch_permute(x, topk_ids, (int)T, (int)H, (int)E, top_k, capacity,
                                           elem_bytes(dtype), expert_offsets, sorted_token,
                                           inv_pos, xp, ws, (hipStream_t)stream));
}

moe_status moe_permute(const void* x, const int32_t* topk_ids, int64_t T, int64_t H, int64_t E,
                       int32_t top_k, moe_dtype dtype, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* inv_pos, void* xp, void* ws,
                       size_t ws_bytes, void* stream) {
  return moe_permute_ex(x, topk_ids, T, H, E, top_k, dtype, 0, expert_offsets, sorted_token,
                        inv_pos, xp, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn(const void* xp, const int32_t* expert_offsets, const void* w1,
                          const void* w2, int64_t R, int64_t H, int64_t E, int64_t F,
                          moe_dtype dtype, void* yp, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_shape(R, H, E, 1, F, dtype);
  if (st != MOE_OK) return st;
  if (!xp || !expert_offsets || !w1 || !w2 || !yp || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned({xp, w1, w2, yp, ws}, {expert_offsets})) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_ws_bytes(R, F, dtype)) return MOE_ERR_INVALID_ARG;
  return run_ffn(xp, nullptr, R, expert_offsets, w1, w2, R, H, E, F, dtype, yp, ws, nullptr,
                 ffn_split(ws, R, F, dtype), (hipStream_t)stream);
}

moe_status moe_expert_ffn_gather(const void* x, int64_t T, const int32_t* sorted_token,
                                 const int32_t* expert_offsets, const void* w1, const void* w2,
                                 int64_t R, int64_t H, int64_t E, int64_t F, moe_dtype dtype,
                                 void* yp, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_shape(R, H, E, 1, F, dtype);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (T >= kIndexLimit / H) return MOE_ERR_UNSUPPORTED;
  if (!x || !sorted_token || !expert_offsets || !w1 || !w2 || !yp || !ws)
    return MOE_ERR_INVALID_ARG;
  if (!aligned({x, w1, w2, yp, ws}, {sorted_token, expert_offsets})) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_gather_ws_bytes(R, H, F, dtype)) return MOE_ERR_INVALID_ARG;
  if (R == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  void* split = ffn_split(ws, R, F, dtype);
  if (dtype == MOE_BF16)
    return run_ffn(x, sorted_token, T, expert_offsets, w1, w2, R, H, E, F, dtype, yp, ws,
                   nullptr, split, s);
  void* xp = (char*)ws + ffn_ws_bytes(R, F, dtype);
  if (moe::launch_gather_rows(x, sorted_token, expert_offsets, (int)E, (int)R, (int)T, (int)H,
                              elem_bytes(dtype), xp, s) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return run_ffn(xp, nullptr, R, expert_offsets, w1, w2, R, H, E, F, dtype, yp, ws, nullptr,
                 split, s);
}

moe_status moe_expert_ffn_backward(const void* dyp, const void* xp,
                                   const int32_t* expert_offsets, const void* z, const void* h,
                                   const void* w1, const void* w2, int64_t R, int64_t H,
                                   int64_t E, int64_t F, moe_dtype dtype, void* dxp, void* dw1,
                                   void* dw2, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_shape(R, H, E, 1, F, dtype);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !w1 || !w2 || !dw1 || !dw2 || !ws) return MOE_ERR_INVALID_ARG;
  if (R > 0 && (!dyp || !xp || !z || !h || !dxp)) return MOE_ERR_INVALID_ARG;
  if (!aligned({dyp, xp, z, h, w1, w2, dxp, dw1, dw2, ws}, {expert_offsets}))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ffn_ws_bytes(R, F, dtype)) return MOE_ERR_INVALID_ARG;
  return run_ffn_bwd(dyp, xp, expert_offsets, z, h, w1, w2, R, H, E, F, dtype, dxp, dw1, dw2, ws,
                     ffn_split(ws, R, F, dtype), (hipStream_t)stream);
}

moe_status moe_combine(const void* yp, const int32_t* inv_pos, const float* topk_w, int64_t T,
                       int64_t H, int32_t top_k, moe_dtype dtype, void* y, void* stream) {
  const moe_status st = check_shape(T, H, top_k, top_k, 8, dtype);
  if (st != MOE_OK) return st;
  if (!yp || !inv_pos || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned({yp, y}, {inv_pos, topk_w})) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  return launch_status(moe::launch_combine(yp, inv_pos, topk_w, (int)T, (int)H, top_k,
                                           dtype == MOE_BF16, y, (hipStream_t)stream));
}

}  // extern "C"

namespace moe {

FwdLayout fwd_layout(int64_t T, int64_t H, int64_t E, int32_t k, int64_t F, moe_dtype dt,
                     bool with_split) {
  const int64_t R = T * k;
  const size_t es = elem_bytes(dt);
  FwdLayout L;
  size_t o = 0;
  L.ids = o;     o += align_up((size_t)R * 4);
  L.w = o;       o += align_up((size_t)R * 4);
  L.offsets = o; o += align_up((size_t)(E + 1) * 4);
  L.sorted = o;  o += align_up((size_t)R * 4);
  L.inv = o;     o += align_up((size_t)R * 4);
  L.xp = o;      // fp32 only: the bf16 GEMM gathers token rows from x itself
  if (dt == MOE_F32) o += align_up((size_t)R * H * es);
  L.yp = o;      o += align_up((size_t)R * H * es);
  L.stage = o;
  size_t st = moe::route_ws_bytes((int)T, (int)H, (int)E, dt == MOE_BF16);
  st = std::max(st, moe::permute_ws_bytes((int)R, (int)E));
  st = std::max(st, with_split ? ffn_ws_bytes(R, F, dt) : align_up((size_t)R * F * elem_bytes(dt)));
  L.total = o + st;
  return L;
}


// Dispatched rows (T * top_k) up to which the forward adds the second GEMM's
// split tiles and combines in one launch (launch_reduce_combine).  Against
// the split reduce and the combine pass it saved 2-3% at 1-16 tokens of
// top-2 and 1-2% at 32-64 (up to 128 rows), and lost 2-3% at 256 and
// 2048 tokens and at 512 rows of 64 tokens x 8 slots.
constexpr int64_t kFusedCombineMaxRows = 128;

// The forward's launches into a workspace of layout L (validated by the
// caller); split: the GEMMs may split leftover tiles (L has their region).
moe_status forward_body(const void* x, const void* w_r, const float* router_bias,
                        const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                        int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                        moe_gating gating, int32_t capacity, void* y, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, const FwdLayout& L, bool split,
                        hipStream_t s) {
  char* base = (char*)ws;
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(base + L.ids);
  float* w = topk_w_out ? topk_w_out : (float*)(base + L.w);
  int32_t* off = (int32_t*)(base + L.offsets);
  int32_t* sorted = (int32_t*)(base + L.sorted);
  int32_t* inv = (int32_t*)(base + L.inv);
  void* xp = base + L.xp;
  void* yp = base + L.yp;
  void* stage = base + L.stage;
  const bool bf16 = dtype == MOE_BF16;
  const int64_t R = T * top_k;

  // a decode-sized bf16 batch: the router's one workgroup also dispatches
  const bool rd = bf16 && capacity <= 0 &&
                  moe::route_dispatches((int)T, (int)H, (int)E, bf16, router_dtype != dtype);
  hipError_t err = moe::launch_route(x, w_r, router_bias, (int)T, (int)H, (int)E, top_k, bf16,
                                     router_dtype != dtype, gating == MOE_GATE_SOFTMAX_TOPK,
                                     ids, w, nullptr, stage, s, rd ? off : nullptr,
                                     rd ? sorted : nullptr, rd ? inv : nullptr);
  if (err != hipSuccess) return MOE_ERR_LAUNCH;
  // bf16: the first expert GEMM gathers the token rows from x itself, so the
  // dispatch only builds the indices; fp32 copies the rows into xp.  With a
  // capacity fewer than R rows are kept; the GEMMs take their row counts from
  // the offsets, so R only bounds the grid.
  if (!rd) {
    err = moe::launch_permute(x, ids, (int)T, (int)H, (int)E, top_k, capacity,
                              elem_bytes(dtype), off, sorted, inv, bf16 ? nullptr : xp, stage, s);
    if (err != hipSuccess) return MOE_ERR_LAUNCH;
  }
  void* split_ws = split ? ffn_split(stage, R, F, dtype) : nullptr;
  if (bf16 && top_k == 1 && capacity <= 0) {
    // Top-1 and dropless: every token owns exactly one dispatched row, so
    // the second GEMM's epilogue writes it, weighted, straight to the
    // token's row of y (the combine fused in; no yp, no cross-workgroup
    // sums, the same bits as the separate pass)
    hipError_t e2 = moe::launch_gemm_bf16(x, sorted, (int)T, w1, false, stage, off, (int)E,
                                          (int)R, (int)H, (int)F, moe::EP_GELU, nullptr,
                                          nullptr, split_ws, s);
    if (e2 == hipSuccess)
      e2 = moe::launch_gemm_bf16_scatter(stage, w2, y, off, (int)E, (int)R, (int)F, (int)H,
                                         sorted, w, split_ws, s);
    return launch_status(e2);
  }
  if (bf16 && split_ws != nullptr && R <= kFusedCombineMaxRows) {
    // A decode-sized batch: the second GEMM leaves its split tiles' partials
    // and one launch adds them up and combines (no separate reduce and
    // combine launches; y is bit for bit theirs)
    hipError_t e2 = moe::launch_gemm_bf16(x, sorted, (int)T, w1, false, stage, off, (int)E,
                                          (int)R, (int)H, (int)F, moe::EP_GELU, nullptr,
                                          nullptr, split_ws, s);
    if (e2 == hipSuccess)
      e2 = moe::launch_gemm_bf16(stage, nullptr, (int)R, w2, false, yp, off, (int)E, (int)R,
                                 (int)F, (int)H, moe::EP_PLAIN, nullptr, nullptr, split_ws, s,
                                 true);
    if (e2 == hipSuccess)
      e2 = moe::launch_reduce_combine(yp, split_ws, off, ids, inv, w, y, (int)T, top_k, (int)E,
                                      (int)R, (int)F, (int)H, s);
    return launch_status(e2);
  }
  const moe_status fs =
      bf16 ? run_ffn(x, sorted, T, off, w1, w2, R, H, E, F, dtype, yp, stage, nullptr, split_ws, s)
           : run_ffn(xp, nullptr, R, off, w1, w2, R, H, E, F, dtype, yp, stage, nullptr, split_ws,
                     s);
  if (fs != MOE_OK) return fs;
  return launch_status(moe::launch_combine(yp, inv, w, (int)T, (int)H, top_k, bf16, y, s));
}

// Argument checks of the forward entry points (everything but the workspace).
moe_status check_forward(const void* x, const void* w_r, const float* router_bias,
                         const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                         int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                         moe_gating gating, const void* y, const int32_t* topk_ids_out,
                         const float* topk_w_out) {
  moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  st = check_router(dtype, router_dtype, gating);
  if (st != MOE_OK) return st;
  if (!x || !w_r || !w1 || !w2 || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned({x, w_r, w1, w2, y}, {router_bias, topk_ids_out, topk_w_out}))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status moe_forward_ex(const void* x, const void* w_r, const float* router_bias,
                          const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                          int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                          moe_gating gating, int32_t capacity, void* y, int32_t* topk_ids_out,
                          float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = check_forward(x, w_r, router_bias, w1, w2, T, H, E, top_k, F, dtype,
                                      router_dtype, gating, y, topk_ids_out, topk_w_out);
  if (st != MOE_OK) return st;
  if (!ws || !aligned({ws}, {})) return MOE_ERR_INVALID_ARG;
  const FwdLayout L = fwd_layout(T, H, E, top_k, F, dtype);
  if (ws_bytes < L.total) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  return forward_body(x, w_r, router_bias, w1, w2, T, H, E, top_k, F, dtype, router_dtype,
                      gating, capacity, y, topk_ids_out, topk_w_out, ws, L, true,
                      (hipStream_t)stream);
}

moe_status moe_forward(const void* x, const void* w_r, const float* router_bias, const void* w1,
                       const void* w2, int64_t T, int64_t H, int64_t E, int32_t top_k,
                       int64_t F, moe_dtype dtype, void* y, int32_t* topk_ids_out,
                       float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  return moe_forward_ex(x, w_r, router_bias, w1, w2, T, H, E, top_k, F, dtype, dtype,
                        MOE_GATE_TOPK_SOFTMAX, 0, y, topk_ids_out, topk_w_out, ws, ws_bytes,
                        stream);
}

moe_status moe_saved_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k, int64_t F,
                           moe_dtype dtype, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  *bytes = saved_layout(T, H, E, top_k, F, dtype).total;
  return MOE_OK;
}

moe_status moe_backward_workspace_bytes(int64_t T, int64_t H, int64_t E, int32_t top_k,
                                        int64_t F, moe_dtype dtype, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  *bytes = bwd_layout(T, H, E, top_k, F, dtype).total;
  return MOE_OK;
}

moe_status moe_forward_train(const void* x, const void* w_r, const float* router_bias,
                             const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                             int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                             moe_gating gating, int32_t capacity, void* y, int32_t* topk_ids,
                             float* topk_w, void* saved, size_t saved_bytes, void* ws,
                             size_t ws_bytes, void* stream) {
  moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  st = check_router(dtype, router_dtype, gating);
  if (st != MOE_OK) return st;
  // (buffers of T rows are empty, and may be NULL, when T == 0)
  if (!w_r || !w1 || !w2 || !saved || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !y || !topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (!aligned({x, w_r, w1, w2, y, saved, ws}, {router_bias, topk_ids, topk_w}))
    return MOE_ERR_INVALID_ARG;
  const FwdLayout L = fwd_layout(T, H, E, top_k, F, dtype);
  const SavedLayout V = saved_layout(T, H, E, top_k, F, dtype);
  if (ws_bytes < L.total || saved_bytes < V.total) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  char* sv = (char*)saved;
  int32_t* off = (int32_t*)(sv + V.offsets);
  int32_t* sorted = (int32_t*)(sv + V.sorted);
  int32_t* inv = (int32_t*)(sv + V.inv);
  float* logits = (float*)(sv + V.logits);
  void* xp = base + L.xp;
  void* stage = base + L.stage;
  const bool bf16 = dtype == MOE_BF16;
  const int64_t R = T * top_k;

  const bool rd = bf16 && capacity <= 0 &&
                  moe::route_dispatches((int)T, (int)H, (int)E, bf16, router_dtype != dtype);
  hipError_t err = moe::launch_route(x, w_r, router_bias, (int)T, (int)H, (int)E, top_k, bf16,
                                     router_dtype != dtype, gating == MOE_GATE_SOFTMAX_TOPK,
                                     topk_ids, topk_w, logits, stage, s, rd ? off : nullptr,
                                     rd ? sorted : nullptr, rd ? inv : nullptr);
  if (err != hipSuccess) return MOE_ERR_LAUNCH;
  if (!rd) {
    err = moe::launch_permute(x, topk_ids, (int)T, (int)H, (int)E, top_k, capacity,
                              elem_bytes(dtype), off, sorted, inv, bf16 ? nullptr : xp, stage, s);
    if (err != hipSuccess) return MOE_ERR_LAUNCH;
  }
  void* h = sv + V.h;
  void* z = sv + V.z;
  void* yp = sv + V.yp;
  const moe_status fs =
      bf16 ? run_ffn(x, sorted, T, off, w1, w2, R, H, E, F, dtype, yp, h, z, stage, s)
           : run_ffn(xp, nullptr, R, off, w1, w2, R, H, E, F, dtype, yp, h, z, stage, s);
  if (fs != MOE_OK) return fs;
  return launch_status(moe::launch_combine(yp, inv, topk_w, (int)T, (int)H, top_k, bf16, y, s));
}

moe_status moe_backward(const void* dy, const void* x, const void* w_r, const void* w1,
                        const void* w2, int64_t T, int64_t H, int64_t E, int32_t top_k,
                        int64_t F, moe_dtype dtype, moe_dtype router_dtype, moe_gating gating,
                        const int32_t* topk_ids, const float* topk_w, const void* saved,
                        size_t saved_bytes, void* dx, void* dw_r, float* db_r, void* dw1,
                        void* dw2, float* dtopk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(T, H, E, top_k, F, dtype);
  if (st != MOE_OK) return st;
  st = check_router(dtype, router_dtype, gating);
  if (st != MOE_OK) return st;
  // (buffers of T rows are empty, and may be NULL, when T == 0)
  if (!w_r || !w1 || !w2 || !saved || !dw_r || !dw1 || !dw2 || !ws) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!dy || !x || !topk_ids || !topk_w || !dx)) return MOE_ERR_INVALID_ARG;
  if (!aligned({dy, x, w_r, w1, w2, saved, dx, dw_r, dw1, dw2, ws},
               {topk_ids, topk_w, db_r, dtopk_w}))
    return MOE_ERR_INVALID_ARG;
  const SavedLayout V = saved_layout(T, H, E, top_k, F, dtype);
  const BwdLayout L = bwd_layout(T, H, E, top_k, F, dtype);
  if (saved_bytes < V.total || ws_bytes < L.total) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dtype == MOE_BF16;
  const bool w_bf16 = router_dtype == MOE_BF16;
  const int64_t R = T * top_k;
  const char* sv = (const char*)saved;
  const int32_t* off = (const int32_t*)(sv + V.offsets);
  const int32_t* sorted = (const int32_t*)(sv + V.sorted);
  const int32_t* inv = (const int32_t*)(sv + V.inv);
  const float* logits = (const float*)(sv + V.logits);
  const void* z = sv + V.z;
  const void* h = sv + V.h;
  const void* yp = sv + V.yp;
  char* base = (char*)ws;
  float* dw = dtopk_w ? dtopk_w : (float*)(base + L.dw);
  float* dl = (float*)(base + L.dl);
  uint16_t* dlp = bf16 ? (uint16_t*)(base + L.dlp) : nullptr;   // (for bf16 tokens only)
  const bool sparse = gating == MOE_GATE_TOPK_SOFTMAX;   // dl zero outside the k selected experts
  float* dlk = sparse ? (float*)(base + L.dlk) : nullptr;
  void* dyp = base + L.dyp;
  void* dxp = base + L.dyp;      // dyp's last reader (dW2) runs before dxp is written
  void* dz = base + L.dz;
  void* xp = base + L.xp;
  void* stage = base + L.stage;
  hipError_t err;
  // combine and gating
  err = moe::launch_combine_bwd(dy, yp, inv, topk_w, (int)T, (int)H, top_k, bf16, dw, dyp, s);
  if (err == hipSuccess)
    err = moe::launch_router_bwd(logits, topk_ids, topk_w, dw, (int)T, (int)E, top_k,
                                 gating == MOE_GATE_SOFTMAX_TOPK, dl, dlp, dlk, s);
  if (err == hipSuccess)
    err = moe::launch_router_wgrad(x, dl, dlp, (int)T, (int)H, (int)E, bf16, w_bf16, dw_r, db_r,
                                   stage, s);
  if (err != hipSuccess) return MOE_ERR_LAUNCH;
  if (T == 0) {
    // no rows (and no dispatch state): every expert's weight gradient is zero
    const size_t wbytes = (size_t)E * H * F * elem_bytes(dtype);
    err = moe::launch_fill_zero(dw1, wbytes, s);
    if (err == hipSuccess) err = moe::launch_fill_zero(dw2, wbytes, s);
    return launch_status(err);
  }
  // experts, over the token rows re-gathered into xp
  err = moe::launch_gather_rows(x, sorted, off, (int)E, (int)R, (int)T, (int)H, elem_bytes(dtype),
                                xp, s);
  if (err != hipSuccess) return MOE_ERR_LAUNCH;
  const moe_status fs = run_ffn_bwd(dyp, xp, off, z, h, w1, w2, R, H, E, F, dtype, dxp, dw1,
                                    dw2, dz, stage, s);
  if (fs != MOE_OK) return fs;
  return launch_status(moe::launch_dx_finish(dxp, inv, topk_ids, dl, dlk, w_r, (int)T, (int)H,
                                             (int)E, top_k, bf16, w_bf16, base + L.wrt, dx, s));
}

}  // extern "C"
