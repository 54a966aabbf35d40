// The layer forward's launch sequence and workspace layout, shared by the
// forward entry points (internal to the library, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// moe_forward workspace: routing outputs, dispatch indices, xp (fp32 only),
// yp, and one stage region shared in time by the router's partial logits,
// the dispatch counters, h and (with_split) the GEMMs' split-tile partials.
struct FwdLayout {
  size_t ids, w, offsets, sorted, inv, xp, yp, stage, total;
};
// with_split false: no region for the split-tile partials (the GEMMs then run
// their leftover tiles whole)
FwdLayout fwd_layout(int64_t T, int64_t H, int64_t E, int32_t k, int64_t F, moe_dtype dt,
                     bool with_split = true);

// Argument checks of a forward entry point, everything but the workspace.
moe_status check_forward(const void* x, const void* w_r, const float* router_bias,
                         const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                         int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                         moe_gating gating, const void* y, const int32_t* topk_ids_out,
                         const float* topk_w_out);

// The forward's launches on stream s into workspace ws of layout L (the
// caller has validated every argument; T > 0); split: the GEMMs may split
// leftover tiles along K (L must have been made with_split).
moe_status forward_body(const void* x, const void* w_r, const float* router_bias,
                        const void* w1, const void* w2, int64_t T, int64_t H, int64_t E,
                        int32_t top_k, int64_t F, moe_dtype dtype, moe_dtype router_dtype,
                        moe_gating gating, int32_t capacity, void* y, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, const FwdLayout& L, bool split,
                        hipStream_t s);

}  // namespace moe
