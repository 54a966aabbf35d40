// Internal host-side launchers of the MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

// Router work split: TPW expert tiles (of 16) per wave, EG expert groups,
// S splits of the H axis of KL elements each; logits padded to EP columns.
struct RoutePlan {
  int EP, TPW, EG, S, KL;
};
// wf32: W_r is fp32 while x is bf16 (an fp32 router for bf16 tokens)
RoutePlan plan_route(int T, int H, int E, bool bf16, bool wf32);
// enough for either router weight type
size_t route_ws_bytes(int T, int H, int E, bool bf16);
// softmax_all: gate weights are the top-k probabilities of the softmax over
// all E logits (not renormalised); otherwise the softmax of the k winners
hipError_t launch_route(const void* x, const void* w_r, const float* bias, int T, int H,
                        int E, int k, bool bf16, bool wf32, bool softmax_all, int32_t* ids,
                        float* w, void* ws, hipStream_t s);

size_t permute_ws_bytes(int R, int E);
// xp == nullptr: indices only (the rows are gathered later by the GEMM).
// capacity > 0: each expert keeps its first `capacity` pairs, the others get
// inv_pos = -1; capacity <= 0: dropless.
hipError_t launch_permute(const void* x, const int32_t* ids, int T, int H, int E, int k,
                          int capacity, size_t elem_bytes, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_pos, void* xp, void* ws,
                          hipStream_t s);

// Split-tile workspace of the bf16 grouped GEMM: fp32 partials of at most
// kMaxSlots pieces (written by one GEMM launch, summed by the next kernel on
// the stream; nothing in it needs clearing).
constexpr int kMaxSlots = 256;
size_t split_ws_bytes();
// A holds a_rows rows of K; with gather != nullptr, dispatched row p is row
// gather[p] of A (the dispatch fused into the GEMM's loads), else row p.
hipError_t launch_gemm_bf16(const void* A, const int* gather, int a_rows, const void* W,
                            void* C, const int* off, int E, int R, int K, int N, bool gelu,
                            void* split_ws, hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const float* W, float* C, const int* off, int E,
                           int R, int K, int N, int ldc, bool gelu, hipStream_t s);

hipError_t launch_combine(const void* yp, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, bool bf16, void* y, hipStream_t s);

}  // namespace moe
