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
// all E logits (not renormalised); otherwise the softmax of the k winners.
// logits != nullptr: the fp32 logits [T,E] (bias included) are kept there.
// doff != nullptr (only where route_dispatches): the router's one workgroup
// also does the dropless dispatch of the pairs (expert offsets doff[E+1],
// sorted_token, inv_pos), as launch_permute with xp == nullptr would.
hipError_t launch_route(const void* x, const void* w_r, const float* bias, int T, int H,
                        int E, int k, bool bf16, bool wf32, bool softmax_all, int32_t* ids,
                        float* w, float* logits, void* ws, hipStream_t s,
                        int32_t* doff = nullptr, int32_t* dsorted = nullptr,
                        int32_t* dinv = nullptr);
// A bf16 routing of a few tokens (16 with E <= 16 on the one-launch router,
// else 4), whose selection kernel (one workgroup) can take the dispatch
// along (see launch_route).
bool route_dispatches(int T, int H, int E, bool bf16, bool wf32);

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
// GEMM epilogues: C = acc, GELU(acc), or acc * GELU'(z) with z read from an
// [R][N] matrix at the place C is written; EP_SCATTER (launch_gemm_bf16_scatter
// only): row p of the product, rounded to bf16 and scaled by row_w[scatter[p]],
// becomes row scatter[p] of C.
enum Epilogue { EP_PLAIN = 0, EP_GELU = 1, EP_DGELU = 2, EP_SCATTER = 3 };
// C[rows_e] = epilogue(A[rows_e] . B_e) for every expert e.  A holds a_rows
// rows of K; with gather != nullptr, dispatched row p is row gather[p] of A
// (the dispatch fused into the GEMM's loads), else row p.  B_e is W[e] as
// [K][N] (w_nk false) or its transpose, W[e] stored [N][K] (w_nk true).
// zout != nullptr: the accumulators are also stored there before the
// epilogue (the pre-activation a training forward keeps).  split_ws ==
// nullptr: no tile is split along K (the leftover tiles run whole).
// defer_reduce: the split tiles' partials stay in split_ws for
// launch_reduce_combine (no split reduce launch, their rows of C unwritten).
hipError_t launch_gemm_bf16(const void* A, const int* gather, int a_rows, const void* W,
                            bool w_nk, void* C, const int* off, int E, int R, int K, int N,
                            int ep, const void* aux, void* zout, void* split_ws,
                            hipStream_t s, bool defer_reduce = false);
// After launch_gemm_bf16(..., defer_reduce = true) of the second expert GEMM
// (EP_PLAIN, C = yp [R][N], the same off, E, R, K, N and split_ws): the
// combine y[t] = sum_j w[t,j] yp[inv_pos[t,j]] in slot order, each row of a
// split tile summed from its partials and rounded to bf16 first, as the
// split reduce and launch_combine would give (bf16; one workgroup per token
// and 256 columns: for decode-sized batches of up to 128 rows).
hipError_t launch_reduce_combine(const void* yp, void* split_ws, const int* off,
                                 const int32_t* ids, const int32_t* inv_pos, const float* w,
                                 void* y, int T, int k, int E, int R, int K, int N,
                                 hipStream_t s);
// The second expert GEMM with the combine of a top-1 layer in its epilogue:
// product row p (A's row p, expert e's W[K][N]) is rounded to bf16, scaled by
// row_w[scatter[p]] in fp32 (an fma with a zero addend) and rounded again into
// row scatter[p] of C.  With one dispatched row per token (scatter = the
// dispatch's sorted_token, row_w = the gate weights) that is y, bit for bit
// what storing the rows and then launch_combine would give; C rows that no p
// names are not written.
hipError_t launch_gemm_bf16_scatter(const void* A, const void* W, void* C, const int* off,
                                    int E, int R, int K, int N, const int* scatter,
                                    const float* row_w, void* split_ws, hipStream_t s);
// C[e] = P_e^T . Q_e ([M][N] per expert) with P_e, Q_e the rows
// [off[e], off[e+1]) of P [R][M] and Q [R][N] (expert weight gradients).
hipError_t launch_gemm_bf16_wgrad(const void* P, const void* Q, void* C, const int* off, int E,
                                  int R, int M, int N, hipStream_t s);
// zout != nullptr: the accumulators are also stored there before GELU
hipError_t launch_gemm_f32(const float* A, const float* W, float* C, const int* off, int E,
                           int R, int K, int N, int ldc, bool gelu, float* zout, hipStream_t s);
// C[rows_e] = A[rows_e] . W_e^T with W stored [E][N][K]; with dgelu_z != nullptr
// the result is multiplied by GELU'(dgelu_z) ([R][N], like C)
hipError_t launch_gemm_f32_nt(const float* A, const float* W, float* C, const int* off, int E,
                              int R, int K, int N, const float* dgelu_z, hipStream_t s);
// C[e] = P_e^T . Q_e ([M][N] per expert), rows [off[e], off[e+1]) of P [R][M], Q [R][N]
hipError_t launch_gemm_f32_wgrad(const float* P, const float* Q, float* C, const int* off, int E,
                                 int R, int M, int N, hipStream_t s);

hipError_t launch_combine(const void* yp, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, bool bf16, void* y, hipStream_t s);

// xp[p] = x[sorted_token[p]] for the rows p < min(offsets[E], R) (a token
// index outside [0, T) gives a zero row; grid sized by R)
hipError_t launch_gather_rows(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                              int E, int R, int T, int H, size_t elem_bytes, void* xp,
                              hipStream_t s);

// Backward kernels (backward.hip)
// zero `bytes` (a multiple of 16) at p (16-byte aligned) with a kernel
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
size_t router_wgrad_ws_bytes(int T, int H, int E);
// bytes of dl's three bf16 planes ([T][3][E rounded up to 16])
size_t router_planes_bytes(int T, int E);
// dw[T*k] = dy[t] . yp[p] and dyp[p] = w * dy[t] for every kept pair
hipError_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv_pos,
                              const float* w, int T, int H, int k, bool bf16, float* dw,
                              void* dyp, hipStream_t s);
// dl[T,E] (fp32, dense) from the gate weights' gradient dw; with dlp, also
// dl's three bf16 planes (router_planes_bytes) for launch_router_wgrad
// and, with dlk (top-k then softmax gating only), each slot's own logit
// gradient dlk[t*k + j] = dl[t, ids_j]
hipError_t launch_router_bwd(const float* logits, const int32_t* ids, const float* w,
                             const float* dw, int T, int E, int k, bool softmax_all, float* dl,
                             uint16_t* dlp, float* dlk, hipStream_t s);
// dW_r = x^T dl (W_r's type), db_r = sum_t dl (skipped when db_r is null);
// bf16 x with dlp: on the matrix cores from the planes, else from dl
hipError_t launch_router_wgrad(const void* x, const float* dl, const uint16_t* dlp, int T,
                               int H, int E, bool x_bf16, bool w_bf16, void* dw_r, float* db_r,
                               void* ws, hipStream_t s);
// dx[t] = sum_j dxp[inv_pos[t,j]] + dl[t] . W_r^T; w_rt: scratch for W_r^T
// (E*H elements of W_r's type); with dlk (dl zero outside ids[t, 0..k), the
// top-k-then-softmax gating) the router term takes the k slots' rows only
hipError_t launch_dx_finish(const void* dxp, const int32_t* inv_pos, const int32_t* ids,
                            const float* dl, const float* dlk, const void* w_r, int T, int H,
                            int E, int k, bool bf16, bool w_bf16, void* w_rt, void* dx,
                            hipStream_t s);

}  // namespace moe
