// Grouped fp32 GEMM on the vector ALUs: C[rows_e] = act(A[rows_e] . W[e]).
//
//   A [R, K] fp32, W [E, K, N] fp32, C [R, ldc] fp32 (columns 0..N-1 written)
//
// Used for the fp32 layer (expert FFN and router logits).  On MI355X the fp32
// matrix-core rate equals the fp32 vector rate (157.3 TFLOP/s), so fp32 work
// stays on the VALUs: 64x64 output tile, 256 threads with 4x4 outputs each,
// K step 16 through LDS.  The token tile is stored k-major in LDS so each
// thread reads 4 consecutive rows with one 16-byte read.  Tile order and the
// grouped row mapping are shared with the bf16 kernel (map_tile).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool GELU, bool NVEC>
__global__ __launch_bounds__(256) void gemm_f32_grouped(
    const float* __restrict__ A, const float* __restrict__ W,
    float* __restrict__ C, const int* __restrict__ off, int E, int R, int K,
    int N, int ldc) {
  __shared__ __attribute__((aligned(16))) float As[FBK][FBM + 4];
  __shared__ __attribute__((aligned(16))) float Ws[FBK][FBN + 4];

  const int NTN = (N + FBN - 1) / FBN;
  const Tile tile = map_tile(off, E, R, FBM, NTN, blockIdx.x);
  if (!tile.valid) return;

  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int n0 = tile.nt * FBN;
  const float* __restrict__ We = W + (size_t)tile.e * K * N;

  // A loader: row ar = tid/4, k chunk ac = (tid%4)*4
  const int ar = tid / 4, ac = (tid % 4) * 4;
  const float* a_row = A + (size_t)(tile.row0 + min(ar, tile.mrows - 1)) * K;
  // W loader: k row wr = tid/16, n chunk wc = (tid%16)*4
  const int wr = tid / 16, wc = (tid % 16) * 4;

  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k0 + ac < K) av = *(const float4*)(a_row + k0 + ac);   // K % 4 == 0
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
    const int k = k0 + wr;
    if (k < K) {
      const float* wp = We + (size_t)k * N + n0 + wc;
      if (NVEC) {
        if (n0 + wc < N) {
          const float4 t = *(const float4*)wp;
          wv[0] = t.x; wv[1] = t.y; wv[2] = t.z; wv[3] = t.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n0 + wc + q < N) wv[q] = wp[q];
      }
    }
    __syncthreads();
    As[ac + 0][ar] = av.x;
    As[ac + 1][ar] = av.y;
    As[ac + 2][ar] = av.z;
    As[ac + 3][ar] = av.w;
    *(float4*)&Ws[wr][wc] = make_float4(wv[0], wv[1], wv[2], wv[3]);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      const float4 a = *(const float4*)&As[kk][ty * 4];
      const float4 b = *(const float4*)&Ws[kk][tx * 4];
      const float aa[4] = {a.x, a.y, a.z, a.w};
      const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(aa[i], bb[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (m >= tile.mrows) continue;
    float* crow = C + (size_t)(tile.row0 + m) * ldc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) crow[n] = GELU ? gelu_tanh(acc[i][j]) : acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, const float* W, float* C, const int* off,
                           int E, int R, int K, int N, int ldc, bool gelu,
                           hipStream_t s) {
  const int NTN = (N + FBN - 1) / FBN;
  const long mt_max = off ? (long)(R + FBM - 1) / FBM + (long)min(E, R) : (long)(R + FBM - 1) / FBM;
  long blocks = mt_max * NTN;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  const bool nvec = (N % 4) == 0;
  dim3 g((unsigned)blocks), b(256);
  if (gelu) {
    if (nvec) hipLaunchKernelGGL((gemm_f32_grouped<true, true>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc);
    else hipLaunchKernelGGL((gemm_f32_grouped<true, false>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc);
  } else {
    if (nvec) hipLaunchKernelGGL((gemm_f32_grouped<false, true>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc);
    else hipLaunchKernelGGL((gemm_f32_grouped<false, false>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc);
  }
  return hipGetLastError();
}

}  // namespace moe
