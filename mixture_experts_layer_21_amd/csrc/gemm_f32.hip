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
    int N, int ldc, float* __restrict__ zout) {
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
      if (zout && n < N) zout[(size_t)(tile.row0 + m) * ldc + n] = acc[i][j];
    }
  }
}

// Backward products on the vector ALUs, same tiling (64x64, K step 16):
//   NT  C[rows_e] = epilogue(A[rows_e] . W_e^T), W stored [E][N][K]; the
//       epilogue is C = acc or acc * GELU'(aux) (aux [R][N] like C);
//   TN  C[e] = P_e^T . Q_e ([M][N] per expert), P_e and Q_e the rows
//       [off[e], off[e+1]) of P [R][M] and Q [R][N].
template <bool TN>
__global__ __launch_bounds__(256) void gemm_f32_bwd(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
    const int* __restrict__ off, int E, int R, int K, int M, int N, int dgelu,
    const float* __restrict__ aux) {
  __shared__ __attribute__((aligned(16))) float As[FBK][FBM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[FBK][FBN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  Tile tile;
  int kb = 0;
  if constexpr (TN) {
    const int MT = (M + FBM - 1) / FBM, NTN = (N + FBN - 1) / FBN;
    const int L = xcd_remap(blockIdx.x, E * MT * NTN);
    if (L < 0) return;
    tile.e = L / (MT * NTN);
    const int r = L % (MT * NTN);
    tile.row0 = (r % MT) * FBM;
    tile.mrows = min(FBM, M - tile.row0);
    tile.nt = r / MT;
    expert_rows(off, tile.e, R, kb, K);
    C += (size_t)tile.e * M * N;
  } else {
    const int NTN = (N + FBN - 1) / FBN;
    tile = map_tile(off, E, R, FBM, NTN, blockIdx.x);
    if (!tile.valid) return;
  }
  const int n0 = tile.nt * FBN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    float av[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (TN) {
      // P row kb+k0+kr, columns row0+c..+3; Q row kb+k0+kr, columns n0+c..+3
      const int kr = tid / 16, c = (tid % 16) * 4;
      if (k0 + kr < K) {
        const size_t row = (size_t)(kb + k0 + kr);
        if (tile.row0 + c < M) {
          const float4 t = *(const float4*)(A + row * M + tile.row0 + c);
          av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
        }
        if (n0 + c < N) {
          const float4 t = *(const float4*)(B + row * N + n0 + c);
          bv[0] = t.x; bv[1] = t.y; bv[2] = t.z; bv[3] = t.w;
        }
      }
      __syncthreads();
      *(float4*)&As[kr][c] = make_float4(av[0], av[1], av[2], av[3]);
      *(float4*)&Bs[kr][c] = make_float4(bv[0], bv[1], bv[2], bv[3]);
    } else {
      // A row row0+rr, k0+kc..+3; W_e row n0+rr (K contiguous), k0+kc..+3
      const int rr = tid / 4, kc = (tid % 4) * 4;
      if (k0 + kc < K) {
        if (rr < tile.mrows) {
          const float4 t = *(const float4*)(A + (size_t)(tile.row0 + rr) * K + k0 + kc);
          av[0] = t.x; av[1] = t.y; av[2] = t.z; av[3] = t.w;
        }
        if (n0 + rr < N) {
          const float4 t = *(const float4*)(B + ((size_t)tile.e * N + n0 + rr) * K + k0 + kc);
          bv[0] = t.x; bv[1] = t.y; bv[2] = t.z; bv[3] = t.w;
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[kc + q][rr] = av[q];
        Bs[kc + q][rr] = bv[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      const float4 a = *(const float4*)&As[kk][ty * 4];
      const float4 b = *(const float4*)&Bs[kk][tx * 4];
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
    const size_t row = (size_t)(tile.row0 + m) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = acc[i][j];
      if (dgelu) v *= gelu_tanh_grad(aux[row + n]);
      C[row + n] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, const float* W, float* C, const int* off,
                           int E, int R, int K, int N, int ldc, bool gelu, float* zout,
                           hipStream_t s) {
  const int NTN = (N + FBN - 1) / FBN;
  const long mt_max = off ? (long)(R + FBM - 1) / FBM + (long)min(E, R) : (long)(R + FBM - 1) / FBM;
  long blocks = mt_max * NTN;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  const bool nvec = (N % 4) == 0;
  dim3 g((unsigned)blocks), b(256);
  if (gelu) {
    if (nvec) hipLaunchKernelGGL((gemm_f32_grouped<true, true>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc, zout);
    else hipLaunchKernelGGL((gemm_f32_grouped<true, false>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc, zout);
  } else {
    if (nvec) hipLaunchKernelGGL((gemm_f32_grouped<false, true>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc, zout);
    else hipLaunchKernelGGL((gemm_f32_grouped<false, false>), g, b, 0, s, A, W, C, off, E, R, K, N, ldc, zout);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32_nt(const float* A, const float* W, float* C, const int* off, int E,
                              int R, int K, int N, const float* dgelu_z, hipStream_t s) {
  const int NTN = (N + FBN - 1) / FBN;
  const long mt_max = (long)(R + FBM - 1) / FBM + (long)min(E, R);
  long blocks = (mt_max * NTN + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_bwd<false>), dim3((unsigned)blocks), dim3(256), 0, s, A, W, C,
                     off, E, R, K, 0, N, dgelu_z ? 1 : 0, dgelu_z);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_wgrad(const float* P, const float* Q, float* C, const int* off, int E,
                                 int R, int M, int N, hipStream_t s) {
  const long tiles = (long)E * ((M + FBM - 1) / FBM) * ((N + FBN - 1) / FBN);
  if (tiles == 0) return hipSuccess;
  const long blocks = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_f32_bwd<true>), dim3((unsigned)blocks), dim3(256), 0, s, P, Q, C, off,
                     E, R, 0, M, N, 0, nullptr);
  return hipGetLastError();
}

}  // namespace moe
