// Grouped expert GEMM on bf16 MFMA (gfx950): C[rows_e] = act(A[rows_e] . W[e])
// for every expert e, rows_e = [off[e], off[e+1]).
//
//   A  [R, K] bf16 row-major (dispatched token rows, K contiguous)
//   W  [E, K, N] bf16 row-major (N contiguous, as the layer stores W1/W2)
//   C  [R, N] bf16 row-major, fp32 accumulation, rounded to nearest even
//
// This is the expert step of the fused MoE article (Mmad -> GELU -> Mmad per
// expert, section 2) run as one launch over all experts, with the article's
// weight-reuse idea (an expert's weights stay in use while its token blocks
// stream past, section "tiling") mapped onto a tile order that keeps the
// row tiles of one weight slab adjacent (see map_tile).
//
// Design (one 256x256 output tile per workgroup, 4 waves as 2x2, 128x128 per
// wave, K step 64):
//  * the weight slab W[e][k0:k0+64, n0:n0+256] is loaded with 16-byte global
//    loads (8 k-rows x 8 n per thread), transposed in registers with byte
//    permutes and written to LDS as Ws[n][k] (k contiguous), which is the
//    operand layout MFMA wants; the token tile goes to LDS as As[m][k];
//  * rows are padded to 72 bf16 (144 B) so the 16-byte LDS reads of a
//    32-lane column of rows hit distinct banks;
//  * the product is computed transposed, D[n][m] = W^T A^T with
//    v_mfma_f32_32x32x16_bf16 (W as the MFMA A operand), so each lane ends up
//    holding 4 consecutive output columns of one token row: epilogue stores
//    are 8 bytes per lane;
//  * double-buffered LDS: global loads of step k+1 are in flight while step k
//    computes; one barrier per step;
//  * 32-row token blocks beyond the tile's valid rows skip their LDS reads
//    and MFMAs, so a tile with few rows costs little compute.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (144 B)

template <int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int NT = kWave * WM * WN;          // threads
  static constexpr int TM = BM / WM;                  // tokens per wave
  static constexpr int TN = BN / WN;                  // columns per wave
  static constexpr int FM = TM / 32;                  // MFMA blocks (tokens)
  static constexpr int FN = TN / 32;                  // MFMA blocks (columns)
  static constexpr int A_LOADS = BM * (BK / 8) / NT;  // 16-B chunks per thread
  static constexpr int KR = 8 * BN / NT;              // W k-rows per thread
  static constexpr int KCH = BK / KR;                 // k-chunks per column group
  static_assert(A_LOADS >= 1 && BM * (BK / 8) % NT == 0, "A tile split");
  static_assert(KR == 4 || KR == 8, "W tile split");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static constexpr int LDS_A = BM * LDS_STRIDE;       // elements per stage
  static constexpr int LDS_W = BN * LDS_STRIDE;
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kWave * WM * WN) void gemm_bf16_grouped(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    uint16_t* __restrict__ C, const int* __restrict__ off, int E, int R,
    int K, int N, int gelu) {
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (S::LDS_A + S::LDS_W)];

  const int NTN = (N + BN - 1) / BN;
  const Tile tile = map_tile(off, E, R, BM, NTN, blockIdx.x);
  if (!tile.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int n0 = tile.nt * BN;
  const uint16_t* __restrict__ We = W + (size_t)tile.e * K * N;

  // --- global -> register loaders -----------------------------------------
  // A: chunk c (8 bf16) of rows r = tid/8 + i*(NT/8)
  const int a_c = tid % 8;
  const uint16_t* a_src[S::A_LOADS];
#pragma unroll
  for (int i = 0; i < S::A_LOADS; ++i) {
    const int r = tid / 8 + i * (S::NT / 8);
    const int rr = min(r, tile.mrows - 1);   // padded rows re-read a valid row
    a_src[i] = A + (size_t)(tile.row0 + rr) * K + a_c * 8;
  }
  // W: KR consecutive k-rows x 8 columns per thread
  const int w_kc = tid % S::KCH;
  const int w_nc = tid / S::KCH;
  const int w_n = n0 + w_nc * 8;
  const bool w_n_ok = w_n < N;
  const uint16_t* w_src = We + (size_t)(w_kc * S::KR) * N + (w_n_ok ? w_n : 0);

  u32x4 a_reg[S::A_LOADS];
  u32x4 w_reg[S::KR];

  auto load_tiles = [&](int k0) {
    const bool a_ok = (k0 + a_c * 8) < K;
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
      a_reg[i] = a_ok ? *(const u32x4*)(a_src[i] + k0) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < S::KR; ++i) {
      const int k = k0 + w_kc * S::KR + i;
      w_reg[i] = (w_n_ok && k < K) ? *(const u32x4*)(w_src + (size_t)(k0 + i) * N)
                                   : u32x4{0, 0, 0, 0};
    }
  };

  auto store_tiles = [&](int buf) {
    uint16_t* As = lds + buf * (S::LDS_A + S::LDS_W);
    uint16_t* Ws = As + S::LDS_A;
#pragma unroll
    for (int i = 0; i < S::A_LOADS; ++i) {
      const int r = tid / 8 + i * (S::NT / 8);
      *(u32x4*)(As + r * LDS_STRIDE + a_c * 8) = a_reg[i];
    }
    // transpose the KR x 8 block: column n gets KR consecutive k values
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
      uint32_t p[S::KR / 2];
#pragma unroll
      for (int q = 0; q < S::KR / 2; ++q) {
        p[q] = __builtin_amdgcn_perm(w_reg[2 * q + 1][n >> 1], w_reg[2 * q][n >> 1], sel);
      }
      uint16_t* dst = Ws + (w_nc * 8 + n) * LDS_STRIDE + w_kc * S::KR;
      if constexpr (S::KR == 8) {
        *(u32x4*)dst = u32x4{p[0], p[1], p[2], p[3]};
      } else {
        *(u32x2*)dst = u32x2{p[0], p[1]};
      }
    }
  };

  f32x16 acc[S::FN][S::FM];
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < S::FM; ++j) acc[i][j] = f32x16{};

  // token blocks of this wave that hold at least one valid row
  const int wrow0 = wm * S::TM;
  const int nfm = max(0, min(S::FM, (tile.mrows - wrow0 + 31) / 32));

  const int KT = (K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tiles((kt + 1) * BK);
    if (nfm > 0) {
      const uint16_t* As = lds + buf * (S::LDS_A + S::LDS_W);
      const uint16_t* Ws = As + S::LDS_A;
      const int kl = (lane / 32) * 8;
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        bf16x8 wf[S::FN];
        bf16x8 af[S::FM];
#pragma unroll
        for (int i = 0; i < S::FN; ++i) {
          const int n = wn * S::TN + i * 32 + (lane % 32);
          wf[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(Ws + n * LDS_STRIDE + kk + kl));
        }
#pragma unroll
        for (int j = 0; j < S::FM; ++j) {
          if (j < nfm) {
            const int m = wrow0 + j * 32 + (lane % 32);
            af[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(As + m * LDS_STRIDE + kk + kl));
          }
        }
#pragma unroll
        for (int j = 0; j < S::FM; ++j) {
          if (j < nfm) {
#pragma unroll
            for (int i = 0; i < S::FN; ++i) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
            }
          }
        }
      }
    }
    if (kt + 1 < KT) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue: lane holds D[n][m] for m = lane%32 and 4 consecutive n ----
#pragma unroll
  for (int j = 0; j < S::FM; ++j) {
    if (j >= nfm) continue;
    const int m = wrow0 + j * 32 + (lane % 32);
    if (m >= tile.mrows) continue;
    uint16_t* crow = C + (size_t)(tile.row0 + m) * N;
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * S::TN + i * 32 + g * 8 + (lane / 32) * 4;
        if (n < N) {
          float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
          float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
          if (gelu) {
            v0 = gelu_tanh(v0); v1 = gelu_tanh(v1);
            v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
          }
          *(u32x2*)(crow + n) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const void* A, const void* W, void* C, const int* off,
                      int E, int R, int K, int N, bool gelu, hipStream_t s) {
  const int NTN = (N + BN - 1) / BN;
  // upper bound of row tiles: sum_e ceil(rows_e / BM) <= ceil(R / BM) + min(E, R)
  const long mt_max = off ? (long)(R + BM - 1) / BM + (long)min(E, R) : (long)(R + BM - 1) / BM;
  long blocks = mt_max * NTN;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_grouped<BM, BN, WM, WN>), dim3((unsigned)blocks),
                     dim3(kWave * WM * WN), 0, s, (const uint16_t*)A, (const uint16_t*)W,
                     (uint16_t*)C, off, E, R, K, N, gelu ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const void* A, const void* W, void* C, const int* off,
                            int E, int R, int K, int N, bool gelu, hipStream_t s) {
  return launch_cfg<256, 256, 2, 2>(A, W, C, off, E, R, K, N, gelu, s);
}

}  // namespace moe
