// Grouped expert GEMM on bf16 MFMA (gfx950): C[rows_e] = act(A[rows_e] . W[e])
// for every expert e, rows_e = [off[e], off[e+1]).
//
//   A  [R, K] bf16 row-major (dispatched token rows, K contiguous), or the
//      token matrix x itself with a row-gather list (dispatch fused in)
//   W  [E, K, N] bf16 row-major (N contiguous, as the layer stores W1/W2)
//   C  [R, N] bf16 row-major, fp32 accumulation, rounded to nearest even
//
// This is the expert step of the fused MoE article (Mmad -> GELU -> Mmad per
// expert, section 2) run as one launch over all experts, with the article's
// weight-reuse idea (an expert's weights stay in use while its token blocks
// stream past, section "tiling") mapped onto a tile order that keeps the
// row tiles of one weight slab adjacent (see map_tile).
//
// Design (256x256 output tiles, one workgroup per CU; 8 waves as 2 along
// the tokens x 4 along the columns, two waves per SIMD, 128x64 per wave; K
// step 32):
//  * the forward kernel is persistent: a workgroup runs its tiles one after
//    another and each tile's last steps already load the next tile's first
//    ones, so no tile starts with an empty pipeline;
//  * operands move global -> LDS with buffer_load ... lds (no VGPRs), 1 KB
//    per instruction, into multi-stage rings (128 KB), steps in flight;
//  * W stays in its natural k-major layout in LDS; the MFMA operand (4
//    consecutive k of one column) comes from ds_read_b64_tr_b16; both
//    tiles are XOR-swizzled so the operand reads are free of bank conflicts;
//  * the product is computed transposed, D[n][m] = W^T A^T with
//    v_mfma_f32_32x32x16_bf16 (W as the MFMA A operand), so each lane ends up
//    holding 4 consecutive output columns of one token row: epilogue stores
//    are 8 bytes per lane;
//  * 32-row token blocks beyond the tile's valid rows skip their LDS reads
//    and MFMAs (compile-time count per wave), so a tile with few rows costs
//    little compute;
//  * tiles of the last partial round are split along K (deterministic
//    stream-K, see split_plan).
// The same pipeline, with other operand arrangements, serves the backward
// (gemm_bf16_nt, gemm_bf16_wgrad).
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kWM = 2;          // waves along the token rows
constexpr int kWN = 4;          // waves along the columns (8 waves: two per SIMD)
constexpr int BK = 32;          // K step (bf16 elements): two 16-wide MFMA slices
constexpr int W_STAGES = 4;     // weight ring: one K step per stage, 3 in flight
constexpr int MIN_SPLIT_STEPS = 16;   // K steps per piece of a split tile, at least
// Pacing of a light tile (s_sleep units of 64 cycles per missing 32-row block
// per K step; see gemm_bf16_grouped)
constexpr int kPaceSleep = 3;

template <int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int NT = kWave * WM * WN;          // threads
  static constexpr int NW = WM * WN;                  // waves
  static constexpr int TM = BM / WM;                  // tokens per wave
  static constexpr int TN = BN / WN;                  // columns per wave
  static constexpr int FM = TM / 32;                  // MFMA blocks (tokens)
  static constexpr int FN = TN / 32;                  // MFMA blocks (columns)
  static constexpr int A_ROW = 2 * BK * 2;            // bytes per token row per stage (128)
  static constexpr int W_ROW = BN * 2;                // bytes per k row (512)
  static constexpr int LDS_A = BM * A_ROW;            // bytes per token stage (32 KB)
  static constexpr int LDS_W = BK * W_ROW;            // bytes per weight stage (16 KB)
  // direct-to-LDS loads: one instruction moves 64 lanes x 16 B = 1 KB
  static constexpr int A_INSTS = LDS_A / 1024 / NW;   // per wave per token stage
  static constexpr int W_INSTS = LDS_W / 1024 / NW;   // per wave per K step
  static constexpr int PER_PIECE = FN * FM * 16 * NT; // fp32 partials of a split tile piece
  static_assert(A_ROW == 128 && W_ROW == 512, "layout below assumes BK=32, BN=256");
  static_assert(A_INSTS * NW * 1024 == LDS_A && W_INSTS * NW * 1024 == LDS_W, "load split");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
};

// Why the token rows are 128 bytes: the vector memory path keeps a bounded
// number of cache-line requests in flight per CU, so the load rate is set by
// the request count, and a 64-byte row piece costs a whole request for half a
// line.  Loading two K steps of a row at once makes every request a full line.
//
// LDS layouts (16-byte chunks XOR-swizzled so that MFMA operand reads are
// free of bank conflicts):
//   token stage [BM][64] bf16, 128-byte rows: chunk c of row m at c ^ ((m >> 1) & 7);
//     16 lanes reading 16 rows of one chunk hit 64 distinct banks.
//   weight stage [32][BN] bf16 (the weight slab's natural k-major layout),
//     512-byte rows: chunk c of row k at c ^ (4 * (k & 3)); a transposed read
//     covering 4 k-rows x 32 columns hits 64 distinct banks.
__device__ __forceinline__ int swz_a(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int swz_w(int k) { return 4 * (k & 3); }


// How a tile's K range is shared: S pieces (S = 1: the whole tile in one
// workgroup); this piece is s; partials of split tile `slot` live in `part`.
struct Split {
  int S, s, slot;
  float* part;
};

// Operand arrangements (C = A . B for each expert):
//   NN  A [rows][K] (K contiguous) and B = W_e [K][N] (N contiguous): the
//       forward's expert products;
//   NT  A [rows][K] and B = W_e^T with W_e stored [N][K] (K contiguous): the
//       backward's products with a transposed expert weight;
//   TN  A = P_e^T and B = Q_e with P_e [K][M], Q_e [K][N] row-major, K running
//       over the expert's dispatched rows: the expert weight gradients.
// A K-contiguous operand is staged as rows of 128 bytes (two K steps) and
// read with plain 16-byte LDS reads; a k-major operand is staged as 32 rows of
// 256 columns (one K step) and read with the transposed LDS read.
enum Kind { kNN = 0, kNT = 1, kTN = 2 };
// epilogues each arrangement is used with (bit 1 << EP_x)
constexpr int kind_epilogues(int kind) {
  return kind == kNN ? (1 << EP_PLAIN) | (1 << EP_GELU)
                     : kind == kNT ? (1 << EP_PLAIN) | (1 << EP_DGELU) : (1 << EP_PLAIN);
}

// Arguments of one grouped GEMM launch.
struct GemmArgs {
  const uint16_t* A;      // NN/NT: token rows [a_rows][K]; TN: P (this expert's rows first)
  const int* gather;      // NN/NT: dispatched row p is row gather[p] of A (nullptr: row p)
  int a_rows;             // NN/NT: rows of A
  const uint16_t* B;      // NN: W [E][K][N]; NT: W [E][N][K]; TN: Q (this expert's rows first)
  uint16_t* C;            // NN/NT: [R][N] dispatched rows; TN: this expert's [M][N]
  int K, N, M;            // M: TN only (row length of P)
  int ep;                 // epilogue (EP_PLAIN, EP_GELU, EP_DGELU, EP_SCATTER)
  const uint16_t* aux;    // EP_DGELU: z [R][N], read where C is written
  uint16_t* zout;         // NN: also store the accumulators before GELU here ([R][N])
  const int* scatter;     // EP_SCATTER: row p goes to row scatter[p] of C ...
  const float* row_w;     // ... scaled by row_w[scatter[p]]
  int wrow;               // wave layout (wave_mn)
};

// Which row half (wm) and column quarter (wn) of the tile wave w computes.
// wrow 0: wm = w % WM, so the two waves of a SIMD (w and w + 4) share a row
// half; wrow 1: wm = w / WN, so every SIMD holds one wave of each half and a
// tile whose rows fit in the first half still keeps all four SIMDs' matrix
// units busy (for launches whose tiles are mostly that short).
template <int WM, int WN>
__device__ __forceinline__ void wave_mn(int wave, int wrow, int& wm, int& wn) {
  wm = wrow ? wave / WN : wave % WM;
  wn = wrow ? wave % WN : wave / WM;
}

// LDS of one workgroup: one array per stage, so the compiler can tell that a
// read of one stage does not wait on the loads into another.
//   NN: a[0..1] token stages (32 KB), w[0..3] weight stages (16 KB)
//   NT: a[0..1] token stages, w[0..2] transposed-weight stages (32 KB)
//   TN: a[0..3] P stages, w[0..3] Q stages (16 KB)
// stg: this wave's 8 KB epilogue staging area (inside the rings).
struct Lds {
  char* a[4];
  char* w[4];
  char* stg;
};

// Epilogue of one output tile from the accumulators: acc[.][j] holds 32-row
// block jbase + j of the wave (callers have made the rings free: no wave
// reads them any more).
//   EP_PLAIN  C = acc;  EP_GELU  C = GELU(acc);
//   EP_DGELU  C = acc * GELU'(z), z read from aux at the same row and column;
//   EP_SCATTER  row scat[p] of C = bf16(fma(sw[scat[p]], bf16(acc row p), 0)).
// EPS: the epilogues this instantiation supports (bit 1 << EP_x), so that a
// kernel carries only the code of its own.  PB: 32-row blocks per staging
// pass (the wave's staging area is PB * 4 KB).  NTS: non-temporal stores, for
// output that this launch's readers will not read back soon.
template <int BM, int BN, int WM, int WN, int EPS, int NFM, int FMA, int PB = 2,
          bool NTS = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[GemmShape<BM, BN, WM, WN>::FN][FMA],
                                           uint16_t* __restrict__ C, const Tile& tile, int N,
                                           int ep, const uint16_t* __restrict__ aux,
                                           const int* __restrict__ scat,
                                           const float* __restrict__ sw, char* stg, int wrow,
                                           int jbase = 0) {
  using S = GemmShape<BM, BN, WM, WN>;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int wm, wn;
  wave_mn<WM, WN>(wave, wrow, wm, wn);
  const int n0 = tile.nt * BN;
  const int wrow0 = wm * S::TM;
  // Lane holds D[n][m] for m = lane%32 and 4 consecutive n.  Stored straight
  // to C, one instruction would touch 32 rows with 16 bytes each, 32 partial
  // lines; instead each wave stages 64 rows of its TM x TN block at a time
  // (epilogue applied, bf16) in its own 8 KB of the idle rings, 128-byte
  // rows with 16-byte chunk c of row r at c ^ (r & 7), and writes them back
  // row by row: each instruction then stores 8 whole 128-byte row pieces.
  static_assert(S::TN * 2 == 128, "staging layout");
  if constexpr (NFM > 0) {
    // EP_SCATTER: the destination row and the weight of the row this lane
    // stages in each 32-row block (m = lane % 32), loaded before anything is
    // staged; the store loop takes the destinations from these lanes
    constexpr bool SC = (EPS & (1 << EP_SCATTER)) != 0;
    const bool scatter = SC && (EPS == (1 << EP_SCATTER) || ep == EP_SCATTER);
    int dst[NFM];
    float scl[NFM];
    if constexpr (SC) {
      if (scatter) {
#pragma unroll
        for (int j = 0; j < NFM; ++j) {
          const int m = wrow0 + (jbase + j) * 32 + (lane % 32);
          dst[j] = scat[tile.row0 + min(m, tile.mrows - 1)];   // (rows past the tile: unused)
        }
#pragma unroll
        for (int j = 0; j < NFM; ++j) scl[j] = sw[dst[j]];
      }
    }
#pragma unroll
    for (int p = 0; p < NFM; p += PB) {              // PB blocks of 32 rows per pass
#pragma unroll
      for (int j = p; j < p + PB && j < NFM; ++j) {
        const int r = (j - p) * 32 + (lane % 32);
        u32x2 zq[S::FN][4];
        if ((EPS & (1 << EP_DGELU)) && ep == EP_DGELU) {
          const int m = wrow0 + (jbase + j) * 32 + (lane % 32);
          const int nc = n0 + wn * S::TN + 4 * (lane / 32);
          const uint16_t* zr = aux + (size_t)(tile.row0 + min(m, tile.mrows - 1)) * N + nc;
#pragma unroll
          for (int i = 0; i < S::FN; ++i)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              zq[i][gq] = (m < tile.mrows && nc + 32 * i + 8 * gq < N)
                              ? *(const u32x2*)(zr + 32 * i + 8 * gq)
                              : u32x2{0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < S::FN; ++i) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            float v0 = acc[i][j][4 * gq + 0], v1 = acc[i][j][4 * gq + 1];
            float v2 = acc[i][j][4 * gq + 2], v3 = acc[i][j][4 * gq + 3];
            if ((EPS & (1 << EP_GELU)) && ep == EP_GELU) {
              v0 = gelu_tanh(v0); v1 = gelu_tanh(v1);
              v2 = gelu_tanh(v2); v3 = gelu_tanh(v3);
            } else if ((EPS & (1 << EP_DGELU)) && ep == EP_DGELU) {
              const u32x2 z = zq[i][gq];
              v0 *= gelu_tanh_grad(bf16_to_f32(z[0] & 0xFFFFu));
              v1 *= gelu_tanh_grad(bf16_to_f32(z[0] >> 16));
              v2 *= gelu_tanh_grad(bf16_to_f32(z[1] & 0xFFFFu));
              v3 *= gelu_tanh_grad(bf16_to_f32(z[1] >> 16));
            } else if (SC && scatter) {
              // the dispatched row as stored in bf16, then its gate weight
              // applied as the combine applies it
              v0 = __builtin_fmaf(scl[j], bf16_to_f32(f32_to_bf16(v0)), 0.f);
              v1 = __builtin_fmaf(scl[j], bf16_to_f32(f32_to_bf16(v1)), 0.f);
              v2 = __builtin_fmaf(scl[j], bf16_to_f32(f32_to_bf16(v2)), 0.f);
              v3 = __builtin_fmaf(scl[j], bf16_to_f32(f32_to_bf16(v3)), 0.f);
            }
            const int c = i * 4 + gq;                // 16-byte chunk of the 128-byte row
            *(u32x2*)(stg + r * 128 + ((c ^ (r & 7)) * 16) + (lane / 32) * 8) =
                u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): this wave's writes are in
      __builtin_amdgcn_wave_barrier();
      constexpr int ROWS = 32 * PB;
#pragma unroll
      for (int q = 0; q < ROWS / 8; ++q) {           // 8 rows per instruction
        const int r = q * 8 + lane / 8;
        if (p * 32 + r >= NFM * 32) break;           // (odd NFM: half a pass)
        const int slot = lane % 8;
        const int m = wrow0 + (jbase + p) * 32 + r;
        const int n = n0 + wn * S::TN + (slot ^ (r & 7)) * 8;
        const u32x4 v = *(const u32x4*)(stg + r * 128 + slot * 16);
        int row = tile.row0 + m;
        if constexpr (SC)   // (row r of the pass: lane r % 32 of its block holds it)
          if (scatter) row = __shfl(dst[min(p + q / 4, NFM - 1)], r % 32);
        if (m < tile.mrows && n < N) {
          u32x4* out = (u32x4*)(C + (size_t)row * N + n);
          if constexpr (NTS)
            __builtin_nontemporal_store(v, out);
          else
            *out = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);            // reads done before the next pass writes
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// K-contiguous operand loader: ROWS rows of 128 bytes (two K steps) per
// stage, row r of the stage is memory row row_of(r) (-1: none, reads zero).
// A stage that starts at or past k_limit reads zero (an empty descriptor: a
// scalar choice).  With MASK, 8-element chunks at or past k_limit read zero
// in every stage, for a stage that can straddle k_limit (read unmasked, its
// chunks past K would hold the next row's leading elements).
template <int ROWS, int NW, bool MASK>
struct RowLoader {
  static constexpr int INSTS = ROWS * 128 / 1024 / NW;   // 1 KB per instruction
  uint32_t voff[INSTS];
  int q0;                 // first instruction index of this wave (uniform)
  const uint16_t* base;
  uint32_t bytes;
  int k_limit;
  // logical 16-byte chunk a lane moves in instruction q (rows 8q .. 8q+7)
  __device__ __forceinline__ static int chunk(int q, int lane) {
    return (lane % 8) ^ swz_a(q * 8 + lane / 8);
  }
  template <class RowOf>
  __device__ __forceinline__ void init(const uint16_t* b, uint32_t nbytes, int K, int kl,
                                       int wave, int lane, RowOf row_of) {
    base = b;
    bytes = nbytes;
    k_limit = kl;
    q0 = __builtin_amdgcn_readfirstlane(wave * INSTS);
#pragma unroll
    for (int u = 0; u < INSTS; ++u) {
      const int q = q0 + u;                          // 8 rows per instruction
      const int mr = row_of(q * 8 + lane / 8);
      voff[u] = mr >= 0 ? (uint32_t)mr * K * 2 + chunk(q, lane) * 16 : kPastEnd;
    }
  }
  // K steps k0 / BK and k0 / BK + 1
  template <int AUX = 0>
  __device__ __forceinline__ void load(int k0, char* st) const {
    const uint32_t skip = (uint32_t)k0 * 2;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(base + k0, k0 < k_limit && bytes > skip ? bytes - skip : 0u);
    const int lane = lane_id();
#pragma unroll
    for (int u = 0; u < INSTS; ++u) {
      uint32_t vo = voff[u];
      if constexpr (MASK) vo = (k0 + chunk(q0 + u, lane) * 8 < k_limit) ? vo : kPastEnd;
      load_to_lds<AUX>(r, st + (q0 + u) * 1024, vo);
    }
  }
};

// k-major operand loader: 32 k rows of 256 columns (512 bytes) per stage.
// Rows at or past k_limit read zero (the descriptor ends there); columns
// past the operand's width read neighbouring data that feeds only outputs
// that are never stored.
template <int NW>
struct ColLoader {
  static constexpr int INSTS = 32 * 512 / 1024 / NW;     // 2 k rows per instruction
  uint32_t voff[INSTS];
  int dst[INSTS];
  const uint16_t* base;
  int ld;
  uint32_t bytes;
  __device__ __forceinline__ void init(const uint16_t* b, int ldim, int k_limit, int col0,
                                       int wave, int lane) {
    base = b;
    ld = ldim;
    bytes = (uint32_t)k_limit * ldim * 2;
#pragma unroll
    for (int u = 0; u < INSTS; ++u) {
      const int q = wave * INSTS + u;
      const int kr = 2 * q + lane / 32;
      const int c = (lane % 32) ^ swz_w(kr);
      voff[u] = (uint32_t)kr * ldim * 2 + (uint32_t)(col0 + c * 8) * 2;
      dst[u] = q * 1024;
    }
  }
  // k0 may pass the limit on the last steps: the size clamps to 0 and every
  // load returns zero without touching memory.
  template <int AUX = 0>
  __device__ __forceinline__ void load(int k0, char* st) const {
    const uint32_t skip = (uint32_t)k0 * ld * 2;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(base + (size_t)k0 * ld, bytes > skip ? bytes - skip : 0u);
#pragma unroll
    for (int u = 0; u < INSTS; ++u) load_to_lds<AUX>(r, st + dst[u], voff[u]);
  }
};

// Persistent forward GEMM: what a work item (a tile, or a split piece of one)
// hands over to the next item of its workgroup.  The last 4 steps of an item
// issue the next item's first 4 steps' loads, in the order the prologue
// would, so the next item starts with them in flight.
struct Carry {
  bool carry_in;          // this item's prologue loads were issued by the previous item
  bool pace;              // this wave sleeps in each K step (see gemm_bf16_grouped)
  bool has_next;
  Tile next;              // the next item's tile
  int next_kb, next_ke;   // and its K-step range
};

// One output tile.  NFM (compile time) is the number of 32-row blocks of
// this wave that hold valid rows, so the main loop has no branches around
// its LDS reads and MFMAs (the accumulators stay in registers).
//
// Global loads use buffer descriptors whose base advances with k0 and whose
// size ends at the last valid row of the tile (token rows) or at the piece's
// K limit (k-major operands): rows past the tile and k rows past the piece's
// K range read as zero, so no clamping appears in the loop.  No token row
// may take in elements past its K range, not even against zero W rows: a
// NaN or Inf in the next row times zero would reach this row's outputs.
// Stages start at even K steps (pieces of split tiles start at even steps);
// with K a multiple of 64 they never straddle the range's end and a stage
// past it reads zero; otherwise (KM, and always in NT, which masks W's K
// tail too) the token rows' K tail is masked in 8-element chunks.
// WAUX: cache policy of the weight loads, NN and NT (kNonTemporal when no
// other workgroup reads the same weight slab).  XEP != 0: the epilogues of
// this instantiation (bit 1 << EP_x) in place of the arrangement's own.
template <int KIND, int BM, int BN, int WM, int WN, int NFM, bool PERSIST = false, int WAUX = 0,
          int XEP = 0, bool KM = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Tile& tile, int kt_begin,
                                          int kt_end, const Split& sp, const Lds& lds,
                                          const Carry* cy = nullptr) {
  static_assert(!PERSIST || KIND == kNN, "the persistent form is the forward's");
  using S = GemmShape<BM, BN, WM, WN>;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int wm, wn;
  wave_mn<WM, WN>(wave, g.wrow, wm, wn);
  const int n0 = tile.nt * BN;
  const int wrow0 = wm * S::TM;
  const int K = g.K, N = g.N;
  const int k_limit = min(K, kt_end * BK);

  // --- loaders (offsets constant over the K loop) ----------------------------
  // m side: token rows (NN, NT), or P's k rows (TN)
  // n side: W's k rows (NN), W's rows n (NT), or Q's k rows (TN)
  RowLoader<BM, S::NW, KIND == kNT || KM> la;
  ColLoader<S::NW> lp;
  ColLoader<S::NW> lw;
  RowLoader<BN, S::NW, true> lb;
  if constexpr (KIND != kTN) {
    // Token rows: row0+m of A, or row gather[row0+m] of A when the token rows
    // are gathered straight from x (dispatch fused into the load).  Contiguous
    // A ends at the tile's last row, so that a read past it returns zeros:
    // rows beyond the tile, such as the unwritten rows of a capacity-limited
    // dispatch, may hold any bits, NaN included.
    const uint32_t a_bytes =
        (uint32_t)(g.gather ? g.a_rows : min(g.a_rows, tile.row0 + tile.mrows)) * K * 2;
    la.init(g.A, a_bytes, K, k_limit, wave, lane, [&](int m) {
      return m < tile.mrows ? (g.gather ? g.gather[tile.row0 + m] : tile.row0 + m) : -1;
    });
  } else {
    lp.init(g.A, g.M, K, tile.row0, wave, lane);
  }
  const uint16_t* We = g.B + (KIND == kTN ? 0 : (size_t)tile.e * K * N);
  if constexpr (KIND == kNT) {
    lb.init(We, (uint32_t)N * K * 2, K, k_limit, wave, lane,
            [&](int r) { return n0 + r < N ? n0 + r : -1; });
  } else {
    lw.init(We, N, k_limit, n0, wave, lane);
  }
  constexpr int AI = KIND == kTN ? ColLoader<S::NW>::INSTS : RowLoader<BM, S::NW, false>::INSTS;
  constexpr int BI = KIND == kNT ? RowLoader<BN, S::NW, true>::INSTS : ColLoader<S::NW>::INSTS;
  const int k0 = kt_begin * BK;
  const int nsteps = kt_end - kt_begin;
  // persistent: the loaders of the next item (or, with none, this item's
  // loaders past its K range, which read zeros)
  RowLoader<BM, S::NW, KIND == kNT || KM> la_n;
  ColLoader<S::NW> lw_n;
  int k0n = 0;
  const int nsr = (nsteps + 3) / 4 * 4;
  if constexpr (PERSIST) {
    if (cy->has_next) {
      const Tile& t2 = cy->next;
      const int kl2 = min(K, cy->next_ke * BK);
      const uint32_t a_bytes2 =
          (uint32_t)(g.gather ? g.a_rows : min(g.a_rows, t2.row0 + t2.mrows)) * K * 2;
      la_n.init(g.A, a_bytes2, K, kl2, wave, lane, [&](int m) {
        return m < t2.mrows ? (g.gather ? g.gather[t2.row0 + m] : t2.row0 + m) : -1;
      });
      lw_n.init(g.B + (size_t)t2.e * K * N, N, kl2, t2.nt * BN, wave, lane);
      k0n = cy->next_kb * BK;
    } else {
      la_n = la;
      lw_n = lw;
      k0n = k0 + nsr * BK;
    }
  }

  // --- fragment read offsets ------------------------------------------------
  // K-contiguous operand (16-byte reads): row rbase + lane%32 (+ 32 per
  // block), k = 32 par + 16 h + 8 (lane/32) + 0..7 of the stage (par: which of
  // its two K steps).
  const int fr = lane % 32;
  auto row_off = [&](int rbase, int (&o)[2][2]) {
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 4 * par + 2 * h + lane / 32;
        o[par][h] = (rbase + fr) * 128 + ((c ^ swz_a(fr)) * 16);
      }
  };
  // k-major operand (transposed reads): two reads per 32-column block i, for
  // k = 16 h + 8 (g/2) + 4 rd + (0..3), g = lane/16, and column cbase + 32 i +
  // 16 (g%2) + lane%16.  The block offset 4i sits in chunk bits 2..3, which
  // the swizzle also flips, so each (h, rd, i) keeps its own offset.
  const int gg = lane / 16, li = lane % 16;
  auto col_off = [&](int cbase, auto& o, int nblk) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int i = 0; i < nblk; ++i) {
          const int kr = 16 * h + 8 * (gg / 2) + 4 * rd + li / 4;
          const int nn = cbase + 32 * i + 16 * (gg % 2) + 4 * (li % 4);
          o[h][rd][i] = kr * 512 + (((nn / 8) ^ swz_w(kr)) * 16) + (nn % 8) * 2;
        }
  };
  constexpr int FMA = NFM > 0 ? NFM : 1;
  int fn_row[2][2], fm_row[2][2];
  int fn_col[2][2][S::FN], fm_col[2][2][FMA];
  if constexpr (KIND == kNT) row_off(wn * S::TN, fn_row); else col_off(wn * S::TN, fn_col, S::FN);
  if constexpr (KIND == kTN) col_off(wrow0, fm_col, FMA); else row_off(wrow0, fm_row);

  f32x16 acc[S::FN][FMA];
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int j = 0; j < FMA; ++j) acc[i][j] = f32x16{};

  // n side -> MFMA A operand (rows = output columns n), m side -> MFMA B
  auto read_frags = [&](const char* wst, const char* ast, int par, int h, bf16x8* wf,
                        bf16x8* af) {
#pragma unroll
    for (int i = 0; i < S::FN; ++i) {
      if constexpr (KIND == kNT) {
        wf[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(wst + fn_row[par][h] + i * 32 * 128));
      } else {
        const u32x2 lo = read_tr(wst + fn_col[h][0][i]);
        const u32x2 hi = read_tr(wst + fn_col[h][1][i]);
        wf[i] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
    }
#pragma unroll
    for (int j = 0; j < FMA; ++j) {
      if constexpr (KIND == kTN) {
        const u32x2 lo = read_tr(ast + fm_col[h][0][j]);
        const u32x2 hi = read_tr(ast + fm_col[h][1][j]);
        af[j] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      } else {
        af[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(ast + fm_row[par][h] + j * 32 * 128));
      }
    }
  };

  // Software pipeline.  Step kt (local index, one K step of BK):
  //   first half   MFMAs of slice 0 (operands already in registers), each
  //                paired with an LDS read of slice 1's operands;
  //   middle       wait for this wave's loads of step kt+1, barrier: every
  //                wave's part of step kt+1 has landed and every wave is done
  //                reading step kt, whose stages then take new loads;
  //   second half  MFMAs of slice 1, each paired with an LDS read of step
  //                kt+1's slice-0 operands.
  // Stages and loads (vector-memory counts retire in issue order):
  //   NN  W stage kt % 4, token stage (kt / 2) % 2.  Step j issues W(j+4) and,
  //       odd j, A(j+3, j+4); the prologue W0 W1 A01 W2 W3 A23.  Step kt+1's
  //       data is in once at most 2 W + 2 A (even kt) or 1 W (odd kt) loads
  //       are outstanding.
  //   NT  token stage (kt / 2) % 2, weight stage (kt / 2) % 3 (pairs of
  //       steps).  Odd j issues A(j+3, j+4) then B(j+5, j+6); the prologue
  //       B01 A01 B23 A23 B45.  Wait: 2 B + A (even kt), B (odd kt).
  //   TN  both stages kt % 4.  Step j issues P(j+4) Q(j+4); the prologue
  //       P0 Q0 .. P3 Q3.  Wait: 2 (P + Q).
  // (A bare s_barrier: a release fence would wait for every outstanding load.)
  bf16x8 wf0[S::FN], af0[FMA], wf1[S::FN], af1[FMA];
  constexpr int NRD = (KIND == kNT ? S::FN : 2 * S::FN) + (KIND == kTN ? 2 * FMA : FMA);
  constexpr int NMF = S::FN * NFM;         // MFMAs per slice

  auto mfma_slice = [&](const bf16x8* wf, const bf16x8* af) {
    if constexpr (NFM > 0) {
#pragma unroll
      for (int j = 0; j < NFM; ++j)
#pragma unroll
        for (int i = 0; i < S::FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
  };
  auto interleave = [&]() {
    // [MFMA, LDS read] pairs, then the remaining MFMAs or reads
    constexpr int P = NRD < NMF ? NRD : NMF;
#pragma unroll
    for (int r = 0; r < P; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NMF > P) __builtin_amdgcn_sched_group_barrier(0x008, NMF - P, 0);
    if constexpr (NRD > P) __builtin_amdgcn_sched_group_barrier(0x100, NRD - P, 0);
  };

  bool pace = false;
  if constexpr (PERSIST) pace = cy->pace;
  // step kt of the unrolled group of 4
  auto step = [&](int kt, auto st_c, auto last_c) {
    constexpr int ST = decltype(st_c)::value;
    constexpr bool LAST = decltype(last_c)::value;   // persistent: an item's last 4 steps
    constexpr int PAR = ST % 2;
    constexpr int WS = KIND == kNT ? (ST / 2) % 3 : ST;        // n-side stage
    constexpr int WN1 = KIND == kNT ? ((ST + 1) / 2) % 3 : (ST + 1) % 4;
    constexpr int AS = KIND == kTN ? ST : (ST / 2) % 2;        // m-side stage
    constexpr int AN1 = KIND == kTN ? (ST + 1) % 4 : ((ST + 1) / 2) % 2;
    read_frags(lds.w[WS], lds.a[AS], PAR, 1, wf1, af1);
    mfma_slice(wf0, af0);
    interleave();
    if constexpr (KIND == kNN) {
      if constexpr (PAR == 0)
        __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * BI + 2 * AI));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_le(BI));
    } else if constexpr (KIND == kNT) {
      __builtin_amdgcn_s_waitcnt(vmcnt_le(PAR == 0 ? 2 * BI + AI : BI));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * (AI + BI)));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0): reads of step kt done
    if constexpr (KIND == kNN && PERSIST && NFM < S::FM)
      if (pace) __builtin_amdgcn_s_sleep(kPaceSleep * (S::FM - NFM));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if constexpr (KIND == kNN && LAST) {
      // steps kt+4 (and kt+3, kt+4 for the token ring) are the next item's
      lw_n.template load<WAUX>(k0n + (kt + W_STAGES - nsr) * BK, lds.w[ST]);
      if constexpr (PAR == 1) la_n.load(k0n + (kt + 3 - nsr) * BK, lds.a[ST / 2]);
    } else if constexpr (KIND == kNN) {
      lw.template load<WAUX>(k0 + (kt + W_STAGES) * BK, lds.w[ST]);
      if constexpr (PAR == 1) la.load(k0 + (kt + 3) * BK, lds.a[ST / 2]);
    } else if constexpr (KIND == kNT) {
      if constexpr (PAR == 1) {
        la.load(k0 + (kt + 3) * BK, lds.a[(ST / 2) % 2]);
        lb.template load<WAUX>(k0 + (kt + 5) * BK, lds.w[(ST / 2) % 3]);
      }
    } else {
      lp.load(k0 + (kt + 4) * BK, lds.a[ST]);
      lw.load(k0 + (kt + 4) * BK, lds.w[ST]);
    }
    // this step's loads go out right after the barrier: left to itself the
    // scheduler sinks them past the next 16 MFMAs, which shortens their lead
    // by a step and makes the next waits (counted for the order above) wait
    // for one step more than they need
    constexpr int NL = KIND == kNN ? BI + (PAR == 1 ? AI : 0)
                                   : (KIND == kNT ? (PAR == 1 ? AI + BI : 0) : AI + BI);
    if constexpr (NL > 0) __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);
    read_frags(lds.w[WN1], lds.a[AN1], 1 - PAR, 0, wf0, af0);
    mfma_slice(wf1, af1);
    interleave();
  };

  // The loop runs a multiple of 4 steps; steps past the K range meet zero
  // rows (or zero chunks) and add nothing.
  if constexpr (KIND == kNN) {
    if (!PERSIST || !cy->carry_in) {
      lw.template load<WAUX>(k0, lds.w[0]);
      lw.template load<WAUX>(k0 + BK, lds.w[1]);
      la.load(k0, lds.a[0]);
      lw.template load<WAUX>(k0 + 2 * BK, lds.w[2]);
      lw.template load<WAUX>(k0 + 3 * BK, lds.w[3]);
      la.load(k0 + 2 * BK, lds.a[1]);
    }
    // step 0's data (W0, A01) is in once W2, W3, A23 alone are outstanding
    __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * BI + AI));
  } else if constexpr (KIND == kNT) {
    lb.template load<WAUX>(k0, lds.w[0]);
    la.load(k0, lds.a[0]);
    lb.template load<WAUX>(k0 + 2 * BK, lds.w[1]);
    la.load(k0 + 2 * BK, lds.a[1]);
    lb.template load<WAUX>(k0 + 4 * BK, lds.w[2]);
    // pair 0 (B0, A0) is in once B1, A1, B2 alone are outstanding
    __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * BI + AI));
  } else {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      lp.load(k0 + s4 * BK, lds.a[s4]);
      lw.load(k0 + s4 * BK, lds.w[s4]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * (AI + BI)));
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  read_frags(lds.w[0], lds.a[0], 0, 0, wf0, af0);
  if constexpr (PERSIST) {
    // all groups but the last, then the last with the next item's loads
    int kt = 0;
    for (; kt + 4 < nsr; kt += 4) {
      step(kt + 0, std::integral_constant<int, 0>{}, std::false_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
      step(kt + 2, std::integral_constant<int, 2>{}, std::false_type{});
      step(kt + 3, std::integral_constant<int, 3>{}, std::false_type{});
    }
    step(kt + 0, std::integral_constant<int, 0>{}, std::true_type{});
    step(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
    step(kt + 2, std::integral_constant<int, 2>{}, std::true_type{});
    step(kt + 3, std::integral_constant<int, 3>{}, std::true_type{});
  } else if constexpr (KIND == kNT) {
    // stage pattern repeats every 12 steps (2 token x 3 weight stages of two
    // steps): whole periods in the loop, then a remainder of 4, 8 or 12
    // steps (a branch inside the loop body defeats the register allocation)
    const int nmain = nsteps / 12 * 12;
    int kt = 0;
    for (; kt < nmain; kt += 12) {
      step(kt + 0, std::integral_constant<int, 0>{}, std::false_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
      step(kt + 2, std::integral_constant<int, 2>{}, std::false_type{});
      step(kt + 3, std::integral_constant<int, 3>{}, std::false_type{});
      step(kt + 4, std::integral_constant<int, 4>{}, std::false_type{});
      step(kt + 5, std::integral_constant<int, 5>{}, std::false_type{});
      step(kt + 6, std::integral_constant<int, 6>{}, std::false_type{});
      step(kt + 7, std::integral_constant<int, 7>{}, std::false_type{});
      step(kt + 8, std::integral_constant<int, 8>{}, std::false_type{});
      step(kt + 9, std::integral_constant<int, 9>{}, std::false_type{});
      step(kt + 10, std::integral_constant<int, 10>{}, std::false_type{});
      step(kt + 11, std::integral_constant<int, 11>{}, std::false_type{});
    }
    if (kt < nsteps) {
      step(kt + 0, std::integral_constant<int, 0>{}, std::false_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
      step(kt + 2, std::integral_constant<int, 2>{}, std::false_type{});
      step(kt + 3, std::integral_constant<int, 3>{}, std::false_type{});
      if (kt + 4 < nsteps) {
        step(kt + 4, std::integral_constant<int, 4>{}, std::false_type{});
        step(kt + 5, std::integral_constant<int, 5>{}, std::false_type{});
        step(kt + 6, std::integral_constant<int, 6>{}, std::false_type{});
        step(kt + 7, std::integral_constant<int, 7>{}, std::false_type{});
        if (kt + 8 < nsteps) {
          step(kt + 8, std::integral_constant<int, 8>{}, std::false_type{});
          step(kt + 9, std::integral_constant<int, 9>{}, std::false_type{});
          step(kt + 10, std::integral_constant<int, 10>{}, std::false_type{});
          step(kt + 11, std::integral_constant<int, 11>{}, std::false_type{});
        }
      }
    }
  } else {
    for (int kt = 0; kt < nsteps; kt += W_STAGES) {
      step(kt + 0, std::integral_constant<int, 0>{}, std::false_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
      step(kt + 2, std::integral_constant<int, 2>{}, std::false_type{});
      step(kt + 3, std::integral_constant<int, 3>{}, std::false_type{});
    }
  }
  // drain the loads still in flight before the workgroup's LDS is released
  // (persistent: the next item's loads stay in flight; the kernel drains at
  // its end)
  if constexpr (!PERSIST) __builtin_amdgcn_s_waitcnt(vmcnt_le(0));

  // --- split tiles: the piece leaves its fp32 partial sums in the workspace
  // (in register order: thread-contiguous 16-byte groups, so every store
  // instruction writes 8 KB in one run); a second launch adds them up.
  if (sp.S > 1) {
    if constexpr (NFM > 0) {
      float* mine = sp.part + ((size_t)sp.slot * sp.S + sp.s) * S::PER_PIECE;
#pragma unroll
      for (int i = 0; i < S::FN; ++i)
#pragma unroll
        for (int j = 0; j < NFM; ++j)
#pragma unroll
          for (int v = 0; v < 16; v += 4)
            *(f32x4*)(mine + (((i * S::FM + j) * 16 + v) * S::NT + tid * 4)) =
                f32x4{acc[i][j][v], acc[i][j][v + 1], acc[i][j][v + 2], acc[i][j][v + 3]};
    }
    return;
  }
  constexpr int EPS = XEP ? XEP : kind_epilogues(KIND);
  if constexpr (PERSIST) {
    // staging outside the rings (4 KB per wave, one 32-row block per pass):
    // no barrier, the next item's loads land in the rings meanwhile
    if (g.zout)
      store_tile<BM, BN, WM, WN, 1, NFM, FMA, 1>(acc, g.zout, tile, N, EP_PLAIN, nullptr,
                                                 nullptr, nullptr, lds.stg, g.wrow);
    store_tile<BM, BN, WM, WN, EPS, NFM, FMA, 1>(acc, g.C, tile, N, g.ep, g.aux, g.scatter,
                                                 g.row_w, lds.stg, g.wrow);
    return;
  }
  // one barrier first, because other waves may still read the K loop's last
  // stages
  __syncthreads();
  if constexpr (KIND == kNN)
    if (g.zout)
      store_tile<BM, BN, WM, WN, 1, NFM>(acc, g.zout, tile, N, EP_PLAIN, nullptr, nullptr,
                                         nullptr, lds.stg, g.wrow);
  store_tile<BM, BN, WM, WN, EPS, NFM>(acc, g.C, tile, N, g.ep, g.aux, g.scatter, g.row_w,
                                       lds.stg, g.wrow);
}

// gemm_tile with NFM = nfm (0 <= nfm <= NF), chosen at run time from a
// wave-uniform count.
template <int KIND, int BM, int BN, int WM, int WN, int NF, bool PERSIST = false, int WAUX = 0,
          int XEP = 0, bool KM = false>
__device__ __forceinline__ void run_tile(int nfm, const GemmArgs& g, const Tile& tile,
                                         int kt_begin, int kt_end, const Split& sp,
                                         const Lds& lds, const Carry* cy = nullptr) {
  if constexpr (NF == 0) {
    gemm_tile<KIND, BM, BN, WM, WN, 0, PERSIST, WAUX, XEP, KM>(g, tile, kt_begin, kt_end, sp,
                                                               lds, cy);
  } else {
    if (nfm == NF)
      gemm_tile<KIND, BM, BN, WM, WN, NF, PERSIST, WAUX, XEP, KM>(g, tile, kt_begin, kt_end, sp,
                                                                  lds, cy);
    else
      run_tile<KIND, BM, BN, WM, WN, NF - 1, PERSIST, WAUX, XEP, KM>(nfm, g, tile, kt_begin,
                                                                     kt_end, sp, lds, cy);
  }
}

// Work split (stream-K style, deterministic): the first floor(n / slots)
// rounds of `slots` tiles (slots = workgroups the GPU runs at once) run whole;
// the remaining sk tiles are split along K into S pieces each, so that the
// last round keeps every CU busy instead of leaving most of them idle.  The
// pieces leave fp32 partials and gemm_split_reduce adds them in split order
// in the next launch: the end of a launch is what makes one XCD's writes
// visible to another without flushing L2 caches mid-kernel.
struct SplitPlan {
  int dp, sk, nsplit, KT;
};
// (can_split false: no split workspace; the leftover tiles run whole)
template <int BM, int BN>
__device__ __forceinline__ SplitPlan split_plan(const int* __restrict__ off, int E, int R,
                                                int K, int N, int slots, bool can_split) {
  SplitPlan pl;
  const int NTN = (N + BN - 1) / BN;
  pl.KT = (K + BK - 1) / BK;
  const int nreal = count_row_tiles(off, E, R, BM) * NTN;
  pl.dp = (nreal / slots) * slots;                 // tiles run whole
  pl.sk = nreal - pl.dp;                           // tiles split along K
  pl.nsplit = 1;
  // (short-K GEMMs gain less from filling the last round than the partials
  // and shorter pipelines cost them)
  if (can_split && pl.sk > 0 && pl.KT >= 4 * MIN_SPLIT_STEPS)
    pl.nsplit = max(1, min(slots / pl.sk, pl.KT / MIN_SPLIT_STEPS));
  return pl;
}

// The split piece that workgroup slot p (0 <= p < sk * nsplit) runs: tile
// L, K range s.  Pieces are listed K range by K range (range s of every
// split tile, then range s + 1, ...) and each XCD takes a contiguous run of
// the list, so the pieces one XCD runs together cover one K range of
// consecutive tiles: row tiles that share a weight slab, and slabs that
// share token rows, meet in its L2.
__device__ __forceinline__ void split_piece(const SplitPlan& pl, int p, int& L, int& s) {
  const int q = xcd_remap(p, pl.sk * pl.nsplit);
  L = pl.dp + q % pl.sk;
  s = q / pl.sk;
}

// K steps [kb, ke) of range s: near-equal ranges whose bounds are even (a
// stage of two steps never straddles one), the last ending at KT.
__device__ __forceinline__ void piece_steps(const SplitPlan& pl, int s, int& kb, int& ke) {
  kb = (s * pl.KT / pl.nsplit) & ~1;
  ke = s + 1 == pl.nsplit ? pl.KT : ((s + 1) * pl.KT / pl.nsplit) & ~1;
}

// this wave's 8 KB of epilogue staging inside two 32 KB regions
__device__ __forceinline__ char* staging(char* lo, char* hi, int nw) {
  const int wave = threadIdx.x / kWave;
  return (wave < nw / 2 ? lo : hi) + (wave % (nw / 2)) * 8192;
}

// Grouped GEMM over dispatched rows, one work item per workgroup (the NT
// kernel): split plan, tile lookup and the tile.
template <int KIND, int BM, int BN, int WM, int WN, int WAUX = 0>
__device__ __forceinline__ void grouped_body(const GemmArgs& g, const int* __restrict__ off,
                                             int E, int R, float* __restrict__ part, int slots,
                                             const Lds& lds) {
  using S = GemmShape<BM, BN, WM, WN>;
  const SplitPlan pl = split_plan<BM, BN>(off, E, R, g.K, g.N, slots, part != nullptr);
  const int bid = blockIdx.x;
  int L, kt_begin = 0, kt_end = pl.KT;
  Split sp{1, 0, 0, part};
  if (bid < pl.dp) {
    L = xcd_remap(bid, pl.dp);
  } else {
    const int p = bid - pl.dp;              // (pl.dp: a multiple of the XCD count)
    if (p >= pl.sk * pl.nsplit) return;
    split_piece(pl, p, L, sp.s);
    sp.S = pl.nsplit;
    sp.slot = L - pl.dp;
    kt_begin = sp.s * pl.KT / pl.nsplit;
    kt_end = (sp.s + 1) * pl.KT / pl.nsplit;
  }
  const int NTN = (g.N + BN - 1) / BN;
  const Tile tile = lookup_tile(off, E, R, BM, NTN, L);
  if (!tile.valid) return;

  // 32-row token blocks of this wave that hold valid rows (wave-uniform)
  int wm, wn;
  wave_mn<WM, WN>(threadIdx.x / kWave, g.wrow, wm, wn);
  int nfm = max(0, min(S::FM, (tile.mrows - wm * S::TM + 31) / 32));
  nfm = __builtin_amdgcn_readfirstlane(nfm);
  run_tile<KIND, BM, BN, WM, WN, S::FM, false, WAUX>(nfm, g, tile, kt_begin, kt_end, sp, lds);
}

// The forward's expert products, persistent: one workgroup per CU takes its
// whole tiles b, b + G, ... (G = grid; the same XCD-aware order as the
// one-tile-per-workgroup kernel) and then its split piece, if any, handing
// the pipeline from one item to the next (Carry); the epilogue stages
// through its own 32 KB (128 KB of rings + 32 KB = 160 KB).  WAUX: the
// weight loads' cache policy; XEP: as in gemm_tile.
template <int BM, int BN, int WM, int WN, int WAUX = 0, int XEP = 0, bool KM = false>
__global__ __launch_bounds__(kWave * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_bf16_grouped(
    GemmArgs g, const int* __restrict__ off, int E, int R, float* __restrict__ part,
    int slots) {
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) char a0[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char a1[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char w0[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char w1[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char w2[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char w3[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char stg_all[S::NW * 4096];
  static_assert(2 * S::LDS_A + 4 * S::LDS_W + S::NW * 4096 <= 163840, "LDS budget");
  const int wave = threadIdx.x / kWave;
  const Lds lds{{a0, a1, nullptr, nullptr}, {w0, w1, w2, w3}, stg_all + wave * 4096};
  const SplitPlan pl = split_plan<BM, BN>(off, E, R, g.K, g.N, slots, part != nullptr);
  const int G = gridDim.x, b = blockIdx.x;
  const int NTN = (g.N + BN - 1) / BN;
  const int n_whole = pl.dp / G;                       // pl.dp is a multiple of slots = G
  const int n_items = n_whole + (b < pl.sk * pl.nsplit ? 1 : 0);
  // item i: a whole tile (i < n_whole) or this workgroup's split piece
  auto item = [&](int i, Tile& t, int& kb, int& ke, Split& sp) {
    sp = Split{1, 0, 0, part};
    kb = 0;
    ke = pl.KT;
    int L;
    if (i < n_whole) {
      L = xcd_remap(b + i * G, pl.dp);
    } else {
      split_piece(pl, b, L, sp.s);
      sp.S = pl.nsplit;
      sp.slot = L - pl.dp;
      piece_steps(pl, sp.s, kb, ke);
    }
    t = lookup_tile(off, E, R, BM, NTN, L);
    if (!t.valid) {
      // (no tile: L is always in range for offsets the counts came from; an
      // empty item still runs the K loop to keep the carried loads in step,
      // reading expert 0's first slab and storing nothing)
      t.e = 0;
      t.nt = 0;
      t.row0 = 0;
      t.mrows = 0;
      t.mi = 0;
    }
  };
  int wm, wn;
  wave_mn<WM, WN>(wave, g.wrow, wm, wn);
  Carry cy;
  cy.carry_in = false;
  Tile cur;
  int ckb = 0, cke = 0;
  Split csp;
  if (n_items > 0) item(0, cur, ckb, cke, csp);
  for (int i = 0; i < n_items; ++i) {
    cy.has_next = i + 1 < n_items;
    Split nsp;
    if (cy.has_next) item(i + 1, cy.next, cy.next_kb, cy.next_ke, nsp);
    int nfm = max(0, min(S::FM, (cur.mrows - wm * S::TM + 31) / 32));
    nfm = __builtin_amdgcn_readfirstlane(nfm);
    // A whole tile holding an expert's last rows (not its first) shares its
    // weight slab with the expert's other row tiles, which run beside it on
    // this XCD.  With few rows it would run ahead of them and read the slab
    // from memory a second time; instead the waves of its first 128 rows
    // sleep in each K step in proportion to their missing 32-row blocks, so
    // the tile keeps pace and finds the slab in L2 (not with non-temporal
    // weight loads, where slabs are not shared)
    cy.pace = WAUX == 0 && wm == 0 && cur.mi > 0 && csp.S == 1;
    run_tile<kNN, BM, BN, WM, WN, S::FM, true, WAUX, XEP, KM>(nfm, g, cur, ckb, cke, csp, lds,
                                                              &cy);
    cy.carry_in = true;
    cur = cy.next;
    ckb = cy.next_kb;
    cke = cy.next_ke;
    csp = nsp;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

// The backward's products with a transposed expert weight (NT): two token
// stages and three weight stages of 32 KB (the 160 KB a workgroup may hold).
// WAUX: the weight loads' cache policy.
template <int BM, int BN, int WM, int WN, int WAUX = 0>
__global__ __launch_bounds__(kWave * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_bf16_nt(
    GemmArgs g, const int* __restrict__ off, int E, int R, float* __restrict__ part,
    int slots) {
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) char a0[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char a1[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char b0[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char b1[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char b2[S::LDS_A];
  static_assert(5 * S::LDS_A <= 163840 && S::NW * 8192 <= 2 * S::LDS_A, "LDS budget");
  const Lds lds{{a0, a1, nullptr, nullptr}, {b0, b1, b2, nullptr}, staging(a0, a1, S::NW)};
  grouped_body<kNT, BM, BN, WM, WN, WAUX>(g, off, E, R, part, slots, lds);
}

// Expert weight gradients: C_e[M][N] = P_e^T Q_e for every expert e, where
// P_e and Q_e are rows [off[e], off[e+1]) of P [R][M] and Q [R][N]
// (K = the expert's row count; an expert with no rows gets a zero gradient).
//
// K is short here (an expert's rows: hundreds), so a tile is only a few K
// steps and its load prologue and store epilogue would dominate.  The kernel
// is persistent: workgroup b takes tiles b, b + G, b + 2G, ... (G = grid),
// each padded to a multiple of 4 K steps (at least 4), and the K-step
// pipeline runs on across tile boundaries: in a tile's last 4 steps the ring
// loads already fetch the next tile's first 4 steps, so the next tile starts
// with its operands in LDS.  The epilogue stages through its own 32 KB (one
// 32-row block per pass), outside the rings (128 KB + 32 KB = the 160 KB a
// workgroup may hold).  Both operands are k-major: 4-stage rings, transposed
// LDS reads, one step's loads issued per step; the wait before step kt+1 is
// "at most 2 steps' loads outstanding".  Stores share that counter on this
// architecture; an epilogue's stores stay in flight into the next tile, which
// keeps those waits correct: loads complete in issue order among themselves,
// so a count at or below the bound with stores pending still means the older
// loads have landed (pending stores only make a wait longer).
// Tiles are numbered expert by expert, column tile outer, row tile inner.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kWave * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4))) void gemm_bf16_wgrad(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q, uint16_t* __restrict__ C,
    const int* __restrict__ off, int E, int R, int M, int N) {
  using S = GemmShape<BM, BN, WM, WN>;
  constexpr int FM = S::FM, FN = S::FN;
  __shared__ __attribute__((aligned(1024))) char p0[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char p1[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char p2[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char p3[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char q0[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char q1[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char q2[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char q3[S::LDS_W];
  __shared__ __attribute__((aligned(1024))) char stg_all[S::NW * 4096];
  static_assert(S::LDS_W == 16384 && 8 * S::LDS_W + S::NW * 4096 <= 163840, "LDS budget");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % WM;
  const int wn = wave / WM;
  const Lds lds{{p0, p1, p2, p3}, {q0, q1, q2, q3}, stg_all + wave * 4096};

  const int MT = (M + BM - 1) / BM, NTN = (N + BN - 1) / BN;
  const int per_e = MT * NTN;
  const int total = E * per_e;
  const int G = gridDim.x;
  int L = blockIdx.x;
  if (L >= total) return;

  // k-major loads (as ColLoader): instruction u of this wave covers k rows
  // 2q, 2q + 1 (q = wave * LU + u) of a stage; the lane's offset is a part
  // common to every tile (its k row and swizzled 16-byte chunk) plus the
  // tile's first column
  constexpr int LU = ColLoader<S::NW>::INSTS;
  uint32_t pv[LU], qv[LU];
#pragma unroll
  for (int u = 0; u < LU; ++u) {
    const int kr = 2 * (wave * LU + u) + lane / 32;
    const int c = (lane % 32) ^ swz_w(kr);
    pv[u] = (uint32_t)kr * M * 2 + c * 16;
    qv[u] = (uint32_t)kr * N * 2 + c * 16;
  }
  // a tile: everything wave-uniform
  struct State {
    Tile tile;
    int nsteps, rows;
    const uint16_t* pb;      // P rows of the expert
    const uint16_t* qb;      // Q rows of the expert
    uint16_t* c;
  };
  auto make = [&](int l, State& st) {
    const int e = l / per_e, r = l % per_e;
    st.tile.valid = 1;
    st.tile.e = e;
    st.tile.row0 = (r % MT) * BM;
    st.tile.mrows = min(BM, M - st.tile.row0);
    st.tile.nt = r / MT;
    int kb, rows;
    expert_rows(off, e, R, kb, rows);
    st.rows = rows;
    st.nsteps = max(4, ((st.rows + BK - 1) / BK + 3) / 4 * 4);
    st.pb = P + (size_t)kb * M;
    st.qb = Q + (size_t)kb * N;
    st.c = C + (size_t)e * M * N;
  };
  // step ks of tile st into stage ks % 4 of both rings; rows at or past the
  // expert's row count read zero (the descriptors end there)
  auto load_step = [&](const State& st, int ks, int stage) {
    const uint32_t k0 = (uint32_t)ks * BK;
    const uint32_t lim = (uint32_t)st.rows;
    const uint32_t nk = lim > k0 ? lim - k0 : 0u;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(st.pb + (size_t)k0 * M, nk * M * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(st.qb + (size_t)k0 * N, nk * N * 2);
    const uint32_t pc = (uint32_t)st.tile.row0 * 2, qc = (uint32_t)st.tile.nt * BN * 2;
#pragma unroll
    for (int u = 0; u < LU; ++u)
      load_to_lds(rp, lds.a[stage] + (wave * LU + u) * 1024, pv[u] + pc);
#pragma unroll
    for (int u = 0; u < LU; ++u)
      load_to_lds(rq, lds.w[stage] + (wave * LU + u) * 1024, qv[u] + qc);
  };
  State cur, nxt;
  make(L, cur);
  bool has_next = L + G < total;
  if (has_next) make(L + G, nxt);

  // fragment read offsets (transposed reads on both sides), for slice h = 0
  // and the first read rd = 0: the k row is 16 h + 8 (gg/2) + 4 rd + li/4,
  // and moving by 4 or 16 rows keeps k & 3, hence the swizzle, so rd adds
  // 4 rows (2048 bytes) and h 16 rows (8192 bytes) to the same offset
  const int gg = lane / 16, li = lane % 16;
  const int kr0 = 8 * (gg / 2) + li / 4;
  int fn_col[FN], fm_col[FM];
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int nn = wn * S::TN + 32 * i + 16 * (gg % 2) + 4 * (li % 4);
    fn_col[i] = kr0 * 512 + (((nn / 8) ^ swz_w(kr0)) * 16) + (nn % 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int mm = wm * S::TM + 32 * j + 16 * (gg % 2) + 4 * (li % 4);
    fm_col[j] = kr0 * 512 + (((mm / 8) ^ swz_w(kr0)) * 16) + (mm % 8) * 2;
  }
  auto read_frags = [&](const char* wst, const char* ast, int h, bf16x8* wf, bf16x8* af) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const u32x2 lo = read_tr(wst + fn_col[i] + h * 8192);
      const u32x2 hi = read_tr(wst + fn_col[i] + h * 8192 + 2048);
      wf[i] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const u32x2 lo = read_tr(ast + fm_col[j] + h * 8192);
      const u32x2 hi = read_tr(ast + fm_col[j] + h * 8192 + 2048);
      af[j] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };
  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};
  bf16x8 wf0[FN], af0[FM], wf1[FN], af1[FM];
  constexpr int NRD = 2 * FN + 2 * FM;
  constexpr int NMF = FN * FM;
  constexpr int LI = 2 * ColLoader<S::NW>::INSTS;      // loads per step
  auto mfma_slice = [&](const bf16x8* wf, const bf16x8* af) {
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int i = 0; i < FN; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {
    constexpr int PP = NRD < NMF ? NRD : NMF;
#pragma unroll
    for (int r = 0; r < PP; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NMF > PP) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PP, 0);
    if constexpr (NRD > PP) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PP, 0);
  };
  // step kt of the current tile (stage ST = kt % 4); its loads are for step
  // kt + 4: of this tile, else the next tile's step kt + 4 - nsteps, else
  // (no next tile) a zero-size read that keeps the per-step load count
  auto step = [&](int kt, auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    read_frags(lds.w[ST], lds.a[ST], 1, wf1, af1);
    mfma_slice(wf0, af0);
    interleave();
    __builtin_amdgcn_s_waitcnt(vmcnt_le(2 * LI));
    __builtin_amdgcn_s_waitcnt(0xC07F);                    // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // (selects of wave-uniform values: no branch inside the step)
    const int ld = kt + 4;
    const bool own = ld < cur.nsteps || !has_next;
    State sel;
    sel.tile.row0 = own ? cur.tile.row0 : nxt.tile.row0;
    sel.tile.nt = own ? cur.tile.nt : nxt.tile.nt;
    sel.rows = own ? cur.rows : nxt.rows;
    sel.pb = own ? cur.pb : nxt.pb;
    sel.qb = own ? cur.qb : nxt.qb;
    load_step(sel, own ? ld : ld - cur.nsteps, ST);
    __builtin_amdgcn_sched_group_barrier(0x020, LI, 0);    // loads first (as in gemm_tile)
    read_frags(lds.w[(ST + 1) % 4], lds.a[(ST + 1) % 4], 0, wf0, af0);
    mfma_slice(wf1, af1);
    interleave();
  };

#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) load_step(cur, s4, s4);
  __builtin_amdgcn_s_waitcnt(vmcnt_le(3 * LI));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  read_frags(lds.w[0], lds.a[0], 0, wf0, af0);
  while (true) {
    for (int kt = 0; kt < cur.nsteps; kt += 4) {
      step(kt + 0, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
      step(kt + 2, std::integral_constant<int, 2>{});
      step(kt + 3, std::integral_constant<int, 3>{});
    }
    // (the weight gradients: written once, read by no kernel of this pass)
    store_tile<BM, BN, WM, WN, 1 << EP_PLAIN, FM, FM, 1, true>(
        acc, cur.c, cur.tile, N, EP_PLAIN, nullptr, nullptr, nullptr, lds.stg, 0);
    if (!has_next) break;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = f32x16{};
    cur = nxt;
    L += G;
    has_next = L + G < total;
    if (has_next) make(L + G, nxt);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
}

// Split tiles: one workgroup per (split tile, 32-row block jb of every
// wave).  Each wave adds the S partials of its block in split order, two
// pieces' loads in flight per round trip, and stores the block (with the
// launch's epilogue; zout as in the GEMM; XEP as in gemm_tile).
template <int KIND, int BM, int BN, int WM, int WN, int XEP = 0>
__global__ __launch_bounds__(kWave * WM * WN) void gemm_split_reduce(
    GemmArgs g, const int* __restrict__ off, int E, int R, const float* __restrict__ part,
    int slots) {
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) char a0[S::LDS_A];
  __shared__ __attribute__((aligned(1024))) char a1[S::LDS_A];
  char* const stg = staging(a0, a1, S::NW);
  const SplitPlan pl = split_plan<BM, BN>(off, E, R, g.K, g.N, slots, part != nullptr);
  const int slot = blockIdx.x / S::FM, jb = blockIdx.x % S::FM;
  if (pl.nsplit < 2 || slot >= pl.sk) return;
  const int NTN = (g.N + BN - 1) / BN;
  const Tile tile = lookup_tile(off, E, R, BM, NTN, pl.dp + slot);
  if (!tile.valid) return;
  const int tid = threadIdx.x;
  int wm, wn;
  wave_mn<WM, WN>(tid / kWave, g.wrow, wm, wn);
  const int nfm = max(0, min(S::FM, (tile.mrows - wm * S::TM + 31) / 32));
  if (__builtin_amdgcn_readfirstlane(nfm) <= jb) return;   // no valid rows in this block
  const float* all = part + (size_t)slot * pl.nsplit * S::PER_PIECE;
  auto load = [&](int ps, f32x4 (&t)[S::FN][4]) {
    const float* src = all + (size_t)ps * S::PER_PIECE;
#pragma unroll
    for (int i = 0; i < S::FN; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq)
        t[i][vq] = *(const f32x4*)(src + (((i * S::FM + jb) * 16 + 4 * vq) * S::NT + tid * 4));
  };
  f32x4 run[S::FN][4];
  load(0, run);
  for (int ps = 1; ps < pl.nsplit; ps += 2) {
    f32x4 t0[S::FN][4], t1[S::FN][4];
    load(ps, t0);
    const bool two = ps + 1 < pl.nsplit;
    if (two) load(ps + 1, t1);
#pragma unroll
    for (int i = 0; i < S::FN; ++i)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        run[i][vq] += t0[i][vq];
        if (two) run[i][vq] += t1[i][vq];
      }
  }
  f32x16 acc[S::FN][1];
#pragma unroll
  for (int i = 0; i < S::FN; ++i)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][0][4 * vq + e] = run[i][vq][e];
  if constexpr (KIND == kNN)
    if (g.zout)
      store_tile<BM, BN, WM, WN, 1, 1>(acc, g.zout, tile, g.N, EP_PLAIN, nullptr, nullptr,
                                       nullptr, stg, g.wrow, jb);
  store_tile<BM, BN, WM, WN, XEP ? XEP : kind_epilogues(KIND), 1>(acc, g.C, tile, g.N, g.ep,
                                                                  g.aux, g.scatter, g.row_w, stg,
                                                                  g.wrow, jb);
}

int device_slots() {
  // one 256x256 workgroup per CU (128 KB of LDS), capped at kMaxSlots and
  // rounded down to a multiple of the XCD count, so that a persistent
  // workgroup's items b, b + G, ... stay on its own XCD's share of tiles
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxSlots;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = kMaxSlots;
    cus = std::min(cus, kMaxSlots);
    cached[dev] = cus >= kXcds ? cus / kXcds * kXcds : cus;
  }
  return cached[dev];
}

constexpr int kMaxExperts = 1024;   // (the ABI's limit on E)

// The second expert GEMM's split sums and the combine in one launch, for a
// decode-sized batch (a few dispatched rows; the GEMM launch then skips its
// split reduce).  Workgroup (t, column tile) forms 256 columns of y[t] from
// the token's k rows: a row of a whole tile is read from yp as the GEMM
// stored it; a row of a split tile is the sum of its pieces' fp32 partials
// in split order, rounded to bf16 as the reduce would store it.  The k rows
// are then weighted and summed in slot order as the combine does, so y is
// bit for bit that of the separate reduce and combine passes.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void reduce_combine_rows(
    const uint16_t* __restrict__ yp, const float* __restrict__ part,
    const int* __restrict__ off, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ inv, const float* __restrict__ w, uint16_t* __restrict__ y,
    int T, int k, int E, int R, int K, int N, int slots, int wrow) {
  static_assert(BN == 256, "one column per thread");
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ int pre[kMaxExperts];           // row tiles of the experts before e
  const int t = blockIdx.x, nt = blockIdx.y, tid = threadIdx.x;
  const int NTN = (N + BN - 1) / BN;
  const SplitPlan pl = split_plan<BM, BN>(off, E, R, K, N, slots, part != nullptr);
  if (tid < kWave) {
    int carry = 0;
    for (int c = 0; c < E; c += kWave) {
      const int e = c + tid;
      int mt = 0;
      if (e < E) {
        int lo, cnt;
        expert_rows(off, e, R, lo, cnt);
        mt = (cnt + BM - 1) / BM;
      }
      const int incl = wave_incl_scan(mt);
      if (e < E) pre[e] = carry + incl - mt;
      carry += wave_bcast(incl, kWave - 1);
    }
  }
  __syncthreads();
  const int nl = tid, n = nt * BN + nl;
  if (n >= N) return;
  // place of column nl in a piece's partials (the accumulator order the
  // pieces store): column block, 8-column group, half-lane and element
  const int wn = nl / S::TN, nn = nl % S::TN;
  const int ci = nn / 32, r32 = nn % 32;
  const int gq = r32 / 8, hl = (r32 % 8) / 4, e4 = r32 % 4;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int p = inv[t * k + j];
    const bool in = (unsigned)p < (unsigned)(T * k);
    float v = 0.f, wj = 0.f;
    if (in) {
      wj = w[t * k + j];
      const int e = ids[t * k + j];
      int lo, cnt;
      expert_rows(off, e, R, lo, cnt);
      const int mt = (cnt + BM - 1) / BM;
      const int rr = p - lo, mi = rr / BM, m = rr % BM;
      const int L = pre[e] * NTN + nt * mt + mi;
      if (L < pl.dp || pl.nsplit < 2) {
        v = bf16_to_f32(yp[(size_t)p * N + n]);
      } else {
        const int wm = m / S::TM, jj = (m % S::TM) / 32;
        const int wave = wrow ? wm * WN + wn : wn * WM + wm;
        const int lane = hl * 32 + m % 32;
        const size_t o =
            (size_t)((ci * S::FM + jj) * 16 + 4 * gq) * S::NT + (wave * kWave + lane) * 4 + e4;
        const float* base = part + (size_t)(L - pl.dp) * pl.nsplit * S::PER_PIECE + o;
        float run = base[0];
        for (int sp = 1; sp < pl.nsplit; ++sp) run += base[(size_t)sp * S::PER_PIECE];
        v = bf16_to_f32(f32_to_bf16(run));
      }
    }
    acc = __builtin_fmaf(wj, v, acc);
  }
  y[(size_t)t * N + n] = (uint16_t)f32_to_bf16(acc);
}

template <int KIND, int BM, int BN, int WM, int WN, int XEP = 0>
hipError_t launch_cfg(const GemmArgs& g, const int* off, int E, int R, void* split_ws,
                      hipStream_t s, bool reduce = true) {
  static_assert(XEP == 0 || KIND == kNN, "own epilogues: the forward's products only");
  const int NTN = (g.N + BN - 1) / BN;
  // upper bound of row tiles: sum_e ceil(rows_e / BM) <= ceil(R / BM) + min(E, R)
  const long mt_max = off ? (long)(R + BM - 1) / BM + (long)min(E, R) : (long)(R + BM - 1) / BM;
  const int slots = device_slots();
  // whole tiles (< n) plus at most `slots` pieces of split tiles
  long blocks = mt_max * NTN + slots;
  if (blocks <= slots) return hipSuccess;
  float* part = (float*)split_ws;
  // At most half a row tile per expert on average: nearly every weight slab
  // is read by one tile only, so its loads are non-temporal (their L2 lines
  // go first) rather than displacing the token rows that other tiles read
  // again
  const bool stream_w = (long)R * 2 <= (long)E * BM;
  if constexpr (KIND == kNT) {
    if (stream_w)
      hipLaunchKernelGGL((gemm_bf16_nt<BM, BN, WM, WN, kNonTemporal>), dim3((unsigned)blocks),
                         dim3(kWave * WM * WN), 0, s, g, off, E, R, part, slots);
    else
      hipLaunchKernelGGL((gemm_bf16_nt<BM, BN, WM, WN>), dim3((unsigned)blocks),
                         dim3(kWave * WM * WN), 0, s, g, off, E, R, part, slots);
  } else if (g.K % 64 != 0)
    // (persistent: one workgroup per CU; K tails masked, default cache policy)
    hipLaunchKernelGGL((gemm_bf16_grouped<BM, BN, WM, WN, 0, XEP, true>), dim3((unsigned)slots),
                       dim3(kWave * WM * WN), 0, s, g, off, E, R, part, slots);
  else if (stream_w)
    hipLaunchKernelGGL((gemm_bf16_grouped<BM, BN, WM, WN, kNonTemporal, XEP>),
                       dim3((unsigned)slots), dim3(kWave * WM * WN), 0, s, g, off, E, R, part,
                       slots);
  else
    hipLaunchKernelGGL((gemm_bf16_grouped<BM, BN, WM, WN, 0, XEP>), dim3((unsigned)slots),
                       dim3(kWave * WM * WN), 0, s, g, off, E, R, part, slots);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // tiles are split only when K has at least 4 * MIN_SPLIT_STEPS steps, and
  // only with a split workspace
  if (reduce && part != nullptr && (g.K + BK - 1) / BK >= 4 * MIN_SPLIT_STEPS) {
    hipLaunchKernelGGL((gemm_split_reduce<KIND, BM, BN, WM, WN, XEP>),
                       dim3(kMaxSlots / 2 * GemmShape<BM, BN, WM, WN>::FM),
                       dim3(kWave * WM * WN), 0, s, g, off, E, R, (const float*)part, slots);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

size_t split_ws_bytes() { return (size_t)kMaxSlots * 256 * 256 * sizeof(float); }

namespace {
// Wave layout of a launch (wave_mn): with at most 160 rows per expert on
// average most tiles hold one row half or less, and spreading each half over
// all four SIMDs doubles their matrix throughput; fuller tiles keep the
// layout that measured best for them.
int wave_layout(int R, int E) { return (long)R <= 160L * E ? 1 : 0; }
}  // namespace

hipError_t launch_gemm_bf16(const void* A, const int* gather, int a_rows, const void* W,
                            bool w_nk, void* C, const int* off, int E, int R, int K, int N,
                            int ep, const void* aux, void* zout, void* split_ws,
                            hipStream_t s, bool defer_reduce) {
  GemmArgs g;
  g.A = (const uint16_t*)A;
  g.gather = gather;
  g.a_rows = a_rows;
  g.B = (const uint16_t*)W;
  g.C = (uint16_t*)C;
  g.K = K;
  g.N = N;
  g.M = 0;
  g.ep = ep;
  g.aux = (const uint16_t*)aux;
  g.zout = (uint16_t*)zout;
  g.scatter = nullptr;
  g.row_w = nullptr;
  g.wrow = wave_layout(R, E);
  if (ep == EP_SCATTER) return hipErrorInvalidValue;   // (launch_gemm_bf16_scatter)
  if (w_nk) return launch_cfg<kNT, 256, 256, kWM, kWN>(g, off, E, R, split_ws, s);
  return launch_cfg<kNN, 256, 256, kWM, kWN>(g, off, E, R, split_ws, s, !defer_reduce);
}

hipError_t launch_reduce_combine(const void* yp, void* split_ws, const int* off,
                                 const int32_t* ids, const int32_t* inv_pos, const float* w,
                                 void* y, int T, int k, int E, int R, int K, int N,
                                 hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E > kMaxExperts) return hipErrorInvalidValue;
  const dim3 g((unsigned)T, (unsigned)((N + 255) / 256)), b(256);
  hipLaunchKernelGGL((reduce_combine_rows<256, 256, kWM, kWN>), g, b, 0, s, (const uint16_t*)yp,
                     (const float*)split_ws, off, ids, inv_pos, w, (uint16_t*)y, T, k, E, R, K,
                     N, device_slots(), wave_layout(R, E));
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_scatter(const void* A, const void* W, void* C, const int* off,
                                    int E, int R, int K, int N, const int* scatter,
                                    const float* row_w, void* split_ws, hipStream_t s) {
  GemmArgs g;
  g.A = (const uint16_t*)A;
  g.gather = nullptr;
  g.a_rows = R;
  g.B = (const uint16_t*)W;
  g.C = (uint16_t*)C;
  g.K = K;
  g.N = N;
  g.M = 0;
  g.ep = EP_SCATTER;
  g.aux = nullptr;
  g.zout = nullptr;
  g.scatter = scatter;
  g.row_w = row_w;
  g.wrow = wave_layout(R, E);
  return launch_cfg<kNN, 256, 256, kWM, kWN, 1 << EP_SCATTER>(g, off, E, R, split_ws, s);
}

hipError_t launch_gemm_bf16_wgrad(const void* P, const void* Q, void* C, const int* off, int E,
                                  int R, int M, int N, hipStream_t s) {
  const long tiles = (long)E * ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles == 0) return hipSuccess;
  // persistent: one workgroup per CU (or per tile when there are fewer)
  const long blocks = std::min<long>(tiles, device_slots());
  hipLaunchKernelGGL((gemm_bf16_wgrad<256, 256, kWM, kWN>), dim3((unsigned)blocks),
                     dim3(kWave * kWM * kWN), 0, s, (const uint16_t*)P, (const uint16_t*)Q,
                     (uint16_t*)C, off, E, R, M, N);
  return hipGetLastError();
}

}  // namespace moe
