// Shared device helpers for the gfx950 MoE kernels: bf16 bit conversions,
// the GELU epilogue, wave-level scans and the grouped-GEMM tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: 8 XCDs, workgroups dealt round-robin

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// fp32 -> (hi, mid, lo) bf16 bits with hi + mid + lo == w up to the rounding
// of lo (hi, mid: truncations; each remainder is exact in fp32).  A product
// of a bf16 value with each part is exact in fp32, so three bf16 matrix
// products summed in fp32 give an fp32-accurate product with w.
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t u = __float_as_uint(w);
  hi = u >> 16;
  const float r1 = w - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t u1 = __float_as_uint(r1);
  mid = u1 >> 16;
  const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
  const uint32_t u2 = __float_as_uint(r2);
  lo = (u2 + 0x7FFFu + ((u2 >> 16) & 1u)) >> 16;
}

// GELU, tanh form: 0.5 z (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3).
// Since 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), this is
//   z / (1 + 2^(z * (c1 + c2 z^2))),  c1 = -2 sqrt(2/pi) log2(e), c2 = 0.044715 c1,
// one exp2 and one reciprocal per element.  For z -> -inf the exp2 overflows
// to +inf and the result is -0; for z -> +inf it tends to z.
__device__ __forceinline__ float gelu_tanh(float z) {
  constexpr float c1 = -2.3022082f;        // -2 * 0.7978845608 * 1.4426950409
  constexpr float c2 = -0.10294324f;       // c1 * 0.044715
  float z2 = z * z;
  float t = z * __builtin_fmaf(c2, z2, c1);
  float e = __builtin_amdgcn_exp2f(t);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// d GELU / dz of the tanh form.  With s = 1 / (1 + exp(-2u)) = 0.5 (1 + tanh u),
// GELU = z s, so GELU' = s + 2 z s (1 - s) u' with u' = sqrt(2/pi) (1 + 3 * 0.044715 z^2).
// s (1 - s) is formed as s - s^2, which stays 0 (not inf * 0) when exp2 overflows.
__device__ __forceinline__ float gelu_tanh_grad(float z) {
  constexpr float c1 = -2.3022082f;        // -2 * sqrt(2/pi) * log2(e)
  constexpr float c2 = -0.10294324f;       // c1 * 0.044715
  constexpr float k1 = 1.5957692f;         // 2 * sqrt(2/pi)
  constexpr float k2 = 0.21406445f;        // k1 * 3 * 0.044715
  const float z2 = z * z;
  const float e = __builtin_amdgcn_exp2f(z * __builtin_fmaf(c2, z2, c1));
  const float s = __builtin_amdgcn_rcpf(1.0f + e);
  return __builtin_fmaf(z * (s - s * s), __builtin_fmaf(k2, z2, k1), s);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// v of the lane the DPP control CTRL names, 0 where that lane is outside the
// row or the destination lane is masked off (ROW_MASK: rows, BANK_MASK: groups
// of four lanes in each row).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int dpp_or_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, true);
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP moves: shifts
// by 1, 2 and 3 lanes, then by 4 and 8 (into the upper lanes of each row)
// give each row's prefix; broadcasting lane 15 into rows 1 and 3 and lane 31
// into rows 2 and 3 carries the row totals.  (No LDS permutes: seven dependent
// VALU steps instead of six LDS round trips.)
__device__ __forceinline__ int wave_incl_scan(int v) {
  int s = v + dpp_or_zero<0x111, 0xF, 0xF>(v);   // row_shr:1
  s += dpp_or_zero<0x112, 0xF, 0xF>(v);          // row_shr:2
  s += dpp_or_zero<0x113, 0xF, 0xF>(v);          // row_shr:3
  s += dpp_or_zero<0x114, 0xF, 0xE>(s);          // row_shr:4, lanes 4..15 of each row
  s += dpp_or_zero<0x118, 0xF, 0xC>(s);          // row_shr:8, lanes 8..15
  s += dpp_or_zero<0x142, 0xA, 0xF>(s);          // row_bcast:15 into rows 1, 3
  s += dpp_or_zero<0x143, 0xC, 0xF>(s);          // row_bcast:31 into rows 2, 3
  return s;
}

// Sum and maximum over the wave (every lane active, result in every lane):
// inside each row of 16 lanes by DPP exchanges (lane ^ 1, lane ^ 2, the
// half-row mirror, the row mirror: every lane of a row ends with the same
// bits), then the four row results read from lanes 0, 16, 32 and 48 and
// combined in that order.  No LDS permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

__device__ __forceinline__ int wave_bcast(int v, int src_lane) {
  return __builtin_amdgcn_readlane(v, src_lane);
}

// ---------------------------------------------------------------------------
// Buffer loads straight into LDS, transposed LDS reads, and the wait counter.
// ---------------------------------------------------------------------------
constexpr uint32_t kBufFlags = 0x00020000u;   // raw buffer, 32-bit data format
constexpr uint32_t kPastEnd = 0xFFFFFFF0u;    // buffer offset that reads as zero

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding and does not wait on LDS/scalar or export counters
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
__device__ constexpr int vmcnt_le(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// (base and size are wave-uniform; readfirstlane states it, so that the
// descriptor is built in scalar registers and no per-lane loop appears)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes),
                                           (int)kBufFlags);
}

// 64 lanes x 16 bytes from global memory straight into a 1 KB LDS block:
// lane t's bytes land at block + 16 t (no VGPRs involved).  A lane whose
// offset is at or past the descriptor's size writes zeros.
// AUX: the load's cache policy (0: default; kNonTemporal: the lines are
// placed to be evicted first, for data that no other workgroup will read)
constexpr int kNonTemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, char* lds_block,
                                            uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_block, 16, voff, 0, 0, AUX);
}

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): in each group of 16 lanes,
// lane i addresses 8 bytes of row i/4 and receives column i of the 4x16 block
// those addresses cover, i.e. 4 consecutive k of one output column.
__device__ __forceinline__ u32x2 read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// Grouped GEMM tiles (see map_tile below for the numbering and XCD mapping).
// ---------------------------------------------------------------------------
struct Tile {
  int valid;
  int e;       // expert (group)
  int row0;    // first dispatched row of the tile
  int mrows;   // valid rows in the tile (1..BM)
  int nt;      // column tile index
  int mi;      // row tile index within the expert (0: its first rows)
};

// Rows [lo, lo + n) of expert e: the offsets' range clamped into [0, R].
// For non-decreasing offsets within [0, R] this is [off[e], off[e+1]); for
// any other offsets (negative, decreasing, past R) every row index formed
// from it still lies inside the R dispatched rows.
__device__ __forceinline__ void expert_rows(const int* __restrict__ off, int e, int R, int& lo,
                                            int& n) {
  const int a = min(max(off[e], 0), R);
  const int b = min(max(off[e + 1], a), R);
  lo = a;
  n = b - a;
}

// Number of row tiles, sum_e ceil(rows_e / BM) (wave-uniform).
__device__ __forceinline__ int count_row_tiles(const int* __restrict__ off, int E,
                                               int dense_rows, int BM) {
  if (off == nullptr) return (dense_rows + BM - 1) / BM;
  const int lane = lane_id();
  int total = 0;
  for (int c = 0; c < E; c += kWave) {
    const int e = c + lane;
    int mt = 0;
    if (e < E) {
      int lo, n;
      expert_rows(off, e, dense_rows, lo, n);
      mt = (n + BM - 1) / BM;
    }
    const int incl = wave_incl_scan(mt);
    total += wave_bcast(incl, kWave - 1);
  }
  return total;
}

// The tile with logical index L (0 <= L < row_tiles * NT).
__device__ __forceinline__ Tile lookup_tile(const int* __restrict__ off, int E,
                                            int dense_rows, int BM, int NT, int L) {
  Tile tile;
  tile.valid = 0;
  const int lane = lane_id();
  if (off == nullptr) {
    const int mt = (dense_rows + BM - 1) / BM;
    tile.valid = 1;
    tile.e = 0;
    tile.nt = L / mt;
    const int mi = L % mt;
    tile.mi = mi;
    tile.row0 = mi * BM;
    tile.mrows = min(BM, dense_rows - tile.row0);
    return tile;
  }
  int carry = 0;
  for (int c = 0; c < E; c += kWave) {
    const int e = c + lane;
    int cnt = 0, mt = 0, row_lo = 0;
    if (e < E) {
      expert_rows(off, e, dense_rows, row_lo, cnt);
      mt = (cnt + BM - 1) / BM;
    }
    const int incl = wave_incl_scan(mt);
    const int lo = (carry + incl - mt) * NT;
    const int hi = (carry + incl) * NT;
    const uint64_t hit = __ballot(mt > 0 && L >= lo && L < hi);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int e_hit = c + src;
      const int lo_hit = wave_bcast(lo, src);
      const int mt_hit = wave_bcast(mt, src);
      const int cnt_hit = wave_bcast(cnt, src);
      const int row_hit = wave_bcast(row_lo, src);
      const int local = L - lo_hit;
      const int mi = local % mt_hit;
      tile.valid = 1;
      tile.e = e_hit;
      tile.nt = local / mt_hit;
      tile.mi = mi;
      tile.row0 = row_hit + mi * BM;
      tile.mrows = min(BM, cnt_hit - mi * BM);
      return tile;
    }
    carry += wave_bcast(incl, kWave - 1);
  }
  return tile;
}

// Grouped GEMM tile mapping.
//
// Expert e owns rows [off[e], off[e+1]) of the dispatched matrix and splits
// them into m_e = ceil(rows_e / BM) row tiles; each row tile meets all NT
// column tiles, so the layer has NREAL = NT * sum_e m_e tiles.  Tiles are
// numbered expert by expert; inside an expert, consecutive tiles share the
// column tile (the same weight slab) and walk its row tiles, so workgroups
// running together read one weight slab from HBM once.
//
// The grid is launched with an upper bound of tiles (the host does not know
// the per-expert counts).  Workgroup ids are dealt to the 8 XCDs round-robin
// (id b runs on XCD b % 8), so of the ids below n, XCD x holds
// q + (x < r ? 1 : 0) of them (q = n / 8, r = n % 8); the id is remapped so
// that each XCD gets that many consecutive logical tiles, which keeps the
// tiles that share a weight slab in one XCD's L2.  The map is a bijection of
// [0, n) for every n (ids at or past n get -1).  Every wave of the block
// computes the same mapping (no LDS, no sync).
// With off == nullptr the matrix is a single dense group of `dense_rows` rows.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if (bid < 0 || bid >= n) return -1;
  const int x = bid % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + bid / kXcds;
}

__device__ __forceinline__ Tile map_tile(const int* __restrict__ off, int E,
                                         int dense_rows, int BM, int NT, int bid) {
  const int nreal = count_row_tiles(off, E, dense_rows, BM) * NT;
  const int L = xcd_remap(bid, nreal);
  if (L < 0) {
    Tile t;
    t.valid = 0;
    return t;
  }
  return lookup_tile(off, E, dense_rows, BM, NT, L);
}

}  // namespace moe
