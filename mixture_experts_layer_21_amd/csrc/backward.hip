// Backward of the MoE layer: the kernels around the expert GEMMs.
//
// The layer's gradient for an output gradient dy (the chain rule through the
// forward of the fused MoE article, taken step by step in reverse; the CANN
// MoE article's training setting, sections 3 and 4.2):
//   combine_bwd   per (token, slot) pair with dispatched row p:
//                 dw = dy[t] . yp[p] (fp32) and dyp[p] = w * dy[t]
//   router_bwd    per token: the logit gradient dl[t, 0..E) (fp32) through the
//                 softmax's Jacobian (no gradient through the top-k choice)
//   router_wgrad  dW_r = x^T dl and db_r = sum_t dl, split over tokens into
//                 fp32 partials that router_wgrad_reduce adds in split order
//                 (bf16 tokens: router_wgrad_mfma on the matrix cores, with dl
//                 as three bf16 planes that router_bwd also writes)
//   dx_finish     dx[t] = sum_j dxp[inv_pos[t, j]] + dl[t] . W_r^T (through a
//                 transposed copy of W_r, so that its loads are coalesced);
//                 dx_finish_sparse when dl is zero outside the k selected experts
// The expert GEMMs in between (dz = dyp W2^T * GELU'(z), dW2 = h^T dyp,
// dxp = dz W1^T, dW1 = xp^T dz) run on the grouped GEMM kernels.
// Every sum runs in a fixed order: the results are deterministic.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// 8 consecutive elements of a row as fp32 (bf16 rows: one 16-byte load)
template <bool BF16>
__device__ __forceinline__ void load8(const void* row, int c, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 q = ((const u32x4*)row)[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(q[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
    }
  } else {
    const f32x4 a = ((const f32x4*)row)[2 * c], b = ((const f32x4*)row)[2 * c + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// 8 consecutive elements of a row as loaded (bf16: one 16-byte load, kept
// packed until used; fp32: two)
template <bool BF16>
struct Raw8 {
  u32x4 v;
  __device__ __forceinline__ void load(const void* row, int c) { v = ((const u32x4*)row)[c]; }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float operator[](int q) const {
    return bf16_to_f32(q % 2 == 0 ? v[q / 2] & 0xFFFFu : v[q / 2] >> 16);
  }
};
template <>
struct Raw8<false> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const void* row, int c) {
    a = ((const f32x4*)row)[2 * c];
    b = ((const f32x4*)row)[2 * c + 1];
  }
  __device__ __forceinline__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ float operator[](int q) const { return q < 4 ? a[q] : b[q - 4]; }
};

template <bool BF16>
__device__ __forceinline__ void store8(void* row, int c, const float (&v)[8]) {
  if constexpr (BF16) {
    ((u32x4*)row)[c] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  } else {
    ((f32x4*)row)[2 * c] = f32x4{v[0], v[1], v[2], v[3]};
    ((f32x4*)row)[2 * c + 1] = f32x4{v[4], v[5], v[6], v[7]};
  }
}

// One wave per (token, slot) pair i = t * k + j.  Dropped pairs (p < 0) get
// dw = 0 and no dyp row.  A lane takes 8-element chunks lane, lane + 64, ...
// of the row; four of them (dy and yp) are loaded before any is used, so a
// wave has 8 loads in flight instead of one round trip per chunk (the loads
// past the row's end re-read its last chunk and are not used).
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd(const void* __restrict__ dy,
                                                   const void* __restrict__ yp,
                                                   const int32_t* __restrict__ inv_pos,
                                                   const float* __restrict__ w, int T, int H,
                                                   int k, float* __restrict__ dw,
                                                   void* __restrict__ dyp) {
  constexpr int U = 4;
  const int lane = threadIdx.x % kWave;
  // (wave-uniform: the pair's row position and weight come by scalar loads)
  const int i = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
  if (i >= T * k) return;
  const int p = inv_pos[i];
  if (p < 0) {
    if (lane == 0) dw[i] = 0.f;
    return;
  }
  const size_t es = BF16 ? 2 : 4;
  const char* g = (const char*)dy + (size_t)(i / k) * H * es;
  const char* y = (const char*)yp + (size_t)p * H * es;
  char* d = (char*)dyp + (size_t)p * H * es;
  const float wi = w[i];
  const int n8 = H / 8;
  float dot = 0.f;
  for (int c0 = lane; c0 < n8; c0 += U * kWave) {
    float a[U][8], b[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * kWave, n8 - 1);
      load8<BF16>(g, c, a[u]);
      load8<BF16>(y, c, b[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < n8) {
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          dot = __builtin_fmaf(a[u][q], b[u][q], dot);
          o[q] = wi * a[u][q];
        }
        store8<BF16>(d, c, o);
      }
    }
  }
  dot = wave_sum(dot);
  if (lane == 0) dw[i] = dot;
}

// One wave per token: dl[t, e] for every expert (dense, fp32).
//   top-k then softmax:  dl[ids_j] = w_j (dw_j - sum_j' w_j dw_j'), else 0
//   softmax then top-k:  p = softmax(logits[t]);  g_e = dw_j where e = ids_j
//                        (else 0);  dl_e = p_e (g_e - sum_e' p_e' g_e')
// With dlp, also dl's three bf16 planes (split3): dlp[t][q][e] for q = hi,
// mid, lo and e < EP (EP = E rounded up to 16; zero past E).  With dlk (top-k
// then softmax only), also each slot's own logit gradient, dlk[t * k + j] =
// dl[t, ids_j] (0 for an id outside [0, E)), for dx_finish_sparse.
template <int NPL>
__global__ __launch_bounds__(256) void router_bwd(const float* __restrict__ logits,
                                                  const int32_t* __restrict__ ids,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ dw, int T, int E,
                                                  int k, int softmax_all,
                                                  float* __restrict__ dl,
                                                  uint16_t* __restrict__ dlp, int EP,
                                                  float* __restrict__ dlk) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  // slot j's (id, dw, w) in lane j; a slot whose id is outside [0, E) (not
  // an id the training forward produced) takes no part: its weight and
  // gradient are left out of the Jacobian and no logit is addressed for it
  int my_id = -1;
  float my_dw = 0.f, my_w = 0.f;
  if (lane < k) {
    my_id = ids[(size_t)t * k + lane];
    if ((unsigned)my_id < (unsigned)E) {
      my_dw = dw[(size_t)t * k + lane];
      my_w = w[(size_t)t * k + lane];
    } else {
      my_id = -1;
    }
  }
  // g[i]: dw of the slot holding expert lane + 64 i (0 if none)
  float g[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) g[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int id = __builtin_amdgcn_readlane(my_id, j);
    const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_dw), j));
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + i * kWave == id) g[i] = v;
  }
  float out[NPL];
  if (!softmax_all) {
    const float s = wave_sum(my_w * my_dw);
    float wsel[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) wsel[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int id = __builtin_amdgcn_readlane(my_id, j);
      const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + i * kWave == id) wsel[i] = v;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) out[i] = wsel[i] * (g[i] - s);
    // (the same product as out[] at the slot's expert: w_j (dw_j - s))
    if (dlk != nullptr && lane < k) dlk[(size_t)t * k + lane] = my_id >= 0 ? my_w * (my_dw - s) : 0.f;
  } else {
    float l[NPL];
    float m = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      l[i] = e < E ? logits[(size_t)t * E + e] : -__builtin_inff();
      m = fmaxf(m, l[i]);
    }
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      l[i] = lane + i * kWave < E ? __expf(l[i] - m) : 0.f;
      z += l[i];
    }
    const float inv = 1.f / wave_sum(z);
    float pg = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      l[i] *= inv;
      pg += l[i] * g[i];
    }
    const float s = wave_sum(pg);
#pragma unroll
    for (int i = 0; i < NPL; ++i) out[i] = l[i] * (g[i] - s);
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) dl[(size_t)t * E + e] = out[i];
    if (dlp != nullptr && e < EP) {
      uint32_t hi, mid, lo;
      split3(e < E ? out[i] : 0.f, hi, mid, lo);
      uint16_t* row = dlp + (size_t)t * 3 * EP;
      row[e] = (uint16_t)hi;
      row[EP + e] = (uint16_t)mid;
      row[2 * EP + e] = (uint16_t)lo;
    }
  }
}

// Router weight gradient, one workgroup per (512 h block, 16 expert block,
// token split): thread tid owns h = h0 + 2 tid, h0 + 2 tid + 1 and 16
// experts; dl of 64 tokens at a time is staged in LDS and read as broadcasts.
// The split's sums go to part[s][H][E] (and db's to partb[s][E]).
constexpr int kWgH = 512, kWgE = 16, kWgT = 64;

template <bool BF16>
__global__ __launch_bounds__(256) void router_wgrad(const void* __restrict__ x,
                                                    const float* __restrict__ dl, int T, int H,
                                                    int E, int S, float* __restrict__ part,
                                                    float* __restrict__ partb) {
  __shared__ float dls[kWgT][kWgE];
  __shared__ __attribute__((aligned(16))) float stg[kWgH][kWgE];   // the partials, for the store
  const int tid = threadIdx.x;
  const int HB = (H + kWgH - 1) / kWgH, EB = (E + kWgE - 1) / kWgE;
  const int hb = blockIdx.x % HB, eb = (blockIdx.x / HB) % EB, s = blockIdx.x / (HB * EB);
  const int t_begin = (int)((long)s * T / S), t_end = (int)((long)(s + 1) * T / S);
  const int h = hb * kWgH + 2 * tid;
  const int e0 = eb * kWgE;
  float acc[2][kWgE];
#pragma unroll
  for (int e = 0; e < kWgE; ++e) acc[0][e] = acc[1][e] = 0.f;
  // workgroups of the first h block also sum dl over their tokens (db_r):
  // thread e < 16 adds column e of each staged batch
  const bool bias_thread = hb == 0 && tid < kWgE;
  float accb1 = 0.f;
  for (int tb = t_begin; tb < t_end; tb += kWgT) {
    const int nt = min(kWgT, t_end - tb);
    __syncthreads();
    for (int q = tid; q < kWgT * kWgE; q += 256) {
      const int tt = q / kWgE, e = q % kWgE;
      dls[tt][e] = (tt < nt && e0 + e < E) ? dl[(size_t)(tb + tt) * E + e0 + e] : 0.f;
    }
    __syncthreads();
    // 16 tokens' x values are loaded before any is used (the loads overlap)
    for (int tt0 = 0; tt0 < nt; tt0 += 16) {
      float xv[16][2];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        xv[u][0] = xv[u][1] = 0.f;
        if (tt0 + u < nt && h < H) {
          if constexpr (BF16) {
            const uint32_t v =
                *(const uint32_t*)((const uint16_t*)x + (size_t)(tb + tt0 + u) * H + h);
            xv[u][0] = bf16_to_f32(v & 0xFFFFu);
            xv[u][1] = bf16_to_f32(v >> 16);
          } else {
            const float* r = (const float*)x + (size_t)(tb + tt0 + u) * H + h;
            xv[u][0] = r[0];
            xv[u][1] = r[1];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
#pragma unroll
        for (int e = 0; e < kWgE; ++e) {
          const float d = dls[tt0 + u][e];          // 0 past nt
          acc[0][e] = __builtin_fmaf(xv[u][0], d, acc[0][e]);
          acc[1][e] = __builtin_fmaf(xv[u][1], d, acc[1][e]);
        }
      }
    }
    if (bias_thread)
      for (int tt = 0; tt < nt; ++tt) accb1 += dls[tt][tid];
  }
  // partials out through LDS: each thread holds two h rows of 16 experts;
  // stored as 16-byte runs, four lanes per 64-byte row piece (straight from
  // the registers every lane would write 4 bytes into a different row)
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < kWgE; e += 4)
      *(float4*)&stg[2 * tid + r][e] =
          make_float4(acc[r][e], acc[r][e + 1], acc[r][e + 2], acc[r][e + 3]);
  __syncthreads();
  const bool full_e = e0 + kWgE <= E && E % 4 == 0;
  for (int q = tid; q < kWgH * (kWgE / 4); q += 256) {
    const int hl = q / (kWgE / 4), c = (q % (kWgE / 4)) * 4;
    const int hh = hb * kWgH + hl;
    if (hh >= H) continue;
    float* dst = part + ((size_t)s * H + hh) * E + e0 + c;
    const float4 v = *(const float4*)&stg[hl][c];
    if (full_e) {
      *(float4*)dst = v;
    } else {
      const float vv[4] = {v.x, v.y, v.z, v.w};
      for (int u = 0; u < 4; ++u)
        if (e0 + c + u < E) dst[u] = vv[u];
    }
  }
  if (bias_thread && e0 + tid < E) partb[(size_t)s * E + e0 + tid] = accb1;
}

// LDS row bytes for a tile row of `bytes`: padded (by multiples of 16) so
// that the 4 consecutive rows one transposed read covers (8 banks each) fall
// in different banks of the 64.
constexpr int pad_row(int bytes) {
  for (int pad = 0; pad < 256; pad += 16) {
    const int st = ((bytes + pad) / 4) % 64;
    bool ok = true;
    for (int m = 1; m < 4; ++m) {
      const int d = (m * st) % 64;
      if (d < 8 || d > 56) ok = false;
    }
    if (ok) return bytes + pad;
  }
  return bytes + 16;
}

// dW_r = x^T dl on the matrix cores, for bf16 tokens.  dl enters as its three
// bf16 planes (dlp [T][3][EP], written by router_bwd): each product of a bf16
// x with a plane is exact in fp32, so the fp32 accumulation of the three
// products gives x^T dl to fp32 accuracy.  One workgroup per (HB h block, EB
// expert block, token split); a K step stages 32 tokens' rows of x (HB
// columns) and of the three planes (EB columns each) in LDS.  Both operands
// are token-major, so the MFMA fragments (8 consecutive tokens of one h, or
// of one expert, per lane) come from transposed LDS reads.  Wave (wm, wn)
// owns MB x NB blocks of 16 h x 16 experts.  Waves of the first h block with
// wm = 0 also multiply an all-ones operand by the planes: every row of that
// product is the sum of dl over the split's tokens (db_r).  Loads run PF
// steps ahead in registers; the two LDS buffers alternate by step, one
// barrier per step.  The split's sums go to part[s][H][E] and partb[s][E].
template <int MB, int NB, int WM>
__global__ __launch_bounds__(256) void router_wgrad_mfma(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ dlp,
                                                         int T, int H, int E, int EP, int S,
                                                         float* __restrict__ part,
                                                         float* __restrict__ partb) {
  constexpr int WN = 4 / WM;
  constexpr int HB = WM * MB * 16, EB = WN * NB * 16;
  constexpr int XCH = HB / 8, PCH = 3 * EB / 8;               // 16-byte chunks per token row
  constexpr int XROW = pad_row(HB * 2), PROW = pad_row(3 * EB * 2);
  constexpr int XLD = (32 * XCH + 255) / 256, PLD = (32 * PCH + 255) / 256;
  constexpr int PF = 4;                                     // (even: the LDS buffer is p & 1)
  // (tiles whose chunks do not divide among the 256 threads: the spare
  // threads write into `spare`, through an address select, not a branch)
  constexpr bool XFULL = 32 * XCH % 256 == 0, PFULL = 32 * PCH % 256 == 0;
  __shared__ __attribute__((aligned(16))) char xs[2][32 * XROW];
  __shared__ __attribute__((aligned(16))) char ps[2][32 * PROW];
  __shared__ __attribute__((aligned(16))) char spare[XFULL && PFULL ? 16 : 256 * 16];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % WM, wn = wave / WM;
  const int HBn = (H + HB - 1) / HB, EBn = (E + EB - 1) / EB;
  const int hb = blockIdx.x % HBn, eb = (blockIdx.x / HBn) % EBn, s = blockIdx.x / (HBn * EBn);
  const int h0 = hb * HB, e0 = eb * EB;
  const int t_begin = (int)((long)s * T / S), t_end = (int)((long)(s + 1) * T / S);
  const int nst = (t_end - t_begin + 31) / 32;

  // this thread's chunks of a step, as buffer loads: a chunk past the
  // split's tokens, past H or past EP takes an offset past the descriptor's
  // end and reads zero.  Offsets are formed as a per-thread base plus the
  // step times the row stride, and selected without branches, so the loads
  // of later steps stay in flight while an earlier step is waited for.
  const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
  const __amdgpu_buffer_rsrc_t psrc = make_rsrc(dlp, (uint32_t)((size_t)T * 3 * EP * 2));
  const int ntok = t_end - t_begin;
  uint32_t xoff[XLD], poff[PLD];
  int xrow[XLD], prow[PLD];
#pragma unroll
  for (int u = 0; u < XLD; ++u) {
    const int q = tid + 256 * u, h = h0 + 8 * (q % XCH);
    const bool col = q < 32 * XCH && h < H;
    xrow[u] = col ? q / XCH : ntok;                            // (never valid)
    xoff[u] = (uint32_t)(((t_begin + q / XCH) * H + h) * 2);
  }
#pragma unroll
  for (int u = 0; u < PLD; ++u) {
    const int q = tid + 256 * u, c = q % PCH;
    const int pl = c / (EB / 8), e = e0 + 8 * (c % (EB / 8));
    const bool col = q < 32 * PCH && e < EP;
    prow[u] = col ? q / PCH : ntok;
    poff[u] = (uint32_t)((((t_begin + q / PCH) * 3 + pl) * EP + e) * 2);
  }
  const uint32_t xstep = 32u * (uint32_t)H * 2u, pstep = 32u * 3u * (uint32_t)EP * 2u;
  auto load = [&](int st, u32x4 (&xv)[XLD], u32x4 (&pv)[PLD]) {
#pragma unroll
    for (int u = 0; u < XLD; ++u) {
      const uint32_t off = st * 32 + xrow[u] < ntok ? xoff[u] + (uint32_t)st * xstep : kPastEnd;
      xv[u] = __builtin_amdgcn_raw_buffer_load_b128(xsrc, off, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < PLD; ++u) {
      const uint32_t off = st * 32 + prow[u] < ntok ? poff[u] + (uint32_t)st * pstep : kPastEnd;
      pv[u] = __builtin_amdgcn_raw_buffer_load_b128(psrc, off, 0, 0);
    }
  };
  auto store = [&](int buf, const u32x4 (&xv)[XLD], const u32x4 (&pv)[PLD]) {
#pragma unroll
    for (int u = 0; u < XLD; ++u) {
      const int q = tid + 256 * u;
      char* d = (XFULL || q < 32 * XCH) ? xs[buf] + (q / XCH) * XROW + (q % XCH) * 16
                                        : spare + tid * 16;
      *(u32x4*)d = xv[u];
    }
#pragma unroll
    for (int u = 0; u < PLD; ++u) {
      const int q = tid + 256 * u;
      char* d = (PFULL || q < 32 * PCH) ? ps[buf] + (q / PCH) * PROW + (q % PCH) * 16
                                        : spare + tid * 16;
      *(u32x4*)d = pv[u];
    }
  };

  f32x4 acc[MB][NB], accb[NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NB; ++j) accb[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool bias = hb == 0 && wm == 0;                        // (wave-uniform)
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0

  // transposed reads: lane group g = lane / 16 takes tokens 8 g .. 8 g + 7 of
  // the step (two reads of 4 rows), lane lane % 16 the column
  const int li = lane % 16;
  const int rd = 8 * (lane / 16) + li / 4, cb = (li % 4) * 8;
  u32x4 xr[PF][XLD], pr[PF][PLD];
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, xr[p], pr[p]);
  // (whole groups of PF steps, without a per-step guard that would make the
  // waits on the loads conservative: the steps past nst read zeros)
  for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int st = s0 + p;
      {
        const int buf = p & 1;
        store(buf, xr[p], pr[p]);
        load(st + PF, xr[p], pr[p]);
        __syncthreads();
        u32x4 a[MB], bf[3][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const char* xa = xs[buf] + rd * XROW + cb + (wm * MB + i) * 32;
          const u32x2 lo = read_tr(xa), hi = read_tr(xa + 4 * XROW);
          a[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const char* pb = ps[buf] + rd * PROW + cb + pl * EB * 2 + (wn * NB + j) * 32;
            const u32x2 lo = read_tr(pb), hi = read_tr(pb + 4 * PROW);
            bf[pl][j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < MB; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, bf[pl][j]),
                  acc[i][j], 0, 0, 0);
        if (bias) {
#pragma unroll
          for (int pl = 0; pl < 3; ++pl)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              accb[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, bf[pl][j]),
                  accb[j], 0, 0, 0);
        }
      }
    }
  }
  // D: lane holds column li (an expert) of rows 4 (lane / 16) + v (h)
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int e = e0 + (wn * NB + j) * 16 + li;
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = h0 + (wm * MB + i) * 16 + 4 * (lane / 16) + v;
        if (h < H) part[((size_t)s * H + h) * E + e] = acc[i][j][v];
      }
    if (bias && lane < 16) partb[(size_t)s * E + e] = accb[j][0];
  }
}

// dW_r[h][e] = sum over splits in order; stored in W_r's type.  The first
// E threads also finish db_r.
template <bool WBF16>
__global__ __launch_bounds__(256) void router_wgrad_reduce(const float* __restrict__ part,
                                                           const float* __restrict__ partb,
                                                           int H, int E, int S,
                                                           void* __restrict__ dw_r,
                                                           float* __restrict__ db_r) {
  const size_t n = (size_t)H * E;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part[(size_t)s * n + i];
    if constexpr (WBF16)
      ((uint16_t*)dw_r)[i] = (uint16_t)f32_to_bf16(v);
    else
      ((float*)dw_r)[i] = v;
  }
  if (db_r && blockIdx.x == 0 && threadIdx.x < E) {
    for (int e = threadIdx.x; e < E; e += 256) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) v += partb[(size_t)s * E + e];
      db_r[e] = v;
    }
  }
}

// W_r [H][E] -> W_r^T [E][H] (same type), 32x32 tiles through LDS, so that
// dx_finish reads W_r^T rows across the lanes.
template <typename Tw>
__global__ __launch_bounds__(256) void transpose_wr(const Tw* __restrict__ w, int H, int E,
                                                    Tw* __restrict__ wt) {
  __shared__ Tw tile[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;     // 32 x 8
  const int eb = blockIdx.x % ((E + 31) / 32), hb = blockIdx.x / ((E + 31) / 32);
#pragma unroll
  for (int r = 0; r < 32; r += 8) {
    const int h = hb * 32 + ty + r, e = eb * 32 + tx;
    if (h < H && e < E) tile[ty + r][tx] = w[(size_t)h * E + e];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 32; r += 8) {
    const int e = eb * 32 + ty + r, h = hb * 32 + tx;
    if (h < H && e < E) wt[(size_t)e * H + h] = tile[tx][ty + r];
  }
}

// dx for TB tokens x 1024 columns per workgroup: thread tid owns columns
// h0 + 4 tid .. + 3.  The router term sum_e dl[t][e] W_r^T[e][h] reads W_r^T
// rows (a wave covers 256 consecutive columns), 8 experts' loads in flight,
// with dl from LDS (broadcasts); the expert term adds the token's dispatched
// rows of dxp (slots in order).
constexpr int kDxH = 1024;

// 4 consecutive values of a W_r^T row as fp32
template <bool WBF16>
__device__ __forceinline__ void load_wrt4(const void* w_rt, size_t o, float (&w)[4]) {
  if constexpr (WBF16) {
    const u32x2 v = *(const u32x2*)((const uint16_t*)w_rt + o);
    w[0] = bf16_to_f32(v[0] & 0xFFFFu);
    w[1] = bf16_to_f32(v[0] >> 16);
    w[2] = bf16_to_f32(v[1] & 0xFFFFu);
    w[3] = bf16_to_f32(v[1] >> 16);
  } else {
    const f32x4 v = *(const f32x4*)((const float*)w_rt + o);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = v[q];
  }
}

// (dense dl: softmax-then-top-k gating; dx_finish_sparse below takes the
// top-k-then-softmax case, where dl is zero outside each token's k experts)
template <bool BF16, bool WBF16, int TB>
__global__ __launch_bounds__(256) void dx_finish(const void* __restrict__ dxp,
                                                 const int32_t* __restrict__ inv_pos,
                                                 const float* __restrict__ dl,
                                                 const void* __restrict__ w_rt, int T, int H,
                                                 int E, int k, void* __restrict__ dx) {
  extern __shared__ float dls[];      // [TB][E]
  const int tid = threadIdx.x;
  const int HB = (H + kDxH - 1) / kDxH;
  const int t0 = (blockIdx.x / HB) * TB;
  const int h = (blockIdx.x % HB) * kDxH + 4 * tid;
  const int nt = min(TB, T - t0);
  for (int q = tid; q < TB * E; q += 256) {
    const int tt = q / E;
    dls[q] = tt < nt ? dl[(size_t)(t0 + tt) * E + q % E] : 0.f;
  }
  __syncthreads();
  if (h >= H) return;
  float acc[TB][4];
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[tt][q] = 0.f;
  for (int e0 = 0; e0 < E; e0 += 8) {
    // (every load unconditional, rows past E clamped and their values
    // zeroed after the load: a load behind a branch makes the compiler wait
    // for all loads in flight before the next use)
    float wv[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float t4[4];
      load_wrt4<WBF16>(w_rt, (size_t)min(e0 + u, E - 1) * H + h, t4);
      const bool in = e0 + u < E;
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[u][q] = in ? t4[q] : 0.f;
    }
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float d = e0 + u < E ? dls[tt * E + e0 + u] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][q] = __builtin_fmaf(d, wv[u][q], acc[tt][q]);
      }
    }
  }
  const size_t es = BF16 ? 2 : 4;
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
    if (tt < nt) {
      const int t = t0 + tt;
      float v[4] = {acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]};
      // the slots' rows of dxp, 8 at a time: positions, then rows, loaded
      // together; added in slot order (a dropped slot, p < 0, adds nothing)
      for (int j0 = 0; j0 < k; j0 += 8) {
        int pj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int pv = inv_pos[(size_t)t * k + min(j0 + u, k - 1)];
          pj[u] = j0 + u < k ? pv : -1;
        }
        // (unconditional loads; a dropped or absent slot reads row 0 and adds
        // nothing)
        float r[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const char* src = (const char*)dxp + ((size_t)max(pj[u], 0) * H + h) * es;
          if constexpr (BF16) {
            const u32x2 q = *(const u32x2*)src;
            r[u][0] = bf16_to_f32(q[0] & 0xFFFFu);
            r[u][1] = bf16_to_f32(q[0] >> 16);
            r[u][2] = bf16_to_f32(q[1] & 0xFFFFu);
            r[u][3] = bf16_to_f32(q[1] >> 16);
          } else {
            const f32x4 q = *(const f32x4*)src;
#pragma unroll
            for (int c = 0; c < 4; ++c) r[u][c] = q[c];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (pj[u] >= 0)
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] += r[u][c];
      }
      char* dst = (char*)dx + ((size_t)t * H + h) * es;
      if constexpr (BF16)
        *(u32x2*)dst = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      else
        *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

// dx with top-k-then-softmax gating (dl zero outside each token's k experts):
// one wave per (token, 512 columns), lane l owning columns 8 l .. 8 l + 7 of
// the chunk.  The wave fetches every slot's expert id, dispatched row and
// logit gradient dlk (router_bwd's per-slot copy of dl[t, id]) with scalar
// loads in one round trip, and then every slot's W_r^T row and dxp row are
// loaded before any is used, so the token's 2k row loads are in flight
// together.  Router term first (slots in order, fp32 FMAs), then the
// dispatched rows in slot order, as in dx_finish.
template <bool BF16, bool WBF16, int KM>
__global__ __launch_bounds__(256) void dx_finish_sparse(const void* __restrict__ dxp,
                                                        const int32_t* __restrict__ inv_pos,
                                                        const int32_t* __restrict__ ids,
                                                        const float* __restrict__ dlk,
                                                        const void* __restrict__ w_rt, int T,
                                                        int H, int E, int k,
                                                        void* __restrict__ dx) {
  const int lane = threadIdx.x % kWave;
  const int HC = (H + 511) / 512;
  // (wave-uniform: the slots' ids, rows and dl come by scalar loads)
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
  if (item >= T * HC) return;
  const int t = item / HC, h = (item % HC) * 512 + 8 * lane;
  int ej[KM], pj[KM];
  float dj[KM];
#pragma unroll
  for (int u = 0; u < KM; ++u) {
    ej[u] = u < k ? ids[(size_t)t * k + u] : -1;
    if ((unsigned)ej[u] >= (unsigned)E) ej[u] = -1;     // (an id outside [0, E) adds nothing)
    pj[u] = u < k ? inv_pos[(size_t)t * k + u] : -1;
    dj[u] = u < k ? dlk[(size_t)t * k + u] : 0.f;
  }
  const bool col = h < H;
  Raw8<WBF16> wv[KM];
  Raw8<BF16> rv[KM];
#pragma unroll
  for (int u = 0; u < KM; ++u) {
    wv[u].zero();
    rv[u].zero();
    if (ej[u] >= 0 && col) wv[u].load((const char*)w_rt + (size_t)ej[u] * H * (WBF16 ? 2 : 4), h / 8);
    if (pj[u] >= 0 && col) rv[u].load((const char*)dxp + (size_t)pj[u] * H * (BF16 ? 2 : 4), h / 8);
  }
  if (!col) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KM; ++u)
    if (ej[u] >= 0)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(dj[u], wv[u][c], acc[c]);
#pragma unroll
  for (int u = 0; u < KM; ++u)
    if (pj[u] >= 0)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += rv[u][c];
  store8<BF16>((char*)dx + (size_t)t * H * (BF16 ? 2 : 4), h / 8, acc);
}

template <bool BF16, bool WBF16, int TB>
void launch_dx_tb(const void* dxp, const int32_t* inv_pos, const float* dl, const void* w_rt,
                  int T, int H, int E, int k, void* dx, hipStream_t s) {
  const int HB = (H + kDxH - 1) / kDxH;
  dim3 g((unsigned)(((T + TB - 1) / TB) * HB)), b(256);
  const size_t lds = (size_t)TB * E * sizeof(float);
  hipLaunchKernelGGL((dx_finish<BF16, WBF16, TB>), g, b, lds, s, dxp, inv_pos, dl, w_rt, T, H, E,
                     k, dx);
}

template <bool BF16, bool WBF16, bool SPARSE>
void launch_dx(const void* dxp, const int32_t* inv_pos, const int32_t* ids, const float* dl,
               const float* dlk, const void* w_rt, int T, int H, int E, int k, void* dx,
               hipStream_t s) {
  if constexpr (SPARSE) {
    const long items = (long)T * ((H + 511) / 512);
    dim3 g((unsigned)((items + 3) / 4)), b(256);
#define MOE_DXS(KM_) \
  hipLaunchKernelGGL((dx_finish_sparse<BF16, WBF16, KM_>), g, b, 0, s, dxp, inv_pos, ids, dlk, \
                     w_rt, T, H, E, k, dx)
    if (k <= 2) MOE_DXS(2);
    else if (k <= 4) MOE_DXS(4);
    else if (k <= 8) MOE_DXS(8);
    else MOE_DXS(16);
#undef MOE_DXS
  } else {
    // tokens per workgroup: 16, fewer when that leaves the GPU without ~256
    // workgroups
    const long hb = (H + kDxH - 1) / kDxH;
    auto blocks = [&](int tb) { return ((T + tb - 1) / tb) * hb; };
#define MOE_DX(TB_) launch_dx_tb<BF16, WBF16, TB_>(dxp, inv_pos, dl, w_rt, T, H, E, k, dx, s)
    if (blocks(16) >= 256) MOE_DX(16);
    else if (blocks(8) >= 256) MOE_DX(8);
    else if (blocks(4) >= 256) MOE_DX(4);
    else MOE_DX(2);
#undef MOE_DX
  }
}

// zero fill with 16-byte stores (bytes a multiple of 16, base 16-byte aligned)
__global__ __launch_bounds__(256) void fill_zero16(u32x4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// dl's planes: E rounded up to 16 columns each
int planes_width(int E) { return (E + 15) / 16 * 16; }

// router_wgrad_mfma's tile (h x experts per workgroup) for E experts
void wgrad_mfma_tile(int E, int& hb, int& eb) {
  hb = E <= 16 ? 256 : 64;
  eb = E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : 128;
}

// token splits of router_wgrad_mfma: about one workgroup per CU, at least
// four K steps (128 tokens) per split
int wgrad_mfma_splits(int T, int H, int E) {
  int hb, eb;
  wgrad_mfma_tile(E, hb, eb);
  const int blocks = ((H + hb - 1) / hb) * ((E + eb - 1) / eb);
  return std::max(1, std::min((T + 127) / 128, (256 + blocks - 1) / blocks));
}

int wgrad_splits(int T, int H, int E) {
  // about 1024 workgroups (four per CU), at least 32 tokens per split
  const int blocks = ((H + kWgH - 1) / kWgH) * ((E + kWgE - 1) / kWgE);
  const int s = std::max(1, std::min(T / 32, 1024 / std::max(1, blocks)));
  return std::max(1, std::min(s, std::max(1, T)));
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>(4096, (n + 255) / 256);
  hipLaunchKernelGGL(fill_zero16, dim3(blocks), dim3(256), 0, s, (u32x4*)p, n);
  return hipGetLastError();
}

size_t router_wgrad_ws_bytes(int T, int H, int E) {
  const int S = std::max(wgrad_splits(T, H, E), wgrad_mfma_splits(T, H, E));
  return align_up((size_t)S * H * E * sizeof(float)) + align_up((size_t)S * E * sizeof(float));
}

size_t router_planes_bytes(int T, int E) {
  return (size_t)T * 3 * planes_width(E) * sizeof(uint16_t);
}

hipError_t launch_combine_bwd(const void* dy, const void* yp, const int32_t* inv_pos,
                              const float* w, int T, int H, int k, bool bf16, float* dw,
                              void* dyp, hipStream_t s) {
  const int pairs = T * k;
  if (pairs == 0) return hipSuccess;
  dim3 g((pairs + 3) / 4), b(256);
  if (bf16) hipLaunchKernelGGL((combine_bwd<true>), g, b, 0, s, dy, yp, inv_pos, w, T, H, k, dw, dyp);
  else hipLaunchKernelGGL((combine_bwd<false>), g, b, 0, s, dy, yp, inv_pos, w, T, H, k, dw, dyp);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* ids, const float* w,
                             const float* dw, int T, int E, int k, bool softmax_all, float* dl,
                             uint16_t* dlp, float* dlk, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 g((T + 3) / 4), b(256);
  const int npl = (E + kWave - 1) / kWave;
  const int sa = softmax_all ? 1 : 0;
  const int EP = planes_width(E);
#define MOE_RB(N_) \
  hipLaunchKernelGGL((router_bwd<N_>), g, b, 0, s, logits, ids, w, dw, T, E, k, sa, dl, dlp, EP, \
                     softmax_all ? nullptr : dlk)
  if (npl <= 1) MOE_RB(1);
  else if (npl <= 2) MOE_RB(2);
  else if (npl <= 4) MOE_RB(4);
  else if (npl <= 8) MOE_RB(8);
  else MOE_RB(16);
#undef MOE_RB
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const void* x, const float* dl, const uint16_t* dlp, int T,
                               int H, int E, bool x_bf16, bool w_bf16, void* dw_r, float* db_r,
                               void* ws, hipStream_t s) {
  // (the MFMA kernel's buffer offsets are 32-bit: x and the planes below 2 GB)
  const bool mfma = x_bf16 && dlp != nullptr && (size_t)T * H * 2 < ((size_t)1 << 31) &&
                    router_planes_bytes(T, E) < ((size_t)1 << 31);
  const int S = mfma ? wgrad_mfma_splits(T, H, E) : wgrad_splits(T, H, E);
  float* part = (float*)ws;
  float* partb = (float*)((char*)ws + align_up((size_t)S * H * E * sizeof(float)));
  dim3 b(256);
  if (mfma) {
    int hb, eb;
    wgrad_mfma_tile(E, hb, eb);
    dim3 g((unsigned)(((H + hb - 1) / hb) * ((E + eb - 1) / eb) * S));
    const uint16_t* xb = (const uint16_t*)x;
    const int EP = planes_width(E);
    if (E <= 16)
      hipLaunchKernelGGL((router_wgrad_mfma<4, 1, 4>), g, b, 0, s, xb, dlp, T, H, E, EP, S, part, partb);
    else if (E <= 32)
      hipLaunchKernelGGL((router_wgrad_mfma<1, 2, 4>), g, b, 0, s, xb, dlp, T, H, E, EP, S, part, partb);
    else if (E <= 64)
      hipLaunchKernelGGL((router_wgrad_mfma<2, 2, 2>), g, b, 0, s, xb, dlp, T, H, E, EP, S, part, partb);
    else
      hipLaunchKernelGGL((router_wgrad_mfma<4, 2, 1>), g, b, 0, s, xb, dlp, T, H, E, EP, S, part, partb);
  } else {
    const int HB = (H + kWgH - 1) / kWgH, EB = (E + kWgE - 1) / kWgE;
    dim3 g((unsigned)(HB * EB * S));
    if (x_bf16) hipLaunchKernelGGL((router_wgrad<true>), g, b, 0, s, x, dl, T, H, E, S, part, partb);
    else hipLaunchKernelGGL((router_wgrad<false>), g, b, 0, s, x, dl, T, H, E, S, part, partb);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t n = (size_t)H * E;
  dim3 g2((unsigned)((n + 255) / 256));
  if (w_bf16) hipLaunchKernelGGL((router_wgrad_reduce<true>), g2, b, 0, s, part, partb, H, E, S, dw_r, db_r);
  else hipLaunchKernelGGL((router_wgrad_reduce<false>), g2, b, 0, s, part, partb, H, E, S, dw_r, db_r);
  return hipGetLastError();
}

hipError_t launch_dx_finish(const void* dxp, const int32_t* inv_pos, const int32_t* ids,
                            const float* dl, const float* dlk, const void* w_r, int T, int H,
                            int E, int k, bool bf16, bool w_bf16, void* w_rt, void* dx,
                            hipStream_t s) {
  const bool sparse = dlk != nullptr;
  if (T == 0) return hipSuccess;
  dim3 gt((unsigned)(((E + 31) / 32) * ((H + 31) / 32))), b(256);
  if (w_bf16)
    hipLaunchKernelGGL((transpose_wr<uint16_t>), gt, b, 0, s, (const uint16_t*)w_r, H, E,
                       (uint16_t*)w_rt);
  else
    hipLaunchKernelGGL((transpose_wr<float>), gt, b, 0, s, (const float*)w_r, H, E,
                       (float*)w_rt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
#define MOE_DX(B_, W_, S_) launch_dx<B_, W_, S_>(dxp, inv_pos, ids, dl, dlk, w_rt, T, H, E, k, dx, s)
  if (bf16) {
    if (w_bf16) { if (sparse) MOE_DX(true, true, true); else MOE_DX(true, true, false); }
    else { if (sparse) MOE_DX(true, false, true); else MOE_DX(true, false, false); }
  } else {
    if (sparse) MOE_DX(false, false, true); else MOE_DX(false, false, false);
  }
#undef MOE_DX
  return hipGetLastError();
}

}  // namespace moe
