// Routing + gating kernels (fused MoE article, section 1: router logits on
// the matrix unit, per-token TopK, softmax over the k selected scores; the
// routing article's scan fixes ties to the lower expert index).
//
// bf16 path
//   route_logits_bf16 MFMA 16x16x32 bf16 with fp32 accumulation.  A workgroup
//                     owns one expert group (TPW tiles of 16 experts) and one
//                     split of the H axis (KL rows) for 4 token tiles of 16,
//                     one per wave.  The W_r block [KL][16 TPW] is staged in
//                     LDS once in its natural k-major layout and read by the
//                     waves with transposed LDS reads (4 consecutive k of one
//                     expert per lane and read); the token operand comes
//                     straight from global memory.  Partial logits go to
//                     part[S][T][EP] (fp32, EP = E rounded up to 16).
//                     With an fp32 W_r (an fp32 router for bf16 tokens, the
//                     CANN article's section 4.2) each weight is staged as
//                     three bf16 planes, w = hi + mid + lo (hi and mid
//                     truncations, lo the rounded rest), and every k-step
//                     runs three MFMAs: each product x*part is exact in fp32,
//                     so the sum is an fp32-accumulated x . W_r.
// fp32 path: the logits come from the fp32 grouped GEMM in dense mode.
//
//   route_select      (route_select_rows for T >= 1024 and E <= 256: one
//                     token per row of 16 lanes, the same steps with the
//                     arg-max exchanges kept inside the row)
//                     one wave per token: sums the S partial logits in fixed
//                     order, adds the bias, takes k rounds of a 64-lane
//                     (value desc, index asc) arg-max, then the gate weights:
//                     the softmax of the k winners, or (softmax-then-top-k
//                     gating, CANN article section 2.1) their probabilities
//                     under the softmax over all E; writes ids[T,k], w[T,k]
//                     and, for a training forward, the logits[T,E].
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): in each group of 16 lanes,
// lane i addresses 8 bytes of row i/4 and receives column i of the 4x16 block
// those addresses cover.
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// fp32 -> (hi, mid, lo) bf16 bits with hi + mid + lo == w up to the rounding
// of lo (hi, mid: truncations; each remainder is exact in fp32).
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

template <int TPW, bool WF32>
__global__ __launch_bounds__(256) void route_logits_bf16(
    const uint16_t* __restrict__ x, const void* __restrict__ w_r_any,
    float* __restrict__ part, int T, int H, int E, int EP, int EG, int S, int KL) {
  // [NP][KL][16 TPW] bf16: one plane, or the hi/mid/lo planes of an fp32 W_r
  extern __shared__ __attribute__((aligned(16))) char wb[];
  constexpr int NP = WF32 ? 3 : 1;
  constexpr int ROW = TPW * 16 * 2;                            // bytes per k row
  const size_t plane = (size_t)KL * ROW;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int eg = blockIdx.x % EG;
  const int s = (blockIdx.x / EG) % S;
  const int tg = blockIdx.x / (EG * S);
  const int k_begin = s * KL;
  const int k_end = min(H, k_begin + KL);
  const int e0 = eg * TPW * 16;

  // stage W_r[k_begin:k_begin+KL, e0:e0+16 TPW]; rows past H and experts
  // past E are zero.  Each thread moves 8-expert chunks, SB of them per
  // batch with all the batch's loads issued before its LDS stores.
  {
    constexpr int CH = TPW * 2;                    // 8-expert chunks per row
    constexpr int SB = WF32 ? 4 : 8;               // chunks per thread per batch
    const bool vec = (E % 8) == 0;
    const int total = KL * CH;
    for (int q0 = threadIdx.x; q0 < total; q0 += SB * 256) {
      if constexpr (!WF32) {
        const uint16_t* w_r = (const uint16_t*)w_r_any;
        u32x4 v[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int q = q0 + u * 256;
          const int r = q / CH, c = q % CH;
          const int k = k_begin + r, e = e0 + c * 8;
          v[u] = u32x4{0, 0, 0, 0};
          if (q < total && k < k_end) {
            if (vec) {
              if (e < E) v[u] = *(const u32x4*)(w_r + (size_t)k * E + e);
            } else {
              uint16_t h[8];
#pragma unroll
              for (int t = 0; t < 8; ++t)
                h[t] = (e + t < E) ? w_r[(size_t)k * E + e + t] : (uint16_t)0;
              v[u] = u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                           h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
            }
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int q = q0 + u * 256;
          if (q < total) *(u32x4*)(wb + (q / CH) * ROW + (q % CH) * 16) = v[u];
        }
      } else {
        const float* w_r = (const float*)w_r_any;
        float f[SB][8];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int q = q0 + u * 256;
          const int r = q / CH, c = q % CH;
          const int k = k_begin + r, e = e0 + c * 8;
          if (q < total && k < k_end && vec && e < E) {
            const float4 a = *(const float4*)(w_r + (size_t)k * E + e);
            const float4 b = *(const float4*)(w_r + (size_t)k * E + e + 4);
            f[u][0] = a.x; f[u][1] = a.y; f[u][2] = a.z; f[u][3] = a.w;
            f[u][4] = b.x; f[u][5] = b.y; f[u][6] = b.z; f[u][7] = b.w;
          } else {
#pragma unroll
            for (int t = 0; t < 8; ++t)
              f[u][t] = (q < total && k < k_end && e + t < E) ? w_r[(size_t)k * E + e + t] : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int q = q0 + u * 256;
          if (q >= total) continue;
          const int r = q / CH, c = q % CH;
          uint32_t hi[8], mid[8], lo[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) split3(f[u][t], hi[t], mid[t], lo[t]);
          *(u32x4*)(wb + r * ROW + c * 16) =
              u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
          *(u32x4*)(wb + plane + r * ROW + c * 16) =
              u32x4{mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16), mid[4] | (mid[5] << 16), mid[6] | (mid[7] << 16)};
          *(u32x4*)(wb + 2 * plane + r * ROW + c * 16) =
              u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
        }
      }
    }
  }
  __syncthreads();

  const int tt = tg * 4 + wave;
  if (tt * 16 >= T) return;
  const int tok = min(tt * 16 + (lane % 16), T - 1);
  const int kl = (lane / 16) * 8;
  const uint16_t* xr = x + (size_t)tok * H + kl;
  // B operand: lane holds expert e0 + 16 j + lane%16 and k = 8 (lane/16) + 0..7
  // of the step, as two transposed reads of 4 rows each
  const int li = lane % 16;
  const int rd_off = (8 * (lane / 16) + li / 4) * ROW + (li % 4) * 8;

  f32x4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{};

  // token rows: PF K steps of loads in flight ahead of the MFMAs (each step's
  // 16 bytes per lane would otherwise wait a full memory latency)
  constexpr int PF = 8;
  const int nst = (k_end - k_begin + 31) / 32;
  auto load_x = [&](int st) -> u32x4 {
    const int k0 = k_begin + st * 32;
    return (st < nst && k0 + kl < k_end) ? *(const u32x4*)(xr + k0) : u32x4{0, 0, 0, 0};
  };
  u32x4 abuf[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) abuf[p] = load_x(p);
  for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int st = s0 + p;
      if (st < nst) {
        const u32x4 a = abuf[p];
        abuf[p] = load_x(st + PF);
        const char* base = wb + st * 32 * ROW + rd_off;
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) {
#pragma unroll
          for (int j = 0; j < TPW; ++j) {
            const u32x2 lo = lds_read_tr(base + pl * plane + j * 32);
            const u32x2 hi = lds_read_tr(base + pl * plane + 4 * ROW + j * 32);
            const u32x4 b = {lo[0], lo[1], hi[0], hi[1]};
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, b),
                                                             acc[j], 0, 0, 0);
          }
        }
      }
    }
  }
  // D: lane holds expert column lane%16 of tile j, token rows 4*(lane/16)+v
  const int NET = EP / 16;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    if (eg * TPW + j >= NET) continue;
    const int e = e0 + j * 16 + (lane % 16);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = tt * 16 + (lane / 16) * 4 + v;
      if (t < T) part[((size_t)s * T + t) * EP + e] = acc[j][v];
    }
  }
}

// (value, expert) pair of the lane DPP control CTRL names (every lane active)
template <int CTRL>
__device__ __forceinline__ void dpp_pair(float v, int e, float& ov, int& oe) {
  ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  oe = __builtin_amdgcn_update_dpp(0, e, CTRL, 0xF, 0xF, false);
}

// keep the larger value, on equal values the lower expert
__device__ __forceinline__ void take_better(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) {
    bv = ov;
    be = oe;
  }
}

// Arg-max over the wave of (value desc, expert asc); every lane ends with
// the winner.  Within each row of 16 lanes: the partner at lane ^ 1 and ^ 2
// (quad permutes), then the mirrored lane of the other quad (half-row mirror)
// and of the other half-row (row mirror); across rows: the four row winners
// read from lanes 0, 16, 32 and 48.
// The winner is unique, so the order of the exchanges does not matter.
__device__ __forceinline__ void wave_argmax(float& bv, int& be) {
  float ov;
  int oe;
  dpp_pair<0xB1>(bv, be, ov, oe);     // quad_perm [1,0,3,2]
  take_better(bv, be, ov, oe);
  dpp_pair<0x4E>(bv, be, ov, oe);     // quad_perm [2,3,0,1]
  take_better(bv, be, ov, oe);
  dpp_pair<0x141>(bv, be, ov, oe);    // row_half_mirror
  take_better(bv, be, ov, oe);
  dpp_pair<0x140>(bv, be, ov, oe);    // row_mirror
  take_better(bv, be, ov, oe);
  // every lane of a row now holds the row's winner: combine the four rows
  float rv = lane_f32(bv, 0);
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16)
    take_better(rv, re, lane_f32(bv, r), __builtin_amdgcn_readlane(be, r));
  bv = rv;
  be = re;
}

template <int NPL>
__global__ __launch_bounds__(256) void route_select(
    const float* __restrict__ part, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int EP,
    int S, int k, int softmax_all, float* __restrict__ logits) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;

  // sum the S partial logits in split order; all loads of a batch of SB
  // splits (for every expert of the lane, 64 values) are issued before any
  // is added
  constexpr int SB = 64 / NPL < 16 ? 64 / NPL : 16;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = 0.f;
  const size_t sstride = (size_t)T * EP;
  for (int s0 = 0; s0 < S; s0 += SB) {
    float q[NPL][SB];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      const float* p = part + ((size_t)s0 * T + t) * EP + e;
#pragma unroll
      for (int u = 0; u < SB; ++u) q[i][u] = (e < E && s0 + u < S) ? p[u * sstride] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
#pragma unroll
      for (int u = 0; u < SB; ++u) v[i] += q[i][u];
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) {
      if (bias) v[i] += bias[e];
      if (logits) logits[(size_t)t * E + e] = v[i];
    } else {
      v[i] = -__builtin_inff();
    }
  }
  uint32_t taken = 0;            // bit i: v[i] already selected
  float sel_v[16];
  int sel_e[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sel_v[j] = -__builtin_inff();
    sel_e[j] = 0;
    if (j < k) {
      float bv = -__builtin_inff();
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = lane + i * kWave;
        // within a lane e increases with i: strict ">" keeps the lower index
        if (e < E && !((taken >> i) & 1u) && (v[i] > bv || be == 0x7fffffff)) {
          bv = v[i];
          be = e;
        }
      }
      wave_argmax(bv, be);
      if ((be % kWave) == lane) taken |= 1u << (be / kWave);
      sel_v[j] = bv;
      sel_e[j] = be;
    }
  }
  // softmax over the k winners, or over all E experts (slot 0 holds the
  // maximum either way)
  const float m = sel_v[0];
  float sum = 0.f;
  if (softmax_all) {
    float part_sum = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + i * kWave < E) part_sum += expf(v[i] - m);
    sum = wave_sum(part_sum);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) sum += expf(sel_v[j] - m);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && lane == j) {
      ids[(size_t)t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = expf(sel_v[j] - m) / sum;
    }
  }
}

// Arg-max over the 16 lanes of each row (the first four exchanges of
// wave_argmax): every lane of the row ends with the row's winner.
__device__ __forceinline__ void row_argmax(float& bv, int& be) {
  float ov;
  int oe;
  dpp_pair<0xB1>(bv, be, ov, oe);     // quad_perm [1,0,3,2]
  take_better(bv, be, ov, oe);
  dpp_pair<0x4E>(bv, be, ov, oe);     // quad_perm [2,3,0,1]
  take_better(bv, be, ov, oe);
  dpp_pair<0x141>(bv, be, ov, oe);    // row_half_mirror
  take_better(bv, be, ov, oe);
  dpp_pair<0x140>(bv, be, ov, oe);    // row_mirror
  take_better(bv, be, ov, oe);
}

// Sum over the 16 lanes of each row, every lane ending with the total.
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// route_select for many tokens and E <= 256: one token per row of 16 lanes,
// four per wave.  Lane r of a row holds experts r, r + 16, ... (NV values,
// ascending), so each arg-max round is a lane-local scan plus four DPP
// exchanges inside the row, with no cross-row permutes; the split sums, bias,
// selection, tie rule, gate weights and outputs are those of route_select.
template <int NV>
__global__ __launch_bounds__(256) void route_select_rows(
    const float* __restrict__ part, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int EP,
    int S, int k, int softmax_all, float* __restrict__ logits) {
  const int rl = threadIdx.x % 16;
  const int t = (blockIdx.x * 256 + threadIdx.x) / 16;
  if (t >= T) return;   // whole rows leave together: the DPP partners stay in the row

  constexpr int SB = 64 / NV < 16 ? 64 / NV : 16;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = 0.f;
  const size_t sstride = (size_t)T * EP;
  for (int s0 = 0; s0 < S; s0 += SB) {
    float q[NV][SB];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = rl + i * 16;
      const float* p = part + ((size_t)s0 * T + t) * EP + e;
#pragma unroll
      for (int u = 0; u < SB; ++u) q[i][u] = (e < E && s0 + u < S) ? p[u * sstride] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int u = 0; u < SB; ++u) v[i] += q[i][u];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = rl + i * 16;
    if (e < E) {
      if (bias) v[i] += bias[e];
      if (logits) logits[(size_t)t * E + e] = v[i];
    } else {
      v[i] = -__builtin_inff();
    }
  }
  uint32_t taken = 0;            // bit i: v[i] already selected
  float sel_v[16];
  int sel_e[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    sel_v[j] = -__builtin_inff();
    sel_e[j] = 0;
    if (j < k) {
      float bv = -__builtin_inff();
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = rl + i * 16;
        // within a lane e increases with i: strict ">" keeps the lower index
        if (e < E && !((taken >> i) & 1u) && (v[i] > bv || be == 0x7fffffff)) {
          bv = v[i];
          be = e;
        }
      }
      row_argmax(bv, be);
      if ((be % 16) == rl) taken |= 1u << (be / 16);
      sel_v[j] = bv;
      sel_e[j] = be;
    }
  }
  const float m = sel_v[0];
  float sum = 0.f;
  if (softmax_all) {
    float part_sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (rl + i * 16 < E) part_sum += expf(v[i] - m);
    sum = row_sum(part_sum);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) sum += expf(sel_v[j] - m);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && rl == j) {
      ids[(size_t)t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = expf(sel_v[j] - m) / sum;
    }
  }
}

constexpr int kRowSelectMinT = 1024;

template <int NPL>
void launch_select(const float* part, const float* bias, int32_t* ids, float* w,
                   int T, int E, int EP, int S, int k, int softmax_all, float* logits,
                   hipStream_t s) {
  hipLaunchKernelGGL((route_select<NPL>), dim3((T + 3) / 4), dim3(256), 0, s,
                     part, bias, ids, w, T, E, EP, S, k, softmax_all, logits);
}

}  // namespace

RoutePlan plan_route(int T, int H, int E, bool bf16, bool wf32) {
  RoutePlan p;
  p.EP = (E + 15) / 16 * 16;
  const int NET = p.EP / 16;
  if (!bf16) {
    p.TPW = 0; p.EG = 1; p.S = 1; p.KL = H;
    return p;
  }
  int tpw = 1;
  // two expert groups at most (each group re-reads x)
  while (tpw < 16 && tpw * 2 < NET) tpw *= 2;
  p.TPW = tpw;
  p.EG = (NET + tpw - 1) / tpw;
  // about 2048 waves in all, and a staged W_r block of at most 64 KB
  // (KL * 32 TPW bytes per bf16 plane; three planes for an fp32 W_r)
  const int TT = (T + 15) / 16;
  const long base_items = std::max<long>(1, (long)TT * p.EG);
  int S = (int)std::min<long>(64, std::max<long>(1, (2048 + base_items - 1) / base_items));
  int KL = (H + S - 1) / S;
  KL = (KL + 31) / 32 * 32;
  KL = std::min(KL, (wf32 ? 512 : 2048) / tpw);
  p.KL = KL;
  p.S = (H + KL - 1) / KL;
  return p;
}

size_t route_ws_bytes(int T, int H, int E, bool bf16) {
  // enough for either router weight type
  const RoutePlan a = plan_route(T, H, E, bf16, false);
  const RoutePlan b = plan_route(T, H, E, bf16, bf16);
  return align_up((size_t)std::max(a.S, b.S) * T * a.EP * sizeof(float));
}

hipError_t launch_route(const void* x, const void* w_r, const float* bias,
                        int T, int H, int E, int k, bool bf16, bool wf32, bool softmax_all,
                        int32_t* ids, float* w, float* logits, void* ws, hipStream_t s) {
  const RoutePlan p = plan_route(T, H, E, bf16, wf32);
  float* part = (float*)ws;
  if (bf16) {
    const int TG = ((T + 15) / 16 + 3) / 4;
    dim3 g((unsigned)(TG * p.EG * p.S)), b(256);
    const size_t lds = (size_t)p.KL * p.TPW * 32 * (wf32 ? 3 : 1);
    const uint16_t* xb = (const uint16_t*)x;
#define MOE_ROUTE_LOGITS(TPW_)                                                              \
    if (wf32)                                                                                \
      hipLaunchKernelGGL((route_logits_bf16<TPW_, true>), g, b, lds, s, xb, w_r, part, T, H,  \
                         E, p.EP, p.EG, p.S, p.KL);                                          \
    else                                                                                     \
      hipLaunchKernelGGL((route_logits_bf16<TPW_, false>), g, b, lds, s, xb, w_r, part, T, H, \
                         E, p.EP, p.EG, p.S, p.KL)
    switch (p.TPW) {
      case 1: MOE_ROUTE_LOGITS(1); break;
      case 2: MOE_ROUTE_LOGITS(2); break;
      case 4: MOE_ROUTE_LOGITS(4); break;
      case 8: MOE_ROUTE_LOGITS(8); break;
      default: MOE_ROUTE_LOGITS(16); break;
    }
#undef MOE_ROUTE_LOGITS
  } else {
    hipError_t err = launch_gemm_f32((const float*)x, (const float*)w_r, part, nullptr, 1, T, H, E,
                                     p.EP, false, nullptr, s);
    if (err != hipSuccess) return err;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int sa = softmax_all ? 1 : 0;
  // many tokens, E <= 256: one token per row of 16 lanes (enough waves at
  // T / 4 to fill the GPU); otherwise one token per wave
  if (T >= kRowSelectMinT && E <= 256) {
    const int nv = (E + 15) / 16;
    const dim3 g((unsigned)((T + 15) / 16)), b(256);
#define MOE_SELECT_ROWS(NV_)                                                                        hipLaunchKernelGGL((route_select_rows<NV_>), g, b, 0, s, part, bias, ids, w, T, E, p.EP, p.S,                        k, sa, logits)
    if (nv <= 1) MOE_SELECT_ROWS(1);
    else if (nv <= 2) MOE_SELECT_ROWS(2);
    else if (nv <= 4) MOE_SELECT_ROWS(4);
    else if (nv <= 8) MOE_SELECT_ROWS(8);
    else MOE_SELECT_ROWS(16);
#undef MOE_SELECT_ROWS
    return hipGetLastError();
  }
  const int npl = (E + kWave - 1) / kWave;
  if (npl <= 1) launch_select<1>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s);
  else if (npl <= 2) launch_select<2>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s);
  else if (npl <= 4) launch_select<4>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s);
  else if (npl <= 8) launch_select<8>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s);
  else launch_select<16>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s);
  return hipGetLastError();
}

}  // namespace moe
