// Routing + gating kernels (fused MoE article, section 1: router logits on
// the matrix unit, per-token TopK, softmax over the k selected scores, in one
// kernel, so that the logits never make a round trip through HBM; the
// routing article's scan fixes ties to the lower expert index).
//
// bf16 path, E <= 128 in multiples of 8, H <= 4096, a bf16 W_r, and either
// E <= 16 (any T) or T >= 1024
//   route_fused       the whole router in one launch: one workgroup per tile
//                     of 16 tokens, its 8 waves splitting H, W_r read in
//                     whole rows into registers and transposed there,
//                     partial logits summed in LDS, then top-k and softmax in
//                     the same workgroup (see the kernel's comment).
//
// bf16 path, other shapes (E = 24 .. 128 with few tokens, where the
// one-launch form's workgroups, each reading all of W_r, are too few to
// hide its latency; more experts; an fp32 W_r)
//   route_logits_bf16 MFMA 16x16x32 bf16 with fp32 accumulation.  A workgroup
//                     owns one expert group (TPW tiles of 16 experts) and one
//                     split of the H axis (KL rows) for 8 token tiles of 16,
//                     one per wave.  The split's W_r rows [KL][16 TPW] are
//                     staged in LDS chunk by chunk (64 KB each) in their
//                     natural k-major layout and read by the waves with
//                     transposed LDS reads (4 consecutive k of one expert per
//                     lane and read); the token operand comes straight from
//                     global memory.  Partial logits go to part[S][T][EP]
//                     (fp32, EP = E rounded up to 16); many tokens take few
//                     splits, so that traffic stays small.
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

constexpr int kLogitWaves = 8;                    // token tiles of 16 per workgroup
constexpr int kLogitThreads = kLogitWaves * kWave;
constexpr int kLogitLds = 65536;                  // bytes of one staged W_r chunk

template <int TPW, bool WF32>
__global__ __launch_bounds__(kLogitThreads) void route_logits_bf16(
    const uint16_t* __restrict__ x, const void* __restrict__ w_r_any,
    float* __restrict__ part, int T, int H, int E, int EP, int EG, int S, int KL) {
  // [NP][KC][16 TPW] bf16: one plane, or the hi/mid/lo planes of an fp32 W_r
  extern __shared__ __attribute__((aligned(16))) char wb[];
  constexpr int NP = WF32 ? 3 : 1;
  constexpr int ROW = TPW * 16 * 2;                            // bytes per k row
  // rows per staged chunk: whole groups of 8 steps where the budget allows
  constexpr int RAW = kLogitLds / (NP * ROW);
  constexpr int KC = RAW >= 256 ? RAW / 256 * 256 : RAW / 32 * 32;
  constexpr int CST = KC / 32;                                 // K steps per chunk
  constexpr int PF = CST < 8 ? CST : 8;                        // token steps in flight
  static_assert(KC >= 32 && CST % PF == 0, "chunk of whole prefetch groups");
  constexpr size_t plane = (size_t)KC * ROW;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int eg = blockIdx.x % EG;
  const int s = (blockIdx.x / EG) % S;
  const int tg = blockIdx.x / (EG * S);
  const int k_begin = s * KL;
  const int k_end = min(H, k_begin + KL);
  const int nst = (k_end - k_begin + 31) / 32;
  const int e0 = eg * TPW * 16;

  // Token operand: wave w's tile of 16 tokens, lane l reading token l % 16,
  // k = 8 (l / 16) + 0..7 of each step, through a buffer descriptor that ends
  // at the tile's last token (tokens past T, and a tile wholly past T, read
  // zero; k past the split reads zero through the offset), so that no load
  // sits behind a branch.
  const int tt = tg * kLogitWaves + wave;
  const bool active = tt * 16 < T;
  const int ntok = active ? min(16, T - tt * 16) : 0;
  const __amdgpu_buffer_rsrc_t xs =
      make_rsrc(x + (size_t)min(tt * 16, T - 1) * H, (uint32_t)(ntok * H * 2));
  const int kl = (lane / 16) * 8;
  const uint32_t xo = (uint32_t)(((lane % 16) * H + kl) * 2);
  auto load_x = [&](int st) -> u32x4 {
    const int k0 = k_begin + st * 32;
    return __builtin_amdgcn_raw_buffer_load_b128(
        xs, k0 + kl < k_end ? xo + 2u * (uint32_t)k0 : kPastEnd, 0, 0);
  };
  // B operand: lane holds expert e0 + 16 j + lane%16 and k = 8 (lane/16) + 0..7
  // of the step, as two transposed reads of 4 rows each
  const int li = lane % 16;
  const int rd_off = (8 * (lane / 16) + li / 4) * ROW + (li % 4) * 8;

  f32x4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{};
  u32x4 abuf[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) abuf[p] = load_x(p);

  // The split's rows are staged and consumed chunk by chunk (KC rows, the
  // LDS budget); every wave takes part in staging and barriers.  A chunk's
  // steps run in whole prefetch groups: rows past the split are staged as
  // zero and their token loads read zero, so the extra steps add nothing.
  for (int c0 = 0; c0 < nst; c0 += CST) {
    const int c1 = min(nst, c0 + CST);
    const int rows = min(KC, (c1 - c0 + PF - 1) / PF * PF * 32);   // rows the steps read
    const int kc = k_begin + c0 * 32;
    if (c0 > 0) __syncthreads();                   // the previous chunk's reads are done
    // stage W_r[kc : kc + rows, e0 : e0 + 16 TPW]; rows past the split and
    // experts past E are zero.  Each thread moves 8-expert chunks, SB of them
    // per batch with all the batch's loads issued before its LDS stores.
    {
      constexpr int CH = TPW * 2;                  // 8-expert chunks per row
      constexpr int SB = WF32 ? 4 : 8;             // chunks per thread per batch
      const bool vec = (E % 8) == 0;
      const int total = rows * CH;
      for (int q0 = threadIdx.x; q0 < total; q0 += SB * kLogitThreads) {
        if constexpr (!WF32) {
          const uint16_t* w_r = (const uint16_t*)w_r_any;
          u32x4 v[SB];
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int q = q0 + u * kLogitThreads;
            const int r = q / CH, c = q % CH;
            const int k = kc + r, e = e0 + c * 8;
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
            const int q = q0 + u * kLogitThreads;
            if (q < total) *(u32x4*)(wb + (q / CH) * ROW + (q % CH) * 16) = v[u];
          }
        } else {
          const float* w_r = (const float*)w_r_any;
          float f[SB][8];
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int q = q0 + u * kLogitThreads;
            const int r = q / CH, c = q % CH;
            const int k = kc + r, e = e0 + c * 8;
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
            const int q = q0 + u * kLogitThreads;
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
    if (active) {
      for (int s0 = c0; s0 < c1; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
          const int st = s0 + p;
          const u32x4 a = abuf[p];
          abuf[p] = load_x(st + PF);
          const char* base = wb + (st - c0) * 32 * ROW + rd_off;
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) {
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
              const u32x2 lo = read_tr(base + pl * plane + j * 32);
              const u32x2 hi = read_tr(base + pl * plane + 4 * ROW + j * 32);
              const u32x4 b = {lo[0], lo[1], hi[0], hi[1]};
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                               __builtin_bit_cast(bf16x8, b),
                                                               acc[j], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  if (!active) return;
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

// keep the larger value, on equal values the lower expert (the values are
// never NaN: the selection ranks a NaN logit as -inf, so this is a total
// order and every lane that exchanges ends with the same winner)
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

// Token t's selection by one wave (see route_select); sid != nullptr: the
// ids also go to LDS, sid[t k + j].
template <int NPL>
__device__ __forceinline__ void select_token(const float* __restrict__ part,
                                             const float* __restrict__ bias,
                                             int32_t* __restrict__ ids, float* __restrict__ w,
                                             int T, int E, int EP, int S, int k,
                                             int softmax_all, float* __restrict__ logits, int t,
                                             int* sid) {
  const int lane = threadIdx.x % kWave;

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
  bool nan_seen = false;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) {
      if (bias) v[i] += bias[e];
      if (logits) logits[(size_t)t * E + e] = v[i];
      nan_seen |= __builtin_isnan(v[i]);
      v[i] = __builtin_isnan(v[i]) ? -__builtin_inff() : v[i];   // ranks as -inf
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
  // a token with a NaN logit keeps its k distinct experts, with NaN weights
  const bool tok_nan = __ballot(nan_seen) != 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && lane == j) {
      ids[(size_t)t * k + j] = sel_e[j];
      if (sid) sid[t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = tok_nan ? __builtin_nanf("") : expf(sel_v[j] - m) / sum;
    }
  }
}

template <int NPL>
__global__ __launch_bounds__(256) void route_select(
    const float* __restrict__ part, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int EP,
    int S, int k, int softmax_all, float* __restrict__ logits) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  select_token<NPL>(part, bias, ids, w, T, E, EP, S, k, softmax_all, logits, t, nullptr);
}

// The dropless dispatch of the T k pairs whose ids one workgroup holds in
// LDS (sid, pair i = t k + j): what perm_onepass computes, for a batch of a
// few tokens, without a launch of its own.  Expert e's pair count, a
// one-wave exclusive scan of the counts into doff[0..E] (scnt: LDS, E ints,
// then the offsets), and for each pair its rank among its expert's pairs in
// (token, slot) order: sorted_token[doff[e] + rank] = t, inv_pos[i] = that
// row.
__device__ void wg_dispatch(const int* sid, int T, int k, int E, int* scnt,
                            int32_t* __restrict__ doff, int32_t* __restrict__ dsorted,
                            int32_t* __restrict__ dinv) {
  __syncthreads();
  const int R = T * k, nth = blockDim.x, i0 = threadIdx.x;
  for (int e = i0; e < E; e += nth) {
    int c = 0;
    for (int q = 0; q < R; ++q) c += sid[q] == e ? 1 : 0;
    scnt[e] = c;
  }
  __syncthreads();
  if (i0 < kWave) {
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const int e = c0 + i0;
      const int v = e < E ? scnt[e] : 0;
      const int incl = wave_incl_scan(v);
      if (e < E) {
        scnt[e] = carry + incl - v;
        doff[e] = carry + incl - v;
      }
      carry += wave_bcast(incl, kWave - 1);
    }
    if (i0 == 0) doff[E] = carry;
  }
  __syncthreads();
  for (int q = i0; q < R; q += nth) {
    const int e = sid[q];
    int rank = 0;
    for (int q2 = 0; q2 < q; ++q2) rank += sid[q2] == e ? 1 : 0;
    const int p = scnt[e] + rank;
    dsorted[p] = q / k;
    dinv[q] = p;
  }
}

// route_select for a batch of at most 16 tokens (one workgroup, a wave per
// token) that also does the dispatch (wg_dispatch).
template <int NPL>
__global__ __launch_bounds__(1024) void route_select_dispatch(
    const float* __restrict__ part, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int EP,
    int S, int k, int softmax_all, float* __restrict__ logits, int32_t* __restrict__ doff,
    int32_t* __restrict__ dsorted, int32_t* __restrict__ dinv) {
  __shared__ int sid[16 * 16];
  __shared__ int scnt[1024];
  const int t = threadIdx.x / kWave;
  if (t < T)
    select_token<NPL>(part, bias, ids, w, T, E, EP, S, k, softmax_all, logits, t, sid);
  wg_dispatch(sid, T, k, E, scnt, doff, dsorted, dinv);
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

// One token per row of 16 lanes: lane rl of the row holds the summed logits
// (bias not yet added) of experts rl, rl + 16, ... (NV values, ascending).
// Adds the bias, keeps the logits when asked, takes the k winners by (value
// desc, expert asc) in k rounds of a lane-local scan plus the in-row DPP
// arg-max, then writes token t's ids and gate weights: the softmax of the k
// winners, or (softmax_all) their probabilities under the softmax over all E.
template <int NV>
__device__ __forceinline__ void select_row(float (&v)[NV], int rl, int t, const float* bias,
                                           int E, int k, int softmax_all, int32_t* ids,
                                           float* w, float* logits, int* sid = nullptr) {
  bool nan_seen = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = rl + i * 16;
    if (e < E) {
      if (bias) v[i] += bias[e];
      if (logits) logits[(size_t)t * E + e] = v[i];
      nan_seen |= __builtin_isnan(v[i]);
      v[i] = __builtin_isnan(v[i]) ? -__builtin_inff() : v[i];   // ranks as -inf
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
  // a token with a NaN logit keeps its k distinct experts, with NaN weights
  // (the row's 16 bits of the wave's ballot; rows leave only whole)
  const bool tok_nan = ((__ballot(nan_seen) >> (threadIdx.x & 48)) & 0xFFFFull) != 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && rl == j) {
      ids[(size_t)t * k + j] = sel_e[j];
      if (sid) sid[t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = tok_nan ? __builtin_nanf("") : expf(sel_v[j] - m) / sum;
    }
  }
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
  select_row<NV>(v, rl, t, bias, E, k, softmax_all, ids, w, logits);
}

// ---------------------------------------------------------------------------
// The router in one launch (many tokens, E <= 128 in multiples of 8, H <=
// 4096, bf16 W_r): one workgroup of 8 waves per tile of 16 tokens computes
// the tile's logits, top-k and gate weights; no partial logits leave the chip.
//   * Wave w owns the H range [32 NS w, 32 NS (w + 1)), in steps of 32 rows.
//   * W_r is read in its own [H][E] layout in whole rows: in load i of a
//     step, lane group g (lanes 16 g .. 16 g + 15) reads row 8 g + i, lane
//     c of the group experts 8 c .. 8 c + 7 (one 16-byte piece; a row of 128
//     experts is 256 contiguous bytes).  After the 8 loads of a step a lane
//     holds experts 8 c + e (e = 0..7) of rows 8 g + i (i = 0..7), an 8 x 8
//     block that it transposes in its own registers (byte permutes): for each
//     e, rows 8 g + 0..7 of expert 8 c + e, which is the MFMA B fragment of
//     lane 16 g + c for the 16 experts e, 8 + e, ..., 120 + e.  So one step
//     is 8 MFMAs, e = 0..7, each covering 16 experts strided by 8, and a wave
//     keeps the partial logits of all 128 experts in 8 accumulators.
//   * The token operand of a step (16 tokens x 32 rows) is read as 64-byte
//     runs (4 lanes per token) and moved into the MFMA A layout (lane l:
//     token l % 16, rows 8 (l / 16) + 0..7) with LDS permutes.
//   * Loads run D steps ahead of the MFMAs (the compiler waits on each
//     register as it is used).  At the end a wave leaves its 16 x 128 partial
//     logits in LDS; after one barrier the partials of the 8 waves are added
//     in wave order, and waves 0-3 run the selection with one token per row
//     of 16 lanes (select_row).
constexpr int kFuseWaves = 8;
constexpr int kFuseMaxE = 128;
constexpr int kFuseMaxH = kFuseWaves * 16 * 32;
constexpr int kFuseMinT = 1024;

// In each group of 8 lanes, lane i holds v = row i of an 8 x 8 block of bf16
// (element c in half c % 2 of dword c / 2); returns column i of the block in
// the same packing (dword p = rows 2p, 2p + 1).  sel and odd2 depend on the
// lane: sel = (lane & 1) ? 0x03020706 : 0x05040100, odd2 = (lane & 2) != 0.
__device__ __forceinline__ u32x4 transpose8(u32x4 v, uint32_t sel, bool odd2) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // lane ^ 1: the even lane keeps its low halves and takes its partner's,
    // the odd lane the high halves
    const uint32_t q = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[i], 0xB1, 0xF, 0xF, false);
    d[i] = __builtin_amdgcn_perm(q, v[i], sel);
  }
  // lanes 4 apart: lanes 0-3 of the group take dwords 0, 1 of lanes 4-7 into
  // their dwords 2, 3 (row_shl:4, banks 0 and 2), lanes 4-7 take dwords 2, 3
  // of lanes 0-3 into their dwords 0, 1 (row_shr:4, banks 1 and 3)
  const uint32_t n2 = (uint32_t)__builtin_amdgcn_update_dpp((int)d[2], (int)d[0], 0x104, 0xF, 0x5, false);
  const uint32_t n3 = (uint32_t)__builtin_amdgcn_update_dpp((int)d[3], (int)d[1], 0x104, 0xF, 0x5, false);
  const uint32_t n0 = (uint32_t)__builtin_amdgcn_update_dpp((int)d[0], (int)d[2], 0x114, 0xF, 0xA, false);
  const uint32_t n1 = (uint32_t)__builtin_amdgcn_update_dpp((int)d[1], (int)d[3], 0x114, 0xF, 0xA, false);
  // lanes 2 apart (quad_perm [2,3,0,1]): odd pairs' dwords 1, 3 <-> even pairs' 0, 2
  const uint32_t p0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)n0, 0x4E, 0xF, 0xF, false);
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)n1, 0x4E, 0xF, 0xF, false);
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)n2, 0x4E, 0xF, 0xF, false);
  const uint32_t p3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)n3, 0x4E, 0xF, 0xF, false);
  return u32x4{odd2 ? p1 : n0, odd2 ? n1 : p0, odd2 ? p3 : n2, odd2 ? n3 : p2};
}

// Sum of the 8 waves' partial logits (wave order) for waves 0-3's selection:
// one token per row of 16 lanes (select_row).
template <int EPMAX, int TOK = 16>
__device__ __forceinline__ void fused_select(const float (&part)[kFuseWaves][16][EPMAX],
                                             int wave, int lane, int t0, int T,
                                             const float* bias, int E, int k, int softmax_all,
                                             int32_t* ids, float* w, float* logits,
                                             int* sid = nullptr) {
  if (wave >= TOK / 4) return;
  const int tt = wave * 4 + lane / 16;
  const int t = t0 + tt;
  if (t >= T) return;   // whole rows leave together
  const int c = lane % 16;
  constexpr int NV = EPMAX / 16;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = c + 16 * i;
    float sum = 0.f;
    if (e < E) {
#pragma unroll
      for (int ww = 0; ww < kFuseWaves; ++ww) sum += part[ww][tt][e];
    }
    v[i] = sum;
  }
  select_row<NV>(v, c, t, bias, E, k, softmax_all, ids, w, logits, sid);
}

// E <= 16 (one expert tile): W_r is small, the token operand is the stream.
// Every load of a wave (its 16 tokens x 32 NS rows of x as 64-byte runs, its
// 32 NS rows of W_r) is issued at once.  A W_r load of a step reads rows
// 8 (lane / 16) + lane % 8, experts 8 ((lane % 16) / 8) + 0..7 (16 bytes;
// a row of 16 experts is 32 bytes), and transpose8 turns each group of 8
// lanes' 8 x 8 block into the MFMA B fragment (lane: expert lane % 16, rows
// 8 (lane / 16) + 0..7).  The token operand moves into the MFMA A layout with
// LDS permutes, as in route_fused.  TOK: tokens per workgroup, 16 or 8 (then
// the lanes of tokens 8-15 load nothing, the MFMA rows 8-15 stay zero and
// the workgroup streams half as much x: used when 16-token tiles would leave
// CUs without a workgroup).
//
// With doff != nullptr (one workgroup: T <= TOK) the kernel also does the
// dropless dispatch of its T k pairs (what perm_onepass computes, for a
// decode-sized batch, without a second launch): expert offsets doff[E+1],
// sorted_token and inv_pos, in the stable (token, slot) order.
template <int NS, int TOK = 16>
__global__ __launch_bounds__(kWave * kFuseWaves) void route_fused_small(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_r,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ logits, int T, int H, int E, int k, int softmax_all,
    int32_t* __restrict__ doff, int32_t* __restrict__ dsorted, int32_t* __restrict__ dinv) {
  __shared__ __attribute__((aligned(16))) float part[kFuseWaves][16][16];
  __shared__ int sid[16 * 16];                   // the tile's ids (dispatch only)
  __shared__ int scnt[16];                       // pairs per expert, then offsets
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * TOK;
  const int h0 = wave * NS * 32;
  // Buffer loads (an offset past the descriptor's end reads zero, so no
  // load sits behind a branch, which would make the compiler wait for all
  // loads in flight before the first use): lane reads token t0 + lane / 4
  // (tokens past the tile or past T read zero), 16 bytes at h = 8 (lane % 4)
  // of each step, and W_r row 8 (lane / 16) + lane % 8 of the step, experts
  // 8 ((lane % 16) / 8) + 0..7 (rows past H read zero)
  const __amdgpu_buffer_rsrc_t xs =
      make_rsrc(x + (size_t)t0 * H, (uint32_t)(min(TOK, T - t0) * H * 2));
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(w_r, (uint32_t)(H * E * 2));
  const uint32_t xo = (uint32_t)(((lane / 4) * H + 8 * (lane % 4)) * 2);
  const int xsrc = 4 * (4 * (lane % 16) + lane / 16);
  const int r_lane = 8 * (lane / 16) + lane % 8;
  const int e_lane = 8 * ((lane % 16) / 8);
  u32x4 xb[NS], wb[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int hs = h0 + 32 * st;
    xb[st] = __builtin_amdgcn_raw_buffer_load_b128(
        xs, hs + 8 * (lane % 4) < H ? xo + 2u * (uint32_t)hs : kPastEnd, 0, 0);
    const int h = hs + r_lane;
    wb[st] = __builtin_amdgcn_raw_buffer_load_b128(
        ws, e_lane < E ? (uint32_t)((h * E + e_lane) * 2) : kPastEnd, 0, 0);
  }
  const uint32_t sel = (lane & 1) ? 0x03020706u : 0x05040100u;
  const bool odd2 = (lane & 2) != 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    u32x4 xf;
#pragma unroll
    for (int q = 0; q < 4; ++q) xf[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)xb[st][q]);
    const u32x4 b = transpose8(wb[st], sel, odd2);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
  // D: lane holds expert lane % 16, tokens 4 (lane / 16) + v
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][4 * (lane / 16) + v][lane % 16] = acc[v];
  __syncthreads();
  fused_select<16, TOK>(part, wave, lane, t0, T, bias, E, k, softmax_all, ids, w, logits,
                        doff ? sid : nullptr);
  if (doff == nullptr) return;
  wg_dispatch(sid, T, k, E, scnt, doff, dsorted, dinv);   // (t0 = 0: the one workgroup)
}

template <int NS, int D>
__global__ __launch_bounds__(kWave * kFuseWaves) void route_fused(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_r,
    const float* __restrict__ bias, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ logits, int T, int H, int E, int k, int softmax_all) {
  __shared__ __attribute__((aligned(16))) float part[kFuseWaves][16][kFuseMaxE];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * 16;
  // The workgroups of one XCD (b, b + 8, ...) start at different rows of W_r:
  // wave w takes range (w + b / 8) % 8 and starts at step (b / 8) % NS, so
  // they do not all request the same L2 lines at once.  The per-range sums
  // are still added in a fixed order for each workgroup (deterministic).
  const int rot = blockIdx.x / 8;
  const int h0 = ((wave + rot) % kFuseWaves) * NS * 32;
  const int g = lane / 16, c = lane % 16;
  // Buffer loads, as in route_fused_small (no load behind a branch, so each
  // step waits for its own loads only).  Token operand: lane reads token
  // t0 + lane / 4 (tokens past T read zero), rows 8 (lane % 4) + 0..7 of the
  // step; the A fragment of lane l comes from lane 4 (l % 16) + l / 16.
  // W_r: row h of the step's 8 g + i, experts 8 c .. 8 c + 7 (rows past H
  // read zero).
  const __amdgpu_buffer_rsrc_t xs =
      make_rsrc(x + (size_t)t0 * H, (uint32_t)(min(16, T - t0) * H * 2));
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(w_r, (uint32_t)(H * E * 2));
  const uint32_t xo = (uint32_t)(((lane / 4) * H + 8 * (lane % 4)) * 2);
  const int xsrc = 4 * (4 * (lane % 16) + lane / 16);
  // (lanes of experts past E: every offset ORed past the end; a select per
  // load here became a branch around each load)
  const uint32_t wmask = 8 * c < E ? 0u : kPastEnd;
  auto load_step = [&](int st, u32x4 (&xb), u32x4 (&wb)[8]) {
    if (st >= NS) return;   // (a constant once the step loop is unrolled)
    const int hs = h0 + 32 * ((st + rot) % NS);
    xb = __builtin_amdgcn_raw_buffer_load_b128(
        xs, hs + 8 * (lane % 4) < H ? xo + 2u * (uint32_t)hs : kPastEnd, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = hs + 8 * g + i;
      wb[i] = __builtin_amdgcn_raw_buffer_load_b128(
          ws, (uint32_t)((h * E + 8 * c) * 2) | wmask, 0, 0);
    }
  };
  u32x4 xbuf[D], wbuf[D][8];
#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, xbuf[d], wbuf[d]);
  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int d = st % D;
    u32x4 xf;
#pragma unroll
    for (int q = 0; q < 4; ++q) xf[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)xbuf[d][q]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // rows 8 g + 2 p (low half) and 8 g + 2 p + 1 (high) of expert 8 c + e
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 b;
#pragma unroll
      for (int pq = 0; pq < 4; ++pq)
        b[pq] = __builtin_amdgcn_perm(wbuf[d][2 * pq + 1][e / 2], wbuf[d][2 * pq][e / 2], sel);
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf),
                                                       __builtin_bit_cast(bf16x8, b), acc[e], 0,
                                                       0, 0);
    }
    load_step(st + D, xbuf[d], wbuf[d]);
  }
  // D of MFMA e: lane holds tokens 4 (lane / 16) + v, expert 8 (lane % 16) + e;
  // for each v the 8 experts of the lane are contiguous: two 16-byte stores
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float* dst = &part[wave][4 * g + v][8 * c];
    *(f32x4*)dst = f32x4{acc[0][v], acc[1][v], acc[2][v], acc[3][v]};
    *(f32x4*)(dst + 4) = f32x4{acc[4][v], acc[5][v], acc[6][v], acc[7][v]};
  }
  __syncthreads();
  fused_select<kFuseMaxE>(part, wave, lane, t0, T, bias, E, k, softmax_all, ids, w, logits);
}

constexpr int kRowSelectMinT = 1024;

template <int NPL>
void launch_select(const float* part, const float* bias, int32_t* ids, float* w,
                   int T, int E, int EP, int S, int k, int softmax_all, float* logits,
                   hipStream_t s, int32_t* doff, int32_t* dsorted, int32_t* dinv) {
  if (doff != nullptr)   // (T <= 4: one workgroup, a wave per token)
    hipLaunchKernelGGL((route_select_dispatch<NPL>), dim3(1), dim3(kWave * T), 0, s, part, bias,
                       ids, w, T, E, EP, S, k, softmax_all, logits, doff, dsorted, dinv);
  else
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
  // about 512 workgroups in all (each a group of 8 token tiles, one expert
  // group and one split of H, which it stages through LDS in chunks): few
  // splits for many tokens (the partial logits are S * T * EP floats written
  // and read back), up to 64 for few
  const int TG = (T + 16 * kLogitWaves - 1) / (16 * kLogitWaves);
  const long items = std::max<long>(1, (long)TG * p.EG);
  int S = (int)std::min<long>(64, std::max<long>(1, (512 + items - 1) / items));
  // splits of whole prefetch groups of the logits kernel (8 steps, or its
  // chunk when that is shorter), so that no split runs steps of zero rows
  const int row = tpw * 32 * (wf32 ? 3 : 1);
  const int raw = kLogitLds / row;
  const int kc = raw >= 256 ? raw / 256 * 256 : raw / 32 * 32;
  const int grp = std::min(kc, 256);
  int KL = (H + S - 1) / S;
  KL = (KL + grp - 1) / grp * grp;
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

// (E <= 16: one launch at any T; measured against the two kernels at
// T = 1 .. 512, it saves 1-3 us.  E = 24 .. 128 at T = 64: 16.6 -> 24.5 us,
// so those keep the two kernels below kFuseMinT tokens.)
bool route_is_fused(int T, int H, int E, bool bf16, bool wf32) {
  return bf16 && !wf32 && (E <= 16 || T >= kFuseMinT) && E % 8 == 0 && E <= kFuseMaxE &&
         H <= kFuseMaxH;
}

// (route_fused_small up to 16 tokens, or route_select_dispatch after the
// logits kernel up to 4: one workgroup of a wave per token; at 16 tokens
// that one workgroup was slower than four of route_select plus the
// dispatch launch: 256 experts, k = 8 0.857 -> 0.863 ms per forward;
// 64 experts, k = 6 0.173 -> 0.176 ms; at one token it gained 0.6-3%)
bool route_dispatches(int T, int H, int E, bool bf16, bool wf32) {
  if (!bf16 || T < 1) return false;
  return route_is_fused(T, H, E, bf16, wf32) ? T <= 16 : T <= 4;
}

hipError_t launch_route(const void* x, const void* w_r, const float* bias,
                        int T, int H, int E, int k, bool bf16, bool wf32, bool softmax_all,
                        int32_t* ids, float* w, float* logits, void* ws, hipStream_t s,
                        int32_t* doff, int32_t* dsorted, int32_t* dinv) {
  if (doff != nullptr && !route_dispatches(T, H, E, bf16, wf32)) return hipErrorInvalidValue;
  if (route_is_fused(T, H, E, bf16, wf32)) {
    // one launch: NS steps of 32 rows per wave cover H (8 waves), loads D
    // steps ahead
    const int per_wave = (H + kFuseWaves - 1) / kFuseWaves;
    const int ns = (per_wave + 31) / 32;
    const dim3 g((unsigned)((T + 15) / 16)), b(kWave * kFuseWaves);
    const uint16_t* xb = (const uint16_t*)x;
    const uint16_t* wb = (const uint16_t*)w_r;
    const int sa = softmax_all ? 1 : 0;
#define MOE_ROUTE_FUSED(NS_, D_)                                                            \
    hipLaunchKernelGGL((route_fused<NS_, D_>), g, b, 0, s, xb, wb, bias, ids, w, logits, T, H, \
                       E, k, sa)
    // (dispatching: one workgroup, 8-token tiles up to 8 tokens, else 16)
    const bool tok8 = (T + 15) / 16 < 256 && !(doff != nullptr && T > 8);
    const dim3 g8((unsigned)((T + 7) / 8));
#define MOE_ROUTE_FUSED_SMALL(NS_)                                                             \
    do {                                                                                       \
      if (tok8)                                                                                \
        hipLaunchKernelGGL((route_fused_small<NS_, 8>), g8, b, 0, s, xb, wb, bias, ids, w,       \
                           logits, T, H, E, k, sa, doff, dsorted, dinv);                       \
      else                                                                                     \
        hipLaunchKernelGGL((route_fused_small<NS_>), g, b, 0, s, xb, wb, bias, ids, w, logits,   \
                           T, H, E, k, sa, doff, dsorted, dinv);                               \
    } while (0)
    if (E <= 16) {
      if (ns <= 1) MOE_ROUTE_FUSED_SMALL(1);
      else if (ns <= 2) MOE_ROUTE_FUSED_SMALL(2);
      else if (ns <= 4) MOE_ROUTE_FUSED_SMALL(4);
      else if (ns <= 8) MOE_ROUTE_FUSED_SMALL(8);
      else MOE_ROUTE_FUSED_SMALL(16);
    } else {
      if (ns <= 1) MOE_ROUTE_FUSED(1, 1);
      else if (ns <= 2) MOE_ROUTE_FUSED(2, 2);
      else if (ns <= 4) MOE_ROUTE_FUSED(4, 4);
      else if (ns <= 8) MOE_ROUTE_FUSED(8, 5);
      else MOE_ROUTE_FUSED(16, 4);
    }
#undef MOE_ROUTE_FUSED_SMALL
#undef MOE_ROUTE_FUSED
    return hipGetLastError();
  }
  const RoutePlan p = plan_route(T, H, E, bf16, wf32);
  float* part = (float*)ws;
  if (bf16) {
    const int TG = (T + 16 * kLogitWaves - 1) / (16 * kLogitWaves);
    dim3 g((unsigned)(TG * p.EG * p.S)), b(kLogitThreads);
    const size_t lds = kLogitLds;
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
  if (doff == nullptr && T >= kRowSelectMinT && E <= 256) {
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
  if (npl <= 1) launch_select<1>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s, doff,
                                    dsorted, dinv);
  else if (npl <= 2) launch_select<2>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s, doff,
                                    dsorted, dinv);
  else if (npl <= 4) launch_select<4>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s, doff,
                                    dsorted, dinv);
  else if (npl <= 8) launch_select<8>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s, doff,
                                    dsorted, dinv);
  else launch_select<16>(part, bias, ids, w, T, E, p.EP, p.S, k, sa, logits, s, doff, dsorted,
                          dinv);
  return hipGetLastError();
}

}  // namespace moe
