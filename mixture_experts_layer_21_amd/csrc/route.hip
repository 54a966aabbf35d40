// Routing + gating kernels (fused MoE article, section 1: router logits on
// the matrix unit, per-token TopK, softmax over the k selected scores; the
// routing article's scan fixes ties to the lower expert index).
//
// bf16 path
//   wr_transpose      W_r[H,E] -> WrT[EP,H] (EP = E rounded up to 16, zero
//                     rows), so both MFMA operands are k-contiguous.
//   route_logits_bf16 MFMA 16x16x32 bf16 with fp32 accumulation.  Each wave is
//                     an independent work item (16 tokens, TPW expert tiles of
//                     16, one K split) and loads its operands straight from
//                     global memory (x from HBM once per expert group, WrT from
//                     L2).  Partial logits go to part[S][T][EP] (fp32).
// fp32 path: the logits come from the fp32 grouped GEMM in dense mode.
//
//   route_select      one wave per token: sums the S partial logits in fixed
//                     order, adds the bias, takes k rounds of a 64-lane
//                     (value desc, index asc) arg-max, then the softmax of the
//                     k winners; writes ids[T,k] and w[T,k].
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void wr_transpose(const uint16_t* __restrict__ wr,
                                                    uint16_t* __restrict__ wrT,
                                                    int H, int E, int EP) {
  __shared__ uint16_t tile[64][65];
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  for (int i = ty; i < 64; i += 4) {
    const int h = h0 + i, e = e0 + tx;
    tile[i][tx] = (h < H && e < E) ? wr[(size_t)h * E + e] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int e = e0 + i, h = h0 + tx;
    if (e < EP && h < H) wrT[(size_t)e * H + h] = tile[tx][i];
  }
}

template <int TPW>
__global__ __launch_bounds__(256) void route_logits_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wrT,
    float* __restrict__ part, int T, int H, int EP, int EG, int S, int KL,
    int n_items) {
  const int lane = threadIdx.x % kWave;
  const int item = blockIdx.x * 4 + threadIdx.x / kWave;
  if (item >= n_items) return;
  const int eg = item % EG;
  const int s = (item / EG) % S;
  const int tt = item / (EG * S);
  const int NET = EP / 16;

  const int k_begin = s * KL;
  const int k_end = min(H, k_begin + KL);
  const int tok = min(tt * 16 + (lane % 16), T - 1);
  const int kl = (lane / 16) * 8;
  const uint16_t* xr = x + (size_t)tok * H + kl;
  const uint16_t* wr[TPW];
  bool tile_ok[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int et = eg * TPW + j;
    tile_ok[j] = et < NET;
    wr[j] = wrT + (size_t)((tile_ok[j] ? et : 0) * 16 + (lane % 16)) * H + kl;
  }

  f32x4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = f32x4{};

  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    const bool ok = k0 + kl < k_end;
    const u32x4 a = ok ? *(const u32x4*)(xr + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const u32x4 b = ok ? *(const u32x4*)(wr[j] + k0) : u32x4{0, 0, 0, 0};
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b),
                                                       acc[j], 0, 0, 0);
    }
  }
  // D[i][j]: lane holds expert column j = lane%16, token rows 4*(lane/16)+v
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    if (!tile_ok[j]) continue;
    const int e = (eg * TPW + j) * 16 + (lane % 16);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = tt * 16 + (lane / 16) * 4 + v;
      if (t < T) part[((size_t)s * T + t) * EP + e] = acc[j][v];
    }
  }
}

template <int NPL>
__global__ __launch_bounds__(256) void route_select(
    const float* __restrict__ part, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ w, int T, int E, int EP,
    int S, int k) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;

  // sum the S partial logits in split order; the loads of a batch of 8
  // splits are all issued before any is added
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = 0.f;
  const size_t sstride = (size_t)T * EP;
  for (int s0 = 0; s0 < S; s0 += 8) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + i * kWave;
      if (e < E) {
        const float* p = part + ((size_t)s0 * T + t) * EP + e;
        float q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = (s0 + u < S) ? p[u * sstride] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) v[i] += q[u];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + i * kWave;
    if (e < E) {
      if (bias) v[i] += bias[e];
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
#pragma unroll
      for (int d = kWave / 2; d >= 1; d >>= 1) {
        const float ov = __shfl_xor(bv, d, kWave);
        const int oe = __shfl_xor(be, d, kWave);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be % kWave) == lane) taken |= 1u << (be / kWave);
      sel_v[j] = bv;
      sel_e[j] = be;
    }
  }
  // softmax over the k winners (slot 0 holds the maximum)
  const float m = sel_v[0];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) sum += expf(sel_v[j] - m);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k && lane == j) {
      ids[(size_t)t * k + j] = sel_e[j];
      w[(size_t)t * k + j] = expf(sel_v[j] - m) / sum;
    }
  }
}

template <int NPL>
void launch_select(const float* part, const float* bias, int32_t* ids, float* w,
                   int T, int E, int EP, int S, int k, hipStream_t s) {
  hipLaunchKernelGGL((route_select<NPL>), dim3((T + 3) / 4), dim3(256), 0, s,
                     part, bias, ids, w, T, E, EP, S, k);
}

}  // namespace

RoutePlan plan_route(int T, int H, int E, bool bf16) {
  RoutePlan p;
  p.EP = (E + 15) / 16 * 16;
  const int NET = p.EP / 16;
  if (!bf16) {
    p.TPW = 0; p.EG = 1; p.S = 1; p.KL = H;
    return p;
  }
  int tpw = 1;
  while (tpw < 16 && tpw * 4 < NET) tpw *= 2;
  p.TPW = tpw;
  p.EG = (NET + tpw - 1) / tpw;
  const int TT = (T + 15) / 16;
  const long base_items = std::max<long>(1, (long)TT * p.EG);
  int S = (int)std::min<long>(64, std::max<long>(1, (2048 + base_items - 1) / base_items));
  int KL = (H + S - 1) / S;
  KL = (KL + 31) / 32 * 32;
  p.KL = KL;
  p.S = (H + KL - 1) / KL;
  return p;
}

size_t route_ws_bytes(int T, int H, int E, bool bf16) {
  const RoutePlan p = plan_route(T, H, E, bf16);
  size_t b = align_up((size_t)p.S * T * p.EP * sizeof(float));
  if (bf16) b += align_up((size_t)p.EP * H * 2);
  return b;
}

hipError_t launch_route(const void* x, const void* w_r, const float* bias,
                        int T, int H, int E, int k, bool bf16, int32_t* ids,
                        float* w, void* ws, hipStream_t s) {
  const RoutePlan p = plan_route(T, H, E, bf16);
  float* part = (float*)ws;
  if (bf16) {
    uint16_t* wrT = (uint16_t*)((char*)ws + align_up((size_t)p.S * T * p.EP * sizeof(float)));
    hipLaunchKernelGGL(wr_transpose, dim3((H + 63) / 64, (p.EP + 63) / 64), dim3(256), 0, s,
                       (const uint16_t*)w_r, wrT, H, E, p.EP);
    const int TT = (T + 15) / 16;
    const int n_items = TT * p.EG * p.S;
    dim3 g((n_items + 3) / 4), b(256);
    switch (p.TPW) {
      case 1: hipLaunchKernelGGL(route_logits_bf16<1>, g, b, 0, s, (const uint16_t*)x, wrT, part, T, H, p.EP, p.EG, p.S, p.KL, n_items); break;
      case 2: hipLaunchKernelGGL(route_logits_bf16<2>, g, b, 0, s, (const uint16_t*)x, wrT, part, T, H, p.EP, p.EG, p.S, p.KL, n_items); break;
      case 4: hipLaunchKernelGGL(route_logits_bf16<4>, g, b, 0, s, (const uint16_t*)x, wrT, part, T, H, p.EP, p.EG, p.S, p.KL, n_items); break;
      case 8: hipLaunchKernelGGL(route_logits_bf16<8>, g, b, 0, s, (const uint16_t*)x, wrT, part, T, H, p.EP, p.EG, p.S, p.KL, n_items); break;
      default: hipLaunchKernelGGL(route_logits_bf16<16>, g, b, 0, s, (const uint16_t*)x, wrT, part, T, H, p.EP, p.EG, p.S, p.KL, n_items); break;
    }
  } else {
    hipError_t err = launch_gemm_f32((const float*)x, (const float*)w_r, part, nullptr, 1, T, H, E,
                                     p.EP, false, s);
    if (err != hipSuccess) return err;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int npl = (E + kWave - 1) / kWave;
  if (npl <= 1) launch_select<1>(part, bias, ids, w, T, E, p.EP, p.S, k, s);
  else if (npl <= 2) launch_select<2>(part, bias, ids, w, T, E, p.EP, p.S, k, s);
  else if (npl <= 4) launch_select<4>(part, bias, ids, w, T, E, p.EP, p.S, k, s);
  else if (npl <= 8) launch_select<8>(part, bias, ids, w, T, E, p.EP, p.S, k, s);
  else launch_select<16>(part, bias, ids, w, T, E, p.EP, p.S, k, s);
  return hipGetLastError();
}

}  // namespace moe
