// Combine (fused MoE article, ScatterWithWeights): every token's k expert
// rows, scaled by their gate weights, accumulated into y.  The article adds
// into y expert by expert; here it is the equivalent gather form: one thread
// per (token, 16-byte chunk of the row) sums the token's k rows in slot order
// in fp32 (no atomics, so the result is deterministic), then makes one
// rounded store.  All k row loads of a thread are issued before any is used,
// and the grid has one thread per output chunk (bf16: two chunks, 64 apart,
// when the row allows it, for more loads in flight), so the pass is bound by
// HBM bandwidth rather than by load latency even for a handful of tokens.  A
// slot dropped by a capacity-limited dispatch (inv_pos < 0) adds nothing, and
// so does a row index past the T*k rows of yp (never read).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kMaxK = 16;

// bf16: a chunk is 8 elements; CPT chunks per thread (the wave's first
// chunk c, then c + 64, ...).  UNI: a token's threads fill whole waves, so
// the token index is wave-uniform and its k row positions and weights are
// fetched with scalar loads.
template <int CPT, bool UNI>
__global__ __launch_bounds__(256) void combine_bf16(const u32x4* __restrict__ yp,
                                                    const int32_t* __restrict__ inv_pos,
                                                    const float* __restrict__ w,
                                                    u32x4* __restrict__ y, int T, int chunks,
                                                    int k) {
  const int per_tok = chunks / CPT;                  // threads per token
  const int item = blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= T * per_tok) return;
  const int t = UNI ? __builtin_amdgcn_readfirstlane(item / per_tok) : item / per_tok;
  const int r = item % per_tok;
  const int c0 = (r / kWave) * (kWave * CPT) + (r % kWave);
  u32x4 v[kMaxK][CPT];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const int p = inv_pos[t * k + j];
      const bool in = (unsigned)p < (unsigned)(T * k);   // dropped slots (p < 0) add nothing
      wj[j] = in ? w[t * k + j] : 0.f;
#pragma unroll
      for (int u = 0; u < CPT; ++u)
        v[j][u] = in ? yp[(size_t)p * chunks + c0 + u * kWave] : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(wj[j], bf16_to_f32(v[j][u][q] & 0xFFFFu), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(wj[j], bf16_to_f32(v[j][u][q] >> 16), acc[2 * q + 1]);
        }
      }
    }
    y[(size_t)t * chunks + c0 + u * kWave] =
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
}

// fp32: a chunk is 4 elements
__global__ __launch_bounds__(256) void combine_f32(const float4* __restrict__ yp,
                                                   const int32_t* __restrict__ inv_pos,
                                                   const float* __restrict__ w,
                                                   float4* __restrict__ y, int T, int chunks,
                                                   int k) {
  const long item = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (long)T * chunks) return;
  const int t = (int)(item / chunks), c = (int)(item % chunks);
  float4 v[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      const int p = inv_pos[(size_t)t * k + j];
      const bool in = (unsigned)p < (unsigned)(T * k);   // dropped slots (p < 0) add nothing
      wj[j] = in ? w[(size_t)t * k + j] : 0.f;
      v[j] = in ? yp[(size_t)p * chunks + c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      acc.x = __builtin_fmaf(wj[j], v[j].x, acc.x);
      acc.y = __builtin_fmaf(wj[j], v[j].y, acc.y);
      acc.z = __builtin_fmaf(wj[j], v[j].z, acc.z);
      acc.w = __builtin_fmaf(wj[j], v[j].w, acc.w);
    }
  }
  y[item] = acc;
}

}  // namespace

hipError_t launch_combine(const void* yp, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, bool bf16, void* y, hipStream_t s) {
  const int chunks = bf16 ? H / 8 : H / 4;
  const long items = (long)T * chunks;
  dim3 g((unsigned)((items + 255) / 256)), b(256);
  if (bf16) {
    if (chunks % (2 * kWave) == 0 && k <= 8) {
      dim3 g2((unsigned)((items / 2 + 255) / 256));
      hipLaunchKernelGGL((combine_bf16<2, true>), g2, b, 0, s, (const u32x4*)yp, inv_pos, w,
                         (u32x4*)y, T, chunks, k);
    } else if (chunks % kWave == 0) {
      hipLaunchKernelGGL((combine_bf16<1, true>), g, b, 0, s, (const u32x4*)yp, inv_pos, w,
                         (u32x4*)y, T, chunks, k);
    } else {
      hipLaunchKernelGGL((combine_bf16<1, false>), g, b, 0, s, (const u32x4*)yp, inv_pos, w,
                         (u32x4*)y, T, chunks, k);
    }
  } else {
    hipLaunchKernelGGL(combine_f32, g, b, 0, s, (const float4*)yp, inv_pos, w, (float4*)y, T,
                       chunks, k);
  }
  return hipGetLastError();
}

}  // namespace moe
