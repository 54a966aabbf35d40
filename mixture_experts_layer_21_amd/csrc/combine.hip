// Combine (fused MoE article, ScatterWithWeights): every token's k expert
// rows, scaled by their gate weights, accumulated into y.  The article adds
// into y expert by expert; here it is the equivalent gather form, one wave
// per token summing its k rows in slot order in fp32 (no atomics, so the
// result is deterministic), then one rounded store per element.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// bf16: lane handles 8 elements (16 B) per step
__global__ __launch_bounds__(256) void combine_bf16(const u32x4* __restrict__ yp,
                                                    const int32_t* __restrict__ inv_pos,
                                                    const float* __restrict__ w,
                                                    u32x4* __restrict__ y, int T, int H,
                                                    int k) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const int chunks = H / 8;
  for (int c = lane; c < chunks; c += kWave) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = inv_pos[(size_t)t * k + j];
      const float wj = w[(size_t)t * k + j];
      const u32x4 v = yp[(size_t)p * chunks + c];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(wj, bf16_to_f32(v[q] & 0xFFFFu), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wj, bf16_to_f32(v[q] >> 16), acc[2 * q + 1]);
      }
    }
    y[(size_t)t * chunks + c] = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
}

// fp32: lane handles 4 elements (16 B) per step
__global__ __launch_bounds__(256) void combine_f32(const float4* __restrict__ yp,
                                                   const int32_t* __restrict__ inv_pos,
                                                   const float* __restrict__ w,
                                                   float4* __restrict__ y, int T, int H,
                                                   int k) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const int chunks = H / 4;
  for (int c = lane; c < chunks; c += kWave) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int p = inv_pos[(size_t)t * k + j];
      const float wj = w[(size_t)t * k + j];
      const float4 v = yp[(size_t)p * chunks + c];
      acc.x = __builtin_fmaf(wj, v.x, acc.x);
      acc.y = __builtin_fmaf(wj, v.y, acc.y);
      acc.z = __builtin_fmaf(wj, v.z, acc.z);
      acc.w = __builtin_fmaf(wj, v.w, acc.w);
    }
    y[(size_t)t * chunks + c] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const void* yp, const int32_t* inv_pos, const float* w, int T,
                          int H, int k, bool bf16, void* y, hipStream_t s) {
  dim3 g((T + 3) / 4), b(256);
  if (bf16)
    hipLaunchKernelGGL(combine_bf16, g, b, 0, s, (const u32x4*)yp, inv_pos, w, (u32x4*)y, T, H, k);
  else
    hipLaunchKernelGGL(combine_f32, g, b, 0, s, (const float4*)yp, inv_pos, w, (float4*)y, T, H, k);
  return hipGetLastError();
}

}  // namespace moe
