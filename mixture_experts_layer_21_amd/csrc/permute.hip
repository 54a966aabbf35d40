// Dispatch kernels (fused MoE article, GatherTokensByExpert): group the
// R = T*k (token, slot) pairs by expert, keeping the article's order inside
// each expert (ascending token, then slot).  The article scans all pairs once
// per expert (O(E*R)); here it is a counting sort, O(R).  With a capacity
// (the article's [num_experts, expert_capacity] blocks; CANN MoE article,
// section 4.3) each expert keeps only its first `cap` pairs in that order.
//
//   perm_count   per chunk of CH pairs: expert histogram in LDS -> counts[b][e]
//   perm_scan    one workgroup: per-expert exclusive scan over chunks (each
//                chunk's rank base inside its expert) and over experts of
//                min(count, cap) (offsets); each expert's chunks are split
//                among P threads that scan their segments in parallel, then
//                the segment sums are scanned
//   perm_place   per chunk (one pair per thread): stable rank of each pair
//                among its expert's pairs (chunk base + wave ballots +
//                per-wave counts in LDS); rank < cap -> sorted_token[pos] = t,
//                inv_pos[t*k+j] = pos with pos = offsets[e] + rank; otherwise
//                the pair is dropped, inv_pos = -1
//   perm_gather  xp[p,:] = x[sorted_token[p],:] for p < offsets[E], 16-byte
//                copies, one wave per row
//   perm_small   for small layers (E <= 256, R <= 16384) the first three in one
//                workgroup of 16 waves, one launch: each wave ranks a
//                contiguous run of pairs, the per-wave counts are scanned,
//                then every pair is placed (the same stable order)
//
// All counts are integers: placement is exact and deterministic.  A pair
// whose id is outside [0, E) is dropped like a pair beyond the capacity
// (inv_pos = -1), so a bad id never indexes memory.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int CH = 256;    // pairs per chunk (one workgroup of 256 threads)

// Bits of an expert id (ids are in [0, E)).
__device__ __forceinline__ int id_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// The lanes of the wave whose `valid` value equals this lane's (0 for an
// invalid lane), for values below 2^nbits: one ballot per bit, each lane
// keeping the lanes that agree with it on that bit.  ceil(log2 E) ballots,
// however many distinct experts the wave holds.
__device__ __forceinline__ uint64_t wave_match(int v, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (v >> b) & 1;
    const uint64_t s = __ballot(valid && bit);
    m &= bit ? s : ~s;
  }
  return valid ? m : 0ull;
}

__global__ __launch_bounds__(256) void perm_count(const int32_t* __restrict__ ids, int R,
                                                  int E, int32_t* __restrict__ counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int end = min(R, (b + 1) * CH);
  for (int i = b * CH + threadIdx.x; i < end; i += 256) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);   // other ids: dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(size_t)b * E + e] = hist[e];
}

__global__ __launch_bounds__(1024) void perm_scan(const int32_t* __restrict__ counts,
                                                  int nchunks, int E, int cap,
                                                  int32_t* __restrict__ base,
                                                  int32_t* __restrict__ offsets) {
  __shared__ int seg[1024];     // [P][E]: segment sums, then segment bases
  __shared__ int tot[1024];     // per-expert totals, then expert offsets
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  const int P = max(1, 1024 / E);          // threads per expert
  const int e = t % E, p = t / E;
  const bool active = p < P && t < P * E;
  const int L = (nchunks + P - 1) / P;     // chunks per thread (contiguous)
  const int b0 = min(nchunks, p * L), b1 = min(nchunks, b0 + L);
  int sum = 0;
  if (active) {
    // (unrolled: several loads in flight instead of one per trip)
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += counts[(size_t)b * E + e];
  }
  if (active) seg[p * E + e] = sum;
  __syncthreads();
  if (t < E) {
    int run = 0;
    for (int q = 0; q < P; ++q) {
      const int v = seg[q * E + t];
      seg[q * E + t] = run;
      run += v;
    }
    tot[t] = run;
  }
  __syncthreads();
  // exclusive scan of the kept expert totals min(total, cap) (one thread per
  // expert, E <= 1024)
  const int lane = t % kWave, wave = t / kWave;
  const int v = t < E ? min(tot[t], cap) : 0;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  if (t < E) offsets[t] = wbase + incl - v;
  if (t == 0) {
    int all = 0;
    for (int w = 0; w < 16; ++w) all += wsum[w];
    offsets[E] = all;
  }
  // chunk bases: the rank, inside its expert, of each chunk's first pair
  if (active) {
    int run = seg[p * E + e];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      const int c = counts[(size_t)b * E + e];
      base[(size_t)b * E + e] = run;
      run += c;
    }
  }
}

__global__ __launch_bounds__(256) void perm_place(const int32_t* __restrict__ ids, int R,
                                                  int E, int k, int cap,
                                                  const int32_t* __restrict__ base,
                                                  const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ sorted_token,
                                                  int32_t* __restrict__ inv_pos) {
  extern __shared__ int sm[];
  int* running = sm;          // [E]: rank of the next pair of each expert
  int* wcnt = sm + E;         // [4][E]: pairs of each expert in each wave this round
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int b = blockIdx.x;
  const int nbits = id_bits(E);
  for (int e = tid; e < E; e += 256) {
    running[e] = base[(size_t)b * E + e];
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w * E + e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int r = 0; r < CH; r += 256) {
    const int i = b * CH + r + tid;
    const int my_e = i < R ? ids[i] : -1;
    const bool valid = i < R && (unsigned)my_e < (unsigned)E;
    if (i < R && !valid) inv_pos[i] = -1;   // an id outside [0, E): dropped
    // lanes of this wave holding the same expert
    const uint64_t peers = wave_match(my_e, valid, nbits);
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave * E + my_e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int r_e = running[my_e] + rank;
      for (int w = 0; w < wave; ++w) r_e += wcnt[w * E + my_e];
      if (r_e < cap) {
        const int pos = offsets[my_e] + r_e;
        sorted_token[pos] = i / k;
        inv_pos[i] = pos;
      } else {
        inv_pos[i] = -1;
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        add += wcnt[w * E + e];
        wcnt[w * E + e] = 0;
      }
      running[e] += add;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void perm_gather(const u32x4* __restrict__ x,
                                                   const int32_t* __restrict__ sorted_token,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   int R, int T, u32x4* __restrict__ xp,
                                                   int row_chunks) {
  const int lane = threadIdx.x % kWave;
  const int nwaves = gridDim.x * 4;
  const int n = min(max(offsets[E], 0), R);     // kept rows (never past the buffer)
  for (int p = blockIdx.x * 4 + threadIdx.x / kWave; p < n; p += nwaves) {
    const int t = sorted_token[p];
    u32x4* dst = xp + (size_t)p * row_chunks;
    if ((unsigned)t < (unsigned)T) {
      const u32x4* src = x + (size_t)t * row_chunks;
      for (int c = lane; c < row_chunks; c += kWave) dst[c] = src[c];
    } else {
      for (int c = lane; c < row_chunks; c += kWave) dst[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

constexpr int kSmallE = 256, kSmallR = 16384;   // ids fit 8 bits, ranks 16
constexpr int kSmallWaves = 16;

// One workgroup of 16 waves.  Wave w owns a contiguous run of 64-pair chunks
// (pairs in index order), ranks each pair inside its expert among the wave's
// pairs so far (ballot peers + a wave-private running count), and after one
// barrier the per-wave counts give both the expert totals and each wave's
// starting rank.  Every pair's id is loaded up front, so the only serial
// latency is the ranking arithmetic itself.
template <int kSmallChunks>   // 64-pair chunks per wave, at most
__global__ __launch_bounds__(1024) void perm_small(const int32_t* __restrict__ ids, int R, int E,
                                                   int k, int cap, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted_token,
                                                   int32_t* __restrict__ inv_pos) {
  __shared__ int wcnt[kSmallWaves][kSmallE];   // pairs per (wave, expert), then start ranks
  __shared__ int off_s[kSmallE];               // kept-row offset of each expert
  __shared__ int wsum[kSmallWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nch = (R + kWave - 1) / kWave;
  const int cpw = (nch + kSmallWaves - 1) / kSmallWaves;   // chunks per wave
  const int c0 = wave * cpw;
  const int nbits = id_bits(E);
  // pair j of this lane: its expert id, then (after ranking) rank << 8 | id
  // (ids < 256, ranks < 32768); -1 for no pair, -2 for an id outside [0, E)
  int pr[kSmallChunks];
#pragma unroll
  for (int j = 0; j < kSmallChunks; ++j) {
    const int i = (c0 + j) * kWave + lane;
    const int e = (j < cpw && i < R) ? ids[i] : -1;
    pr[j] = (j < cpw && i < R && (unsigned)e >= (unsigned)E) ? -2 : e;
  }
  for (int t = tid; t < kSmallWaves * E; t += 1024) wcnt[t / E][t % E] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int j = 0; j < kSmallChunks; ++j) {
    if (j < cpw) {
      const int e = pr[j];
      const bool valid = e >= 0;
      const uint64_t peers = wave_match(e, valid, nbits);
      const int before = __popcll(peers & lt_mask);
      const int cnt = valid ? wcnt[wave][e] : 0;
      if (valid) pr[j] = (cnt + before) << 8 | e;
      // one lane per peer group advances the count, after every lane has read it
      if (valid && before == 0) wcnt[wave][e] = cnt + __popcll(peers);
    }
  }
  __syncthreads();
  // per expert: start rank of each wave (exclusive scan over waves), total
  int total = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      const int v = wcnt[w][tid];
      wcnt[w][tid] = total;
      total += v;
    }
  }
  // exclusive scan of the kept totals min(total, cap) over experts (4 waves)
  const int v = tid < E ? min(total, cap) : 0;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (tid < E) {
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    off_s[tid] = wbase + incl - v;
    offsets[tid] = wbase + incl - v;
  }
  if (tid == 0) {
    int all = 0;
    for (int w = 0; w < kSmallWaves; ++w) all += wsum[w];
    offsets[E] = all;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSmallChunks; ++j) {
    if (pr[j] == -2) inv_pos[(c0 + j) * kWave + lane] = -1;   // dropped
    if (pr[j] >= 0) {
      const int e = pr[j] & 255;
      const int i = (c0 + j) * kWave + lane;
      const int r_e = wcnt[wave][e] + (pr[j] >> 8);
      if (r_e < cap) {
        const int pos = off_s[e] + r_e;
        sorted_token[pos] = i / k;
        inv_pos[i] = pos;
      } else {
        inv_pos[i] = -1;
      }
    }
  }
}

}  // namespace

size_t permute_ws_bytes(int R, int E) {
  const size_t nchunks = (R + CH - 1) / CH;
  return 2 * align_up(nchunks * E * sizeof(int32_t));
}

hipError_t launch_permute(const void* x, const int32_t* ids, int T, int H, int E, int k,
                          int capacity, size_t elem_bytes, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_pos, void* xp, void* ws,
                          hipStream_t s) {
  const int R = T * k;
  const int cap = capacity > 0 ? capacity : R;   // R: nothing is dropped
  const int nchunks = (R + CH - 1) / CH;
  int32_t* counts = (int32_t*)ws;
  int32_t* base = (int32_t*)((char*)ws + align_up((size_t)nchunks * E * sizeof(int32_t)));
  if (R > 0 && E <= kSmallE && R <= kSmallR) {
    // (one workgroup stops paying beyond 16 chunks per wave: each chunk's
    // rank waits on the previous chunk's count update in LDS)
    hipLaunchKernelGGL(perm_small<kSmallR / (kSmallWaves * kWave)>, dim3(1), dim3(1024), 0, s,
                       ids, R, E, k, cap, offsets, sorted_token, inv_pos);
  } else {
    if (nchunks > 0)
      hipLaunchKernelGGL(perm_count, dim3(nchunks), dim3(256), E * sizeof(int), s, ids, R, E,
                         counts);
    // runs even for R == 0 so that the offsets are written (all zero)
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, counts, nchunks, E, cap, base,
                       offsets);
    if (nchunks == 0) return hipGetLastError();
    hipLaunchKernelGGL(perm_place, dim3(nchunks), dim3(256), 5 * E * sizeof(int), s, ids, R, E,
                       k, cap, base, offsets, sorted_token, inv_pos);
  }
  if (xp == nullptr) return hipGetLastError();
  const int row_chunks = (int)((size_t)H * elem_bytes / 16);
  const int blocks = std::min(8192, (R + 3) / 4);
  hipLaunchKernelGGL(perm_gather, dim3(blocks), dim3(256), 0, s, (const u32x4*)x, sorted_token,
                     offsets, E, R, T, (u32x4*)xp, row_chunks);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* sorted_token, const int32_t* offsets,
                              int E, int R, int T, int H, size_t elem_bytes, void* xp,
                              hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int row_chunks = (int)((size_t)H * elem_bytes / 16);
  const int blocks = std::min(8192, (R + 3) / 4);
  hipLaunchKernelGGL(perm_gather, dim3(blocks), dim3(256), 0, s, (const u32x4*)x, sorted_token,
                     offsets, E, R, T, (u32x4*)xp, row_chunks);
  return hipGetLastError();
}

}  // namespace moe
