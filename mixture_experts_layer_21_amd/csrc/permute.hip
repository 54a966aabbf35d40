// Dispatch kernels (fused MoE article, GatherTokensByExpert): group the
// R = T*k (token, slot) pairs by expert, keeping the article's order inside
// each expert (ascending token, then slot).  The article scans all pairs once
// per expert (O(E*R)); here it is a counting sort, O(R).  With a capacity
// (the article's [num_experts, expert_capacity] blocks; CANN MoE article,
// section 4.3) each expert keeps only its first `cap` pairs in that order.
//
//   (larger layers, three launches:)
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
//   perm_onepass for R <= 65536 pairs the first three in one launch: each
//                workgroup counts all pairs (totals, and those before its own
//                1024) in LDS, so it knows the offsets and its range's base
//                ranks without reading another workgroup's results, then
//                ranks and places its 1024 pairs (the same stable order)
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

// Dispatch in one launch for R <= kOnePassR (any E <= 1024): workgroup g of
// 1024 threads owns the pairs [1024 g, 1024 g + 1024) (one per thread).  It
// first counts, in LDS, every valid pair of the whole layer by expert, and
// separately those before its own range: the totals give every expert's
// offset (each workgroup computes the same exclusive scan of min(total,
// cap); workgroup 0 writes them), the "before" counts give the rank at
// which each expert's pairs of this range start.  Then each pair's rank
// inside the range is found from the ballot peers inside the wave
// plus the counts of the earlier waves, and the pair is placed.  No
// workgroup reads another's results, so nothing crosses workgroups and one
// launch suffices; every workgroup reads all R ids (L2-resident), which is
// why this form stops at kOnePassR pairs.
constexpr int kOnePassR = 65536;
constexpr int kOnePassWaves = 16;

__global__ __launch_bounds__(1024) void perm_onepass(const int32_t* __restrict__ ids, int R,
                                                     int E, int k, int cap,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_token,
                                                     int32_t* __restrict__ inv_pos) {
  extern __shared__ int sm[];
  int* total = sm;                           // [E]: valid pairs of each expert
  int* before = sm + E;                      // [E]: ... before this workgroup's range
  int* wcnt = sm + 2 * E;                    // [16][E]: this range's pairs per wave
  int* off_s = sm + (2 + kOnePassWaves) * E; // [E]: kept-row offset of each expert
  __shared__ int wsum[kOnePassWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int start = blockIdx.x * 1024;
  for (int t = tid; t < (2 + kOnePassWaves) * E; t += 1024) sm[t] = 0;
  __syncthreads();
  // counts over all pairs (8 ids per thread loaded before they are counted),
  // one LDS atomic per pair: the pairs before this range into `before`, the
  // others into `total`, which then takes `before` in
  for (int i0 = tid; i0 < R; i0 += 8 * 1024) {
    int e8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 1024;
      e8[u] = i < R ? ids[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 1024;
      if ((unsigned)e8[u] < (unsigned)E) atomicAdd(i < start ? &before[e8[u]] : &total[e8[u]], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) total[e] += before[e];
  // this range: each pair's expert and its rank among the wave's peers
  const int i = start + tid;
  const int my_e = i < R ? ids[i] : -1;
  const bool valid = i < R && (unsigned)my_e < (unsigned)E;
  const uint64_t peers = wave_match(my_e, valid, id_bits(E));
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int in_wave = __popcll(peers & lt_mask);
  if (valid && in_wave == 0) wcnt[wave * E + my_e] = __popcll(peers);
  __syncthreads();
  // thread e (E <= 1024): the start rank of each wave among expert e's pairs
  // of this range (exclusive scan of the wave counts), and expert e's
  // kept-row offset (exclusive scan of min(total, cap) over the experts)
  const int v = tid < E ? min(total[tid], cap) : 0;
  if (tid < E) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kOnePassWaves; ++w) {
      const int c = wcnt[w * E + tid];
      wcnt[w * E + tid] = run;
      run += c;
    }
  }
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  if (tid < E) {
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wsum[w];
    off_s[tid] = wbase + incl - v;
    if (blockIdx.x == 0) offsets[tid] = wbase + incl - v;
  }
  if (blockIdx.x == 0 && tid == 0) {
    int all = 0;
    for (int w = 0; w < kOnePassWaves; ++w) all += wsum[w];
    offsets[E] = all;
  }
  __syncthreads();
  if (i >= R) return;
  if (!valid) {
    inv_pos[i] = -1;   // an id outside [0, E): dropped
    return;
  }
  const int r_e = before[my_e] + wcnt[wave * E + my_e] + in_wave;
  if (r_e < cap) {
    const int pos = off_s[my_e] + r_e;
    sorted_token[pos] = i / k;
    inv_pos[i] = pos;
  } else {
    inv_pos[i] = -1;
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
  if (R > 0 && R <= kOnePassR) {
    const size_t lds = (size_t)(3 + kOnePassWaves) * E * sizeof(int);
    hipLaunchKernelGGL(perm_onepass, dim3((unsigned)((R + 1023) / 1024)), dim3(1024), lds, s,
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
