// Route permutation and expert offsets.
//
// "Hunyuan Image 3.0 hybrid parallelism", section 6.1: the flattened expert
// ids are sorted by expert (permuted_to_expanded), the per-expert offsets
// come from a bincount and a cumulative sum, and finalize reads the expert
// outputs back through the inverse permutation.  Here the sort is a stable
// counting sort (each expert's routes keep route order r = t*k + j), so perm
// and inv are unique.
//
// The scatter of R routes to expert-sorted positions is spread over at most
// 256 workgroups, each owning a contiguous route chunk [cs, ce).  A workgroup
// needs the expert counts of all routes (for the offsets) and of the routes
// before its chunk (for its write bases):
//   * moe_permute (ids only): every workgroup counts all ids itself (they are
//     a few hundred KB and sit in L2), with LDS atomics on per-wave counters;
//   * the one-call layer: the router already wrote one row of expert counts
//     per 16-token block, and every workgroup sums those rows instead.
// No grid-wide synchronisation is needed either way.  One wave then walks the
// chunk 64 routes at a time, ranks every route among the earlier lanes with
// the same expert (six ballots over the id bits) and scatters.  Positions use
// no atomics, so perm and inv are deterministic; every workgroup computes the
// same counts and offsets and workgroup 0 writes them.
#include "moe_common.h"

#include <algorithm>

namespace moe {
namespace {

constexpr int kWaves = 16;
constexpr int kPer = 16;               // ids per lane per tile
constexpr int kTile = kWave * kPer;    // routes per wave per tile
constexpr int kMinChunk = 512;         // routes scattered per workgroup, at least
constexpr int kMaxBlocks = 256;        // bounds the redundant counting to 256 * R ids

// Wave 0 of the workgroup: t = this lane's expert total, bf = its count
// before the chunk.  Writes the write bases to base[] and, in workgroup 0,
// counts and offsets; then scatters routes [cs, ce) stably by expert.
__device__ __forceinline__ void scan_and_scatter(const int32_t* __restrict__ ids, int E, int cs,
                                                 int ce, int t, int bf, int* base,
                                                 int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm,
                                                 int32_t* __restrict__ inv) {
  const int lane = threadIdx.x & 63;
  if (lane >= E) t = 0;
  int incl = t;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  const int excl = incl - t;
  base[lane] = excl + bf;
  if (blockIdx.x == 0) {
    if (lane < E) {
      counts[lane] = t;
      offsets[lane] = excl;
    }
    if (lane == E - 1) offsets[E] = incl;
  }
  __builtin_amdgcn_wave_barrier();

  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int t0 = cs; t0 < ce; t0 += kTile) {
    // all loads of a tile in flight before the serial ranking: the index is
    // clamped instead of branched on (a branch around each load makes the
    // compiler wait for it), and lanes past ce are masked below
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = ids[min(t0 + kWave * i + lane, ce - 1)];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (t0 + kWave * i >= ce) break;
      const int r = t0 + kWave * i + lane;
      const bool valid = r < ce;
      const int e = min(max(v[i], 0), E - 1);  // clamp keeps every write in bounds
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 6; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(valid && bit);
        peers &= bit ? m : ~m;
      }
      int rank = 0;
      if (valid) {
        rank = __popcll(peers & lt_mask);
        const int pos = base[e] + rank;
        perm[pos] = r;
        inv[r] = pos;
      }
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == 0) base[e] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__global__ __launch_bounds__(kWaves * kWave) void permute_kernel(
    const int32_t* __restrict__ ids, int R, int E, int chunk, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int tot[kWaves][kMaxExperts];     // per-wave counts of all routes
  __shared__ int before[kWaves][kMaxExperts];  // ... of the routes before this chunk
  __shared__ int base[kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cs = min(R, (int)blockIdx.x * chunk), ce = min(R, cs + chunk);

  // wave w counts the routes [w*C, (w+1)*C); ids come from the router and are
  // clamped to [0, E) so every write stays in bounds
  const int per = (R + kWaves - 1) / kWaves;
  const int C = (per + 63) & ~63;
  const int start = min(R, wave * C), end = min(R, start + C);
  tot[wave][lane] = 0;
  before[wave][lane] = 0;
  __syncthreads();
  for (int t0 = start; t0 < end; t0 += kTile) {
    int v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = ids[min(t0 + kWave * i + lane, end - 1)];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = t0 + kWave * i + lane;
      if (r < end) {
        const int e = min(max(v[i], 0), E - 1);
        atomicAdd(&tot[wave][e], 1);
        if (r < cs) atomicAdd(&before[wave][e], 1);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    int t = 0, bf = 0;
    for (int w = 0; w < kWaves; ++w) {
      t += tot[w][lane];
      bf += before[w][lane];
    }
    scan_and_scatter(ids, E, cs, ce, t, bf, base, counts, offsets, perm, inv);
  }
}

// The one-call layer: hist[b][e] = routes of router block b (tokens
// [16b, 16b+16)) that went to expert e.  Workgroup c scatters the routes of
// router blocks [c*G, (c+1)*G).
__global__ __launch_bounds__(kWaves * kWave) void permute_hist_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ hist, int nb, int G,
    int routes_per_block, int R, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int tot[kWaves][kMaxExperts];
  __shared__ int before[kWaves][kMaxExperts];
  __shared__ int base[kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b0 = blockIdx.x * G;
  int t = 0, bf = 0;
  // rows wave, wave + 16, ...: kPer row loads in flight at a time
  for (int bb = wave; bb < nb; bb += kWaves * kPer) {
    int c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = hist[(size_t)min(bb + kWaves * i, nb - 1) * kMaxExperts + lane];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = bb + kWaves * i;
      if (b < nb) t += c[i];
      if (b < min(b0, nb)) bf += c[i];
    }
  }
  tot[wave][lane] = t;
  before[wave][lane] = bf;
  __syncthreads();
  if (wave == 0) {
    t = 0;
    bf = 0;
    for (int w = 0; w < kWaves; ++w) {
      t += tot[w][lane];
      bf += before[w][lane];
    }
    const long long cs = (long long)b0 * routes_per_block;
    const int ce = (int)std::min<long long>(R, cs + (long long)G * routes_per_block);
    scan_and_scatter(ids, E, (int)std::min<long long>(cs, R), ce, t, bf, base, counts, offsets,
                     perm, inv);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x,
                                                     const int32_t* __restrict__ perm, int H,
                                                     int k, T* __restrict__ xp) {
  const int p = blockIdx.x;
  const int t = perm[p] / k;
  constexpr int V = 16 / sizeof(T);
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  uint4* dst = reinterpret_cast<uint4*>(xp + (size_t)p * H);
  for (int c = threadIdx.x; c < H / V; c += blockDim.x) dst[c] = src[c];
}

}  // namespace

// An empty batch: every count and offset is zero (offsets[E] = R = 0).  A
// kernel rather than a memset, so a captured graph holds only kernels.
__global__ __launch_bounds__(kWave * 2) void zero_counts_kernel(int E, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets) {
  const int e = threadIdx.x;
  if (e < E) counts[e] = 0;
  if (e <= E) offsets[e] = 0;
}

hipError_t launch_permute(const Shape& s, const int32_t* ids, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t st) {
  const int R = (int)s.R();
  if (R == 0) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kWave * 2), 0, st, s.E, counts, offsets);
    return hipGetLastError();
  }
  const long long even = ((long long)R + kMaxBlocks - 1) / kMaxBlocks;
  const int chunk = (int)std::max<long long>(kMinChunk, (even + 63) / 64 * 64);
  const unsigned blocks = (unsigned)(((long long)R + chunk - 1) / chunk);
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(kWaves * kWave), 0, st, ids, R, s.E,
                     chunk, counts, offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_permute_hist(const Shape& s, const int32_t* ids, const int32_t* hist,
                               int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                               hipStream_t st) {
  const int R = (int)s.R();
  const int nb = (s.T + kRouteTokTile - 1) / kRouteTokTile;
  const int rpb = kRouteTokTile * s.k;
  const int G = std::max((kMinChunk + rpb - 1) / rpb, (nb + kMaxBlocks - 1) / kMaxBlocks);
  const unsigned blocks = (unsigned)((nb + G - 1) / G);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(blocks), dim3(kWaves * kWave), 0, st, ids, hist,
                     nb, G, rpb, R, s.E, counts, offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather(const Shape& s, const void* x, const int32_t* perm, void* xp,
                         hipStream_t st) {
  const unsigned R = (unsigned)s.R();
  if (s.bf16)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(R), dim3(256), 0, st, (const uint16_t*)x,
                       perm, s.H, s.k, (uint16_t*)xp);
  else
    hipLaunchKernelGGL(gather_kernel<float>, dim3(R), dim3(256), 0, st, (const float*)x, perm,
                       s.H, s.k, (float*)xp);
  return hipGetLastError();
}

}  // namespace moe
